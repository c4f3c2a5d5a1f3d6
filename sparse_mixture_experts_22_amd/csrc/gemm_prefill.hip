// Grouped expert GEMMs for large token counts (prefill), bf16 MFMA on gfx950.
//
// The experts are the SwiGLU feed-forward blocks of the layer equation (card
// 2.1 of the "Mixtral of Experts" study deck): each has two d x f expansion
// matrices and one f x d compression matrix (Part 4 of "Mixture of Experts:
// Why Mixtral Only Wakes Up Two Specialists" counts three 4096 x 14336
// matrices per expert).  Only experts that some token selected get work, and
// each runs once on the contiguous group of its rows produced by the dispatch.
//
//   up   (MODE 1): h[p] = SiLU(x[perm_token[p]] W1_e) * (x[perm_token[p]] W3_e)
//                  -> bf16 (round-to-nearest-even), W1 and W3 share the A tile
//   down (MODE 2): o[p] = h[p] W2_e -> fp32
//
// Tiling: a 256-thread workgroup (4 waves, one per SIMD) computes a 256-row x
// 256-column fp32 accumulator tile (for MODE 1: 128 W1 columns + the same 128
// W3 columns) with v_mfma_f32_32x32x16_bf16; each wave owns 128 x 128 (16 MFMA
// tiles, 256 accumulator registers).  K advances in steps of 32 through a ring
// of 4 LDS stages (32 KiB each): global loads for step k+3 are in flight while
// step k is multiplied.
//
// Data movement is HBM/L2 -> LDS directly (global_load_lds, 16 bytes per lane,
// lane l writing bytes 16*l.. of a 1 KiB block), with no register staging and
// no LDS store instructions.  Which global 16-byte chunk a lane fetches is
// permuted so the LDS image is XOR-swizzled:
//   A (activations, [row][k], 64-byte rows): chunk c of row r sits at
//     position c ^ ((r >> 1) & 3), so the MFMA A reads (one row per lane, 16 B)
//     are bank-conflict free;
//   B (weights, kept in their natural [k][n] layout, 512-byte rows): chunk c of
//     row k sits at position c ^ (2 * (k & 3)).
// The weights are n-contiguous while MFMA wants 8 consecutive k per lane; the
// B fragments are read with ds_read_b64_tr_b16, which transposes 16-bit data
// across each group of 16 lanes: when lane q + 4j of a group points at
// B[k0 + j][n0 + 4q .. 4q + 3], lane i of the group receives B[k0 .. k0+3][n0 + i].
// Two such reads give the 8 k values of one B fragment.
//
// Tile order: the hardware hands workgroup i to XCD (i mod 8).  The grid is
// remapped so each XCD walks a contiguous range of the tile list, and the list
// is ordered expert-major, then groups of 4 column tiles, then row tiles: the
// ~32 tiles an XCD runs at once share 8 row blocks and 4 column blocks of one
// expert, so their A and B k-slices are served from that XCD's L2.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = kPrefillBM;  // 256 rows
constexpr int BN = 256;         // LDS B-tile columns
constexpr int BK = 32;
constexpr int NGROUP = 4;       // column tiles per scheduling group

struct Tile {
  int e, nt, row0, rows;
};

// Maps this workgroup to a tile, or returns false if it has none.  All threads
// compute the same answer from offsets[0..n] (uniform loads).
__device__ bool decode_tile(const int* __restrict__ offsets, int n, int NT, Tile& tc) {
  int total = 0;
  for (int e = 0; e < n; ++e) {
    const int c = offsets[e + 1] - offsets[e];
    total += ((c + BM - 1) / BM) * NT;
  }
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int i = blockIdx.x >> 3;
  if (i >= per) return false;
  int L = xcd * per + i;
  if (L >= total) return false;
  for (int e = 0; e < n; ++e) {
    const int c = offsets[e + 1] - offsets[e];
    const int mt = (c + BM - 1) / BM;
    const int cnt = mt * NT;
    if (L < cnt) {
      const int ng = NT / NGROUP;
      const int gsz = mt * NGROUP;
      const int grp = L / gsz;
      int m, nt;
      if (grp < ng) {
        const int rem = L - grp * gsz;
        m = rem / NGROUP;
        nt = grp * NGROUP + rem % NGROUP;
      } else {
        const int rem = L - ng * gsz;
        const int gt = NT - ng * NGROUP;
        m = rem / gt;
        nt = ng * NGROUP + rem % gt;
      }
      tc.e = e;
      tc.nt = nt;
      tc.row0 = offsets[e] + m * BM;
      const int left = offsets[e + 1] - tc.row0;
      tc.rows = left < BM ? left : BM;
      return true;
    }
    L -= cnt;
  }
  return false;
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int STAGES = 4;
constexpr int A_STAGE = BM * BK * 2;  // 16 KiB
constexpr int B_STAGE = BK * BN * 2;  // 16 KiB

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Written as inline asm so the compiler does not treat the LDS write as an
// unknown store and wait for every load in flight before each LDS read; the
// kernel tracks completion itself with s_waitcnt vmcnt.  The instruction has
// no destination register, so nothing can be overwritten while it is in flight.
__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ bf16x8_t read_b_frag(const char* p0, const char* p1) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const i16x4_t both[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8_t*>(both);
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int* __restrict__ offsets, int n, int Kdim, int N, int a_rows, int TK,
    uint16_t* __restrict__ hout, float* __restrict__ oout) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * (A_STAGE + B_STAGE)];

  constexpr int NTW = (MODE == 1) ? 128 : 256;  // output columns per tile
  const int NT = (N + NTW - 1) / NTW;
  Tile tc;
  if (!decode_tile(offsets, n, NT, tc)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- global -> LDS load assignment: wave w issues 4 A blocks and 4 B
  // blocks (64 chunks of 16 B each) per stage.
  const uint16_t* a_ptr[4];
  const uint16_t* b_ptr[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // A block: 16 rows x 4 chunks; this lane fills position (r, l % 4)
    const int r = (wave * 4 + b) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 1) & 3);
    const int rr = r < tc.rows ? r : tc.rows - 1;  // padded rows: computed, never stored
    const int p = min(max(tc.row0 + rr, 0), TK - 1);
    const int row = (MODE == 1) ? min(max(perm_token[p], 0), a_rows - 1) : p;
    a_ptr[b] = A + (int64_t)row * Kdim + c * 8;
    // B block: 2 rows x 32 chunks; this lane fills position (k, l % 32)
    const int k = (wave * 4 + b) * 2 + (lane >> 5);
    const int cb = (lane & 31) ^ (2 * (k & 3));
    int col;
    const uint16_t* mat;
    if (MODE == 1) {
      col = tc.nt * 128 + (cb & 15) * 8;
      mat = (cb >> 4) ? B3 : B1;
    } else {
      col = tc.nt * 256 + cb * 8;
      mat = B1;
    }
    if (col >= N) col = 0;  // N tail: any valid column; its outputs are never stored
    b_ptr[b] = mat + (int64_t)tc.e * Kdim * N + (int64_t)k * N + col;
  }
  char* a_lds = smem;
  char* b_lds = smem + STAGES * A_STAGE;
  const uint32_t a_lds_u = (uint32_t)(uintptr_t)(lds_void*)a_lds;
  const uint32_t b_lds_u = (uint32_t)(uintptr_t)(lds_void*)b_lds;
  // Loads k-step `kt_data` into ring slot `kt_slot & (STAGES - 1)`.
  auto issue_stage = [&](int kt_slot, int kt_data) {
    const int slot = kt_slot & (STAGES - 1);
    const int kt = kt_data;
    const uint32_t as = a_lds_u + slot * A_STAGE + wave * 4096;
    const uint32_t bs = b_lds_u + slot * B_STAGE + wave * 4096;
    const int64_t koff_a = (int64_t)kt * BK;
    const int64_t koff_b = (int64_t)kt * BK * N;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      load_lds16(a_ptr[b] + koff_a, as + b * 1024);
      load_lds16(b_ptr[b] + koff_b, bs + b * 1024);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- fragment read addresses (byte offsets inside a stage)
  const int m = lane & 31;
  const int kg = lane >> 5;
  int a_off[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + m;
      a_off[ks][i] = r * 64 + (((ks * 2 + kg) ^ ((m >> 1) & 3)) * 16);
    }
  const int g16 = lane >> 4;      // 16-lane group
  const int h16 = g16 & 1;        // column half of a 32-column MFMA tile
  const int kg16 = g16 >> 1;      // k half of the MFMA step
  const int bj = (lane & 15) >> 2;
  const int qq = lane & 3;
  int b_off[2][4][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int nb = (MODE == 1) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
        const int k = ks * 16 + kg16 * 8 + 4 * t + bj;
        const int cc = (nb >> 3) + 2 * h16 + (qq >> 1);
        b_off[ks][j][t] = k * 512 + ((cc ^ (2 * bj)) * 16) + (qq & 1) * 8;
      }

  auto compute = [&](int slot) {
    const char* as = a_lds + slot * A_STAGE;
    const char* bs = b_lds + slot * B_STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(as + a_off[ks][i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = read_b_frag(bs + b_off[ks][j][0], bs + b_off[ks][j][1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- main loop.  Before step kt is consumed each wave waits until only
  // the 16 loads of steps kt+1, kt+2 remain outstanding, then a barrier makes
  // every wave's part of step kt visible.  The loads for step kt+3 reuse the
  // slot of step kt-1, which every wave finished before that barrier.  Steps
  // past the end reload the last k-slice into a slot nobody reads again, so
  // the count of outstanding loads is the same on every iteration.
  const int nk = Kdim / BK;
  issue_stage(0, 0);
  issue_stage(1, min(1, nk - 1));
  issue_stage(2, min(2, nk - 1));
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16), expcnt/lgkmcnt unconstrained
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_stage(kt + 3, min(kt + 3, nk - 1));
    compute(kt & (STAGES - 1));
  }
  // the last (redundant) loads must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  const int lrow = m;
  const int lk = kg;
  // 32x32 MFMA D layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int c = tc.nt * 128 + wn * 64 + jj * 32 + lrow;
        if (c >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          if (row < tc.rows && tc.row0 + row < TK) {
            const float a = acc[i][jj][r];
            const float b = acc[i][jj + 2][r];
            hout[(int64_t)(tc.row0 + row) * N + c] = f32_to_bf16_rne(silu_f32(a) * b);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = tc.nt * 256 + wn * 128 + j * 32 + lrow;
        if (c >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          if (row < tc.rows && tc.row0 + row < TK) oout[(int64_t)(tc.row0 + row) * N + c] = acc[i][j][r];
        }
      }
  }
}

// Upper bound of the tile count: sum_e ceil(c_e / BM) <= ceil(TK / BM) + n.
inline unsigned prefill_grid(int64_t TK, int n, int NT) {
  const int64_t ub = ((TK + BM - 1) / BM + n) * (int64_t)NT;
  return (unsigned)(((ub + 7) / 8) * 8);
}

}  // namespace

hipError_t launch_prefill_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W1,
                             const uint16_t* W3, const int* offsets, int64_t TK, int n, int d, int f,
                             uint16_t* h, hipStream_t s) {
  const int NT = (f + 127) / 128;
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(prefill_grid(TK, n, NT)), dim3(256), 0, s, x,
                     perm_token, W1, W3, offsets, n, d, f, (int)T, (int)TK, h, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const uint16_t* h, const uint16_t* W2, const int* offsets, int64_t TK,
                               int n, int f, int d, float* o, hipStream_t s) {
  const int NT = (d + 255) / 256;
  hipLaunchKernelGGL((grouped_gemm_kernel<2>), dim3(prefill_grid(TK, n, NT)), dim3(256), 0, s, h,
                     (const int*)nullptr, W2, (const uint16_t*)nullptr, offsets, n, f, d, (int)TK,
                     (int)TK, (uint16_t*)nullptr, o);
  return hipGetLastError();
}

}  // namespace moe
