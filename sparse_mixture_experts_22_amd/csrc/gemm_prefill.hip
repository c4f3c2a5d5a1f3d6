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
// tiles, 256 accumulator registers).  K advances in steps of 64 through two
// LDS stages (2 x 64 KiB), global loads of step k+1 overlap the MFMAs of step k.
//
// The weights are [K][N] row-major (N contiguous) but MFMA wants each lane to
// hold 8 consecutive K values of one column.  Each thread therefore loads an
// 8 (k) x 8 (n) bf16 block as eight 16-byte row segments, transposes it in
// registers with byte permutes, and writes eight 16-byte column segments to
// LDS stored [n][k].  A and B rows in LDS are 128 bytes; the 16-byte chunk
// index is XOR-swizzled with (row & 7) so that the MFMA fragment reads (one
// row per lane, same chunk) and the stores hit distinct banks.
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
constexpr int BK = 64;
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

// 8x8 transpose of bf16: in[r] = row r (8 columns), out[c] = column c (8 rows).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t r0 = (&in[2 * q].x)[p];
      const uint32_t r1 = (&in[2 * q + 1].x)[p];
      lo[q] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);  // (r0.lo, r1.lo)
      hi[q] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);  // (r0.hi, r1.hi)
    }
    out[2 * p] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    out[2 * p + 1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int* __restrict__ offsets, int n, int Kdim, int N, int a_rows, int TK,
    uint16_t* __restrict__ hout, float* __restrict__ oout) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

  constexpr int NTW = (MODE == 1) ? 128 : 256;  // output columns per tile
  const int NT = (N + NTW - 1) / NTW;
  Tile tc;
  if (!decode_tile(offsets, n, NT, tc)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // A: thread loads chunk a_c (16 B) of rows a_r0 + 32*i, i = 0..7
  const int a_c = tid & 7;
  const int a_r0 = tid >> 3;
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = a_r0 + 32 * i;
    const int rr = r < tc.rows ? r : tc.rows - 1;  // padded rows: computed, never stored
    const int p = min(max(tc.row0 + rr, 0), TK - 1);
    const int row = (MODE == 1) ? min(max(perm_token[p], 0), a_rows - 1) : p;
    a_src[i] = A + (int64_t)row * Kdim + a_c * 8;
  }
  // B: thread loads the 8x8 block (k rows b_kc*8.., columns of chunk b_nc)
  const int b_kc = tid & 7;
  const int b_nc = tid >> 3;
  const int64_t e_off = (int64_t)tc.e * Kdim * N;
  int col;
  const uint16_t* bbase;
  if (MODE == 1) {
    col = tc.nt * 128 + (b_nc & 15) * 8;
    bbase = (b_nc >> 4) ? B3 : B1;
  } else {
    col = tc.nt * 256 + b_nc * 8;
    bbase = B1;
  }
  const bool b_ok = col < N;
  const uint16_t* b_src = bbase + e_off + (int64_t)(b_kc * 8) * N + (b_ok ? col : 0);

  uint4 ra[8], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
    if (b_ok) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        rb[r] = *reinterpret_cast<const uint4*>(b_src + (int64_t)(k0 + r) * N);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) rb[r] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* as = As[buf];
    uint16_t* bs = Bs[buf];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = a_r0 + 32 * i;
      *reinterpret_cast<uint4*>(as + r * BK + ((a_c ^ (r & 7)) * 8)) = ra[i];
    }
    uint4 tcol[8];
    transpose8x8(rb, tcol);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int nrow = b_nc * 8 + c;
      *reinterpret_cast<uint4*>(bs + nrow * BK + ((b_kc ^ c) * 8)) = tcol[c];
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int lrow = lane & 31;
  const int lk = lane >> 5;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = (MODE == 1) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);

  auto compute = [&](int buf) {
    const uint16_t* as = As[buf];
    const uint16_t* bs = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = ((ks * 2 + lk) ^ (lane & 7)) * 8;
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(as + (wm * 128 + i * 32 + lrow) * BK + ch);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(bs + (brow[j] + lrow) * BK + ch);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = Kdim / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    compute(cur);
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

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
