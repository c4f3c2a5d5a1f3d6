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
// Tiling: a 512-thread workgroup (8 waves, two per SIMD) computes a 256-row
// x 256-column fp32 accumulator tile (for MODE 1: 128 W1 columns + the same
// 128 W3 columns) with v_mfma_f32_32x32x16_bf16; each wave owns 128 rows x 64
// columns (8 MFMA tiles, 128 accumulator registers).  Two waves per SIMD keep
// the matrix cores fed while the partner wave is stalled issuing its share of
// the global loads (a CU can only have a bounded number of L2 requests in
// flight, and a load that cannot be accepted blocks its wave).
//
// Data movement is HBM/L2 -> LDS directly (global_load_lds, 16 bytes per lane,
// lane l writing bytes 16*l.. of a 1 KiB block), with no register staging and
// no LDS store instructions.  Which global 16-byte chunk a lane fetches is
// permuted so the LDS image is XOR-swizzled for gfx950's 64 banks (256 bytes
// per cycle):
//   A (activations, [row][k]): stored in super-stages of 64 k, 128-byte rows
//     (one cache line per row and request); chunk c of row r sits at
//     c ^ ((r >> 1) & 7), so the 16 lanes of an MFMA A read served together
//     (16 rows, same logical chunk) hit 16 distinct 16-byte slots;
//   B (weights, kept in their natural [k][n] layout, stages of 32 k, 512-byte
//     rows): chunk c of row k sits at c ^ (4 * (k & 3)), so the 32 lanes of a
//     transpose read served together (4 rows x 2 column halves) hit distinct
//     32-byte slots.
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
#include <type_traits>

#include "moe_internal.h"
#include "tile_sched.h"

namespace moe {

namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const void gbl_void;

// LDS rings.  The activation operand A moves in "super-stages" of 64 k
// (256 rows x 128 bytes = 32 KiB): a CU keeps a bounded number of L2 requests
// in flight, and 128-byte rows are one full cache line per request where
// 64-byte rows (32 k) would be half a line.  The weight operand
// B moves in stages of 32 k (32 rows x 512 bytes = 16 KiB, four full lines per
// row).  2*SA + SB = 10 fills the CU's 160 KiB.  Waves 0-3 load only B, waves
// 4-7 only A: a wave's vmcnt retires in issue order, so giving each operand
// its own waves lets each stream run as far ahead as its own ring allows.
#ifndef MOE_RING_A
#define MOE_RING_A 3
#endif
#ifndef MOE_RING_B
#define MOE_RING_B 4
#endif
constexpr int SA = MOE_RING_A;  // A super-stages (64 k each)
constexpr int SB = MOE_RING_B;  // B stages (32 k each)
static_assert(SA >= 2 && SB >= 2 && 2 * SA + SB <= 10, "LDS budget is 160 KiB");
constexpr int A_LOADS = 8;  // 1 KiB loads per A-loader wave per super-stage
constexpr int B_LOADS = 4;  // 1 KiB loads per B-loader wave per stage
// the main loop spreads a step's refill over the 4 row blocks of a burst:
// one B load, or two A loads, per block
static_assert(B_LOADS == 4 && A_LOADS == 8, "refill spread assumes 4 B and 8 A loads per wave");
// Publishing k-step kt+1: the wave's own loads of the stage holding it must
// have landed while the later stages may stay in flight, and its LDS reads of
// step kt must have returned (the slot of step kt is refilled after the barrier).
constexpr int WAIT_AHEAD_B = waitcnt_imm(B_LOADS * (SB - 2), 0);
constexpr int WAIT_AHEAD_A = waitcnt_imm(A_LOADS * (SA - 2), 0);  // kt+1 opens a super-stage
constexpr int WAIT_LDS_ONLY = waitcnt_imm(63, 0);                 // kt+1 in the same super-stage
// before the loop every stage is in flight and the first one must have landed
constexpr int WAIT_FIRST_B = waitcnt_imm(B_LOADS * (SB - 1), 15);
constexpr int WAIT_FIRST_A = waitcnt_imm(A_LOADS * (SA - 1), 15);
static_assert(B_LOADS * (SB - 1) < 64 && A_LOADS * (SA - 1) < 64, "vmcnt is a 6-bit counter");

constexpr int A_SUPER = BM * 64 * 2;  // 32 KiB
constexpr int B_STAGE = BK * BN * 2;  // 16 KiB


// A B fragment is two transposing LDS reads (k 0..3 and 4..7 of the lane's column).
__device__ __forceinline__ i16x4_t read_b_half(const char* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ bf16x8_t join_b_halves(i16x4_t lo, i16x4_t hi) {
  const i16x4_t both[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8_t*>(both);
}
__device__ __forceinline__ bf16x8_t read_b_frag(const char* p0, const char* p1) {
  return join_b_halves(read_b_half(p0), read_b_half(p1));
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int* __restrict__ offsets, int n, int Kdim, int N, int a_rows, int TK, int cus,
    uint16_t* __restrict__ hout, float* __restrict__ oout, float* __restrict__ tail_ws) {
  __shared__ __attribute__((aligned(1024))) char smem[SA * A_SUPER + SB * B_STAGE];

  constexpr int NTW = (MODE == 1) ? 128 : 256;  // output columns per tile
  const int NT = (N + NTW - 1) / NTW;
  Tile tc;
  // only the down projection (plain fp32 output) splits leftover tiles over k
  if (!decode_tile(offsets, n, NT, Kdim / BK, cus, MODE == 2 && tail_ws != nullptr, 2, tc)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;  // 128-row half of the tile
  const int wn = wave & 3;  // 64-column quarter of the tile

  // ---- global -> LDS load assignment.  Waves 0-3 (B loaders) each fill 4
  // of the 16 1-KiB blocks of a B stage (2 rows x 32 chunks each); waves 4-7
  // (A loaders) each fill 8 of the 32 blocks of an A super-stage (8 rows x 8
  // chunks each: every row is one full 128-byte line).
  const bool b_loader = wave < 4;
  const int lw = wave & 3;  // index among the loaders of the operand
  const uint16_t* ld_ptr[A_LOADS];
  if (!b_loader) {
#pragma unroll
    for (int b = 0; b < A_LOADS; ++b) {
      const int r = (lw * A_LOADS + b) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int rr = r < tc.rows ? r : tc.rows - 1;  // padded rows: computed, never stored
      const int p = min(max(tc.row0 + rr, 0), TK - 1);
      const int row = (MODE == 1) ? min(max(perm_token[p], 0), a_rows - 1) : p;
      ld_ptr[b] = A + (int64_t)row * Kdim + c * 8;
    }
  } else {
#pragma unroll
    for (int b = 0; b < B_LOADS; ++b) {
      const int k = (lw * B_LOADS + b) * 2 + (lane >> 5);
      const int cb = (lane & 31) ^ (4 * (k & 3));
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
      ld_ptr[b] = mat + (int64_t)tc.e * Kdim * N + (int64_t)k * N + col;
    }
  }
  char* a_lds = smem;
  char* b_lds = smem + SA * A_SUPER;
  const uint32_t a_ld_base = (uint32_t)(uintptr_t)(lds_void*)a_lds + lw * (A_LOADS * 1024);
  const uint32_t b_ld_base = (uint32_t)(uintptr_t)(lds_void*)b_lds + lw * (B_LOADS * 1024);
  // A loaders: super-stage `s_data` of this workgroup's k range into slot s_slot % SA.
  auto issue_a = [&](int s_slot, int s_data) {
    const uint32_t dst = a_ld_base + (s_slot % SA) * A_SUPER;
    const int64_t koff = (int64_t)(tc.k0 / 2 + s_data) * 64;
#pragma unroll
    for (int b = 0; b < A_LOADS; ++b) load_lds16(ld_ptr[b] + koff, dst + b * 1024);
  };
  // B loaders: k-step `kt_data` of this workgroup's k range into slot kt_slot % SB.
  auto issue_b = [&](int kt_slot, int kt_data) {
    const uint32_t dst = b_ld_base + (kt_slot % SB) * B_STAGE;
    const int64_t koff = (int64_t)(tc.k0 + kt_data) * BK * N;
#pragma unroll
    for (int b = 0; b < B_LOADS; ++b) load_lds16(ld_ptr[b] + koff, dst + b * 1024);
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- fragment read addresses (byte offsets inside a super-stage / stage).
  // A: 128-byte rows; 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7), so
  // the 16 lanes of a 16-byte read served together (16 rows, same chunk) hit
  // 16 distinct 16-byte slots of the 64 banks.  Step kt uses chunks
  // 4*(kt & 1) .. +3 of its super-stage; row block i adds i * 4 KiB.
  const int m = lane & 31;
  const int kg = lane >> 5;
  int a_off[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = wm * 128 + m;
      a_off[par][ks] = r * 128 + (((par * 4 + ks * 2 + kg) ^ ((m >> 1) & 7)) * 16);
    }
  const int g16 = lane >> 4;      // 16-lane group
  const int h16 = g16 & 1;        // column half of a 32-column MFMA tile
  const int kg16 = g16 >> 1;      // k half of the MFMA step
  const int bj = (lane & 15) >> 2;
  const int qq = lane & 3;
  int b_off[2][2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // MODE 1: fragment 0 = W1 columns, fragment 1 = the same W3 columns
        const int nb = (MODE == 1) ? (j * 128 + wn * 32) : (wn * 64 + j * 32);
        const int k = ks * 16 + kg16 * 8 + 4 * t + bj;
        const int cc = (nb >> 3) + 2 * h16 + (qq >> 1);
        b_off[ks][j][t] = k * 512 + ((cc ^ (4 * bj)) * 16) + (qq & 1) * 8;
      }

  // fragments of sub-step ks (k 16*ks .. +15) of k-step kt, whose parity is `par`
  auto read_frags = [&](int kt, int par, int ks, bf16x8_t (&a)[4], bf16x8_t (&b)[2]) {
    const char* as = a_lds + ((kt >> 1) % SA) * A_SUPER + a_off[par][ks];
    const char* bs = b_lds + (kt % SB) * B_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(as + i * 4096);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = read_b_frag(bs + b_off[ks][j][0], bs + b_off[ks][j][1]);
  };
  auto mfma_step = [&](const bf16x8_t (&a)[4], const bf16x8_t (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Scheduling pattern of a half step: the 8 fragment reads (4 A + 4
  // transposed B) each followed by one of the 8 MFMAs.
  auto interleave = [] {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
  };

  // ---- main loop.  A k-step has two MFMA sub-steps (k = 0..15, 16..31).
  // The barrier that publishes step kt+1 sits between them: before it, each
  // wave has its sub-step-1 fragments of step kt in registers (lgkmcnt(0))
  // and waits until its own loads holding step kt+1 have landed (vmcnt);
  // after it, the sub-step-0 fragments of step kt+1 are read during the
  // sub-step-1 MFMAs of step kt, and then the slots that only step kt used
  // are refilled (B: every step, with the step SB ahead; A: after odd steps,
  // when a whole super-stage has been consumed, with the super-stage SA
  // ahead).  Loads past the end reload the last k-slice into slots nobody
  // reads again, so the count of outstanding loads never changes.  The loop
  // runs over pairs of steps so the parity of kt is a compile-time constant.
  const int nk = tc.k1 - tc.k0;  // even: Kdim and the pieces are multiples of 64 k
  const int nks = nk / 2;
  if (b_loader) {
    for (int st = 0; st < SB; ++st) issue_b(st, min(st, nk - 1));
    __builtin_amdgcn_s_waitcnt(WAIT_FIRST_B);  // step 0 landed
  } else {
    for (int st = 0; st < SA; ++st) issue_a(st, min(st, nks - 1));
    __builtin_amdgcn_s_waitcnt(WAIT_FIRST_A);  // super-stage 0 landed
  }
  fence();
  __builtin_amdgcn_s_barrier();
  fence();
  bf16x8_t fa0[4], fb0[2], fa1[4], fb1[2];
  read_frags(0, 0, 0, fa0, fb0);
  auto step = [&](int kt, auto par_c) {
    constexpr int par = decltype(par_c)::value;
    read_frags(kt, par, 1, fa1, fb1);
    mfma_step(fa0, fb0);
    interleave();
    if (b_loader)
      __builtin_amdgcn_s_waitcnt(WAIT_AHEAD_B);
    else
      __builtin_amdgcn_s_waitcnt(par ? WAIT_AHEAD_A : WAIT_LDS_ONLY);
    fence();
    __builtin_amdgcn_s_barrier();
    fence();
    // Sub-step 1 of step kt, one row block (two MFMAs) at a time; after each
    // block come two of step kt+1's sub-step-0 fragment reads and a quarter
    // of this step's refill loads (one B load, or two A loads after odd
    // steps).  A load the CU cannot accept yet then stalls this wave with
    // MFMAs still queued behind it, rather than with the whole refill batch
    // ahead of them.
    const char* as = a_lds + (((kt + 1) >> 1) % SA) * A_SUPER + a_off[par ^ 1][0];
    const char* bs = b_lds + ((kt + 1) % SB) * B_STAGE;
    const uint32_t b_dst = b_ld_base + ((kt + SB) % SB) * B_STAGE;
    const int64_t b_koff = (int64_t)(tc.k0 + min(kt + SB, nk - 1)) * BK * N;
    const uint32_t a_dst = a_ld_base + (((kt >> 1) + SA) % SA) * A_SUPER;
    const int64_t a_koff = (int64_t)(tc.k0 / 2 + min((kt >> 1) + SA, nks - 1)) * 64;
    i16x4_t bhalf[2][2];  // transposed halves of fb0[j]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[i], fb1[j], acc[i][j], 0, 0, 0);
      fa0[i] = *reinterpret_cast<const bf16x8_t*>(as + i * 4096);
      bhalf[i >> 1][i & 1] = read_b_half(bs + b_off[0][i >> 1][i & 1]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // the other MFMA
      fence();
      if (b_loader) {
        load_lds16(ld_ptr[i] + b_koff, b_dst + i * 1024);
      } else if (par) {
        load_lds16(ld_ptr[2 * i] + a_koff, a_dst + (2 * i) * 1024);
        load_lds16(ld_ptr[2 * i + 1] + a_koff, a_dst + (2 * i + 1) * 1024);
      }
      fence();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) fb0[j] = join_b_halves(bhalf[j][0], bhalf[j][1]);
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }
  // the last (redundant) loads must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(WAITCNT_ALL);

  const int lrow = m;
  const int lk = kg;
  // 32x32 MFMA D layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  // Up projection: the h tile goes through LDS (the rings are idle now), so
  // that each lane stores 16 contiguous bytes of one row: whole lines, and 8
  // store instructions per wave instead of 64 two-byte ones.  Rows r and r + 4
  // of a 32x32 block (the two half-waves) would share LDS banks, so the
  // 16-byte chunk index is XOR-swizzled by bit 2 of the row.  (The same
  // staging for the down projection's fp32 tile, in two 128 KiB halves, was
  // slower: half the waves idle behind three barriers.)
  if (MODE == 1) {
    __syncthreads();  // every wave's ring loads have landed and its LDS reads are done
    // h: 256 rows x 128 bf16 (64 KiB); chunk c of row r at c ^ (4 * ((r >> 2) & 1))
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
    const int cl = wn * 32 + lrow;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int ch = (cl >> 3) ^ (4 * ((row >> 2) & 1));
        hs[row * 128 + ch * 8 + (cl & 7)] = f32_to_bf16_rne(silu_bf16out(acc[i][0][r]) * acc[i][1][r]);
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = q * 512 + tid;  // chunk idx % 16 (8 columns) of row idx / 16
      const int row = idx >> 4;
      const int ch = idx & 15;
      const int col = tc.nt * 128 + ch * 8;  // N % 64 == 0: a chunk is wholly in or out
      if (row < tc.rows && tc.row0 + row < TK && col < N)
        *reinterpret_cast<u32x4_t*>(hout + (int64_t)(tc.row0 + row) * N + col) =
            *reinterpret_cast<const u32x4_t*>(hs + row * 128 + (ch ^ (4 * ((row >> 2) & 1))) * 8);
    }
  } else if (tc.slot >= 0) {
    // a k-piece: the whole 256 x 256 partial tile goes to its slot
    float* dst = tail_ws + (int64_t)tc.slot * (BM * BN);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          dst[row * BN + wn * 64 + j * 32 + lrow] = acc[i][j][r];
        }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = tc.nt * 256 + wn * 64 + j * 32 + lrow;
        if (c >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          if (row < tc.rows && tc.row0 + row < TK) oout[(int64_t)(tc.row0 + row) * N + c] = acc[i][j][r];
        }
      }
  }
}

// Sums the k-pieces of each split tile in piece order and stores the rows of
// o it owns.  Workgroup b covers 16 rows of leftover tile t = (b / 16) % tmax
// of XCD b / (16 * tmax) (tmax = cus / 2 bounds the leftover tiles of an XCD
// that are split); it recomputes the XCD's plan exactly as the GEMM did.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const int* __restrict__ offsets, int n, int N,
                                                          int nk, int cus, int gran,
                                                          const float* __restrict__ tail_ws,
                                                          float* __restrict__ o) {
  const int NT = (N + 255) / 256;
  const int tmax = cus / 2;
  const int x = blockIdx.x / (16 * tmax);
  const int t = (blockIdx.x / 16) % tmax;
  const int rblk = blockIdx.x % 16;
  const ExpertTiles et = expert_tiles(offsets, n);
  const XcdPlan pl = xcd_plan(et.total * NT, x, cus, nk, true, gran);
  if (pl.s == 1 || t >= pl.r) return;
  Tile tc;
  if (!tile_at(offsets, et, NT, pl.beg + pl.q + t, tc)) return;
  // thread -> (row of 4 in this block's 16, 4 consecutive columns)
  const int c4 = (threadIdx.x & 63) * 4;
  const int c = tc.nt * 256 + c4;
  const int row0 = rblk * 16 + (threadIdx.x >> 6) * 4;
  // Every piece of the thread's 4 rows is loaded before any is added, so the
  // loads travel together instead of one round trip per piece; loads past the
  // piece count re-read the last piece (every piece holds all 256 rows) and
  // are not added.  The sum runs in piece order, as the pieces' order fixes.
  f32x4_t v[4][kMaxTailSplit];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int p = 0; p < kMaxTailSplit; ++p)
      v[k][p] = *reinterpret_cast<const f32x4_t*>(
          tail_ws + (int64_t)(x * cus + min(p, pl.s - 1) * pl.r + t) * (BM * BN) + (row0 + k) * BN + c4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = row0 + k;
    if (row >= tc.rows) break;
    f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kMaxTailSplit; ++p)
      if (p < pl.s) sum += v[k][p];
    float* dst = o + (int64_t)(tc.row0 + row) * N + c;
    if (c + 3 < N) {
      *reinterpret_cast<f32x4_t*>(dst) = sum;
    } else {
      for (int j = 0; j < 4 && c + j < N; ++j) dst[j] = sum[j];
    }
  }
}

}  // namespace

size_t prefill_tail_bytes(int cus_per_xcd) { return (size_t)kXcds * cus_per_xcd * BM * BN * sizeof(float); }

hipError_t launch_prefill_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W1,
                             const uint16_t* W3, const int* offsets, int64_t TK, int n, int d, int f,
                             int cus_per_xcd, uint16_t* h, hipStream_t s) {
  const int NT = (f + 127) / 128;
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(prefill_grid(TK, n, NT, cus_per_xcd)), dim3(512), 0, s,
                     x, perm_token, W1, W3, offsets, n, d, f, (int)T, (int)TK, cus_per_xcd, h,
                     (float*)nullptr, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const uint16_t* h, const uint16_t* W2, const int* offsets, int64_t TK,
                               int n, int f, int d, int cus_per_xcd, float* tail_ws, float* o,
                               hipStream_t s) {
  const int NT = (d + 255) / 256;
  hipLaunchKernelGGL((grouped_gemm_kernel<2>), dim3(prefill_grid(TK, n, NT, cus_per_xcd)), dim3(512), 0, s,
                     h, (const int*)nullptr, W2, (const uint16_t*)nullptr, offsets, n, f, d, (int)TK,
                     (int)TK, cus_per_xcd, (uint16_t*)nullptr, o, tail_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tail_ws == nullptr || cus_per_xcd < 2) return e;  // fewer CUs never split
  return launch_tail_reduce(offsets, n, d, f / BK, cus_per_xcd, 2, tail_ws, o, s);
}

hipError_t launch_tail_reduce(const int* offsets, int n, int N, int nk, int cus_per_xcd, int gran,
                              const float* tail_ws, float* o, hipStream_t s) {
  // split leftover tiles per XCD are at most cus / 2; 16 workgroups of 16 rows per tile
  hipLaunchKernelGGL(tail_reduce_kernel, dim3(kXcds * (cus_per_xcd / 2) * 16), dim3(256), 0, s, offsets, n, N,
                     nk, cus_per_xcd, gran, tail_ws, o);
  return hipGetLastError();
}

}  // namespace moe
