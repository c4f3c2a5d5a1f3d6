// Grouped expert GEMMs on weights stored in MFMA fragment order ("packed"),
// bf16 MFMA on gfx950.
//
// The projections are those of the layer's SwiGLU experts (card 2.1 "Sparse
// Mixture of Experts" of the "Mixtral of Experts" study deck; three d x f
// matrices per expert, Part 4 of "Mixture of Experts: Why Mixtral Only Wakes
// Up Two Specialists"):
//   up   (MODE 1): h[p] = SiLU(x[perm_token[p]] W1_e) * (x[perm_token[p]] W3_e) -> bf16
//   down (MODE 2): o[p] = h[p] W2_e -> fp32
//
// Packed format.  For v_mfma_f32_32x32x16_bf16, lane l of a B fragment holds
// the 8 consecutive reduction indices k = 16 kk + 8 (l / 32) + i (i = 0..7) of
// column l % 32.  A packed stack stores fragments contiguously, four column
// pairs (one group, the columns of one tile) side by side:
//     P[e][g][kk][w][j][l][i]      (bf16; kk = k / 16, w = 0..3, j = 0, 1, l = 0..63)
// so one fragment is 1 KiB, pair pb = 4 g + w, and a group's whole reduction
// is one contiguous stream of 8 KiB per kk.  Up projection (from W1, W3
// [n][d][f]): pair pb < f / 32 holds W1 columns 32 pb .. 32 pb + 31 (j = 0)
// and the same W3 columns (j = 1).  Down projection (from W2 [n][f][d]): pair
// pb < d / 64 holds columns 64 pb + 32 j .. + 31.
//
// Kernel.  A 256-thread workgroup (one wave per SIMD) computes 256-row tiles
// of one expert: 128 h columns (MODE 1; 128 of W1 and the matching 128 of W3)
// or 256 output columns (MODE 2).  Wave w owns all 256 rows against pair
// 4 nt + w: 8 row blocks x 2 fragments of 32x32 fp32 accumulators (256
// registers, kept in AGPRs).  Its weight fragments come from the packed stream
// straight into a ring of registers, PD k16-steps ahead, so the weights never
// pass through LDS (half the LDS traffic of staging both operands).  The
// gathered activation rows go through an LDS ring of PSA super-stages of 64 k
// (256 rows x 128 bytes), filled by direct-to-LDS loads that each wave waits
// for itself (s_waitcnt vmcnt, counted by issue order) before a barrier
// publishes the super-stage; chunk c of row r sits at c ^ ((r >> 1) & 7), so
// the 16 lanes of a 16-byte fragment read served together hit distinct banks.
// The last row tile of an expert is usually part padding: when a launch has
// enough tiles for unequal ones to even out, its padded 32-row blocks are
// neither multiplied nor stored (a copy of the k-loop per live-block count).
// MODE 1 takes the weights as the MFMA's row operand (each lane ends with 4
// consecutive h columns of a row: 8-byte stores, and the SiLU pairs stay in
// one lane); MODE 2 takes the activations (each store instruction writes whole
// 128-byte pieces of two o rows).
//
// One workgroup per compute unit, each looping over a work list of tiles (see
// below), so a tile's first loads fly while the previous tile's results are
// written.  Results equal the caller-layout kernels' bit for bit where no tile
// is split: the same MFMA, the same fragment contents and the same k order.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"
#include "tile_sched.h"

namespace moe {

namespace {

constexpr int A_SUPER = BM * 64 * 2;  // 32 KiB: 256 rows x 64 k
constexpr int PSA = 4;                // activation super-stages in LDS (128 KiB; a power of two keeps the slot a mask)
constexpr int PR = 8;                 // register ring of weight k16-steps
constexpr int PD = 7;                 // weight look-ahead in k16-steps
static_assert(PD < PR, "a weight load must not target the slot in use");
constexpr int kDS = 8;                // 1 KiB activation loads per wave per super-stage
// The barrier that publishes super-stage s + 1 (at step 4 s + 3) releases the slot of
// super-stage s - 1, whose last fragment reads were consumed by MFMAs several steps
// earlier, so the barrier need not wait for the wave's LDS reads: loads issued from
// there on fill super-stage s + PSA - 1 (PSA - LAG super-stages ahead of the one read).
constexpr int LAG = 2;

// Loads one wave issues, in order: the prologue (super-stages 0 .. PSA-LAG-1, kDS
// loads each; piece 0 of super-stage PSA-LAG, kDS/4 loads; the weights of steps
// 0 .. PD-1, 2 loads each), then per k16 step kk: kDS/4 loads of super-stage
// (kk+1)/4 + PSA - LAG (piece (kk+1) % 4) followed by the 2 weight loads of step
// kk + PD.  packed_after(st, kk) = loads issued after the last load of
// super-stage `st` when step `kk` begins.
constexpr int packed_after(int st, int kk) {
  const int pro = (PSA - LAG) * kDS + kDS / 4 + 2 * PD;
  int last = 0;
  if (st <= PSA - LAG - 1) {
    last = (st + 1) * kDS - 1;
  } else {
    const int kl = 4 * (st - PSA + LAG) + 2;  // step that issues the last piece
    last = pro + kl * (kDS / 4 + 2) + kDS / 4 - 1;
  }
  return pro + kk * (kDS / 4 + 2) - 1 - last;
}
// vmcnt bound that guarantees super-stage s+1 has landed at the barrier of
// step 4s+3, for every s: the smallest count over the first super-stages
// (prologue) and the steady state (reached by s = PSA - 1).
constexpr int packed_wait_stage() {
  int w = 63;
  for (int s = 0; s < 3 * PSA; ++s) {
    const int c = packed_after(s + 1, 4 * s + 3);
    if (c < w) w = c;
  }
  return w;
}
constexpr int W_STAGE = packed_wait_stage();
constexpr int W_FIRST = packed_after(0, 0);
static_assert(W_STAGE >= 0 && W_STAGE <= 63 && W_FIRST <= 63, "vmcnt is a 6-bit counter");
// The same bound when the previous tile's epilogue issued the stores of `blocks` row
// blocks after these loads (4 store instructions per row block in MODE 1, 32 in MODE 2).
constexpr int packed_w_late(int mode, int blocks) {
  const int w = W_FIRST + blocks * (mode == 1 ? 4 : 32);
  return w < 63 ? w : 63;
}

// Work-list words (int32) of one launch: taken[kXcds] counts the positions
// handed out beyond the first `cus` of each XCD's share (zero at launch), and
// kHandoffWords hold two hand-over words per workgroup (at most 8 x 64
// workgroups): word 0 for a workgroup without a first position of its own,
// word 1 for the position after each tile.
constexpr int kHandoffWords = 2 * kXcds * 64;
static_assert(kPackedCounterWords == 2 * kXcds && kPackedSchedWords == kPackedCounterWords + 2 * kHandoffWords,
              "work-list words of the two projections");

// 32-row blocks of a tile that hold rows of the expert (the rest are padding)
__device__ __forceinline__ int live_blocks(const Tile& t) { return (t.rows + 31) >> 5; }

// An accumulator register read where it is used (the compiler would copy all
// 256 accumulators to VGPRs at once ahead of the SwiGLU epilogue).
__device__ __forceinline__ float agpr(float v) {
  float r;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
  return r;
}

#ifdef MOE_TILE_TRACE
// Per-tile timeline (tile-trace build only): for each projection, workgroup and
// tile in the order the workgroup ran them, five moments read from the constant
// 100 MHz counter (s_memrealtime) and from the shader clock counter (s_memtime):
// k-loop start (after the tile's first barrier), k-loop end, after the closing
// barrier, after the next tile's loads are issued, after the epilogue; then the
// tile's live row blocks and k-steps, and the row blocks its k-loop multiplies.
__device__ long long g_tile_trace[2][kTileTraceWgs][kTileTraceTiles][kTileTraceFields];
#endif

template <int MODE>
__global__ __launch_bounds__(256, 1) void packed_gemm_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token,
    // not __restrict__: loads through a restrict pointer to read-only data may be
    // moved across the asm statements whose issue order the waits count on
    const uint16_t* Bp, const int* __restrict__ offsets, int n, int Kdim, int N, int a_rows, int TK, int cus,
    uint16_t* __restrict__ hout, float* __restrict__ oout, float* __restrict__ tail_ws, int* taken, int* handoffs) {
  __shared__ __attribute__((aligned(1024))) char smem[PSA * A_SUPER];
  constexpr int NTW = (MODE == 1) ? 128 : 256;  // output columns per tile
  const int NT = N / NTW;
  const int nk = Kdim / BK;
  // pieces of split tiles are whole unrolled loops: PR k16-steps = PR / 2 k-steps of 32
  const bool may_split = MODE == 2 && tail_ws != nullptr;
  const ExpertTiles et = expert_tiles(offsets, n);
  const int total = et.total * NT;
  // Padded row blocks are skipped when the launch has at least 8 tiles per compute unit:
  // tiles of unequal length then even out over the work list.  With only a few long tiles
  // per unit (the long-reduction down projection) equal tiles keep the per-XCD shares,
  // which assume equal tiles, finishing together.
  const bool skip_padding = total >= 8 * kXcds * cus;
  auto nb_of = [&](const Tile& t) { return skip_padding ? live_blocks(t) : 8; };
  const int x = blockIdx.x % kXcds;
  int* const handoff = handoffs + 2 * blockIdx.x;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work list.  Position pos of XCD xq's share is coded pos * kXcds + xq (-1:
  // none).  Workgroup (x, i) starts at position i of its XCD's share; later
  // positions are handed out in order by an atomic counter per XCD, and a
  // workgroup whose own share is used up takes positions of the other XCDs.
  // Wave 0 asks for the next position when a tile starts (the atomic's answer
  // comes in while the tile runs) and hands it to the other waves through a
  // word in global memory (the LDS is all taken by the activation ring),
  // written before the tile's closing barrier and read after it.  Holding one
  // position ahead, not two, keeps the workgroups' end times within about one
  // tile of each other.
  const int len_l = lane < kXcds ? queue_len(xcd_plan(total, lane, cus, nk, may_split, PR / 2)) : 0;
  auto share_len = [&](int xq) { return __builtin_amdgcn_readlane(len_l, xq); };
  auto tile_of = [&](int c, Tile& t) -> bool {
    const int xq = c % kXcds;
    return queue_tile(offsets, et, NT, nk, cus, xq, xcd_plan(total, xq, cus, nk, may_split, PR / 2), c / kXcds, t);
  };
  const bool own_dynamic = share_len(x) > cus;
  // wave 0 only: a request on the own counter (the answer, in lane 0, is read later)
  auto request = [&]() -> int {
    int v = INT32_MAX;
    if (own_dynamic && lane == 0) {
      // an index the compiler cannot prove uniform: it would otherwise turn the
      // add into a wave-wide one whose result is needed (and waited for) at once
      int z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      v = atomicAdd(&taken[x + z], 1);
    }
    return v;
  };
  // wave 0 only: the position a request gave, or one taken from another XCD's share
  auto settle = [&](int req) -> int {
    const int raw = __builtin_amdgcn_readfirstlane(req);
    if (raw != INT32_MAX && cus + raw < share_len(x)) return (cus + raw) * kXcds + x;
    for (int k = 1; k < kXcds; ++k) {
      const int xq = (x + k) % kXcds;
      const int len = share_len(xq);
      if (len <= cus) continue;
      int v = 0;
      if (lane == 0) v = atomicAdd(&taken[xq], 1);
      const int pos = cus + __builtin_amdgcn_readfirstlane(v);
      if (pos < len) return pos * kXcds + xq;
    }
    return -1;
  };

  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  int cur;
  const int i0 = blockIdx.x / kXcds;
  if (i0 < share_len(x)) {
    cur = i0 * kXcds + x;
  } else {
    int c = -1;
    if (wave == 0) {
      c = settle(request());
      if (lane == 0) __hip_atomic_store(&handoff[0], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(WAITCNT_ALL);
    fence();
    __builtin_amdgcn_s_barrier();
    fence();
    if (wave != 0) c = __hip_atomic_load(&handoff[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cur = __builtin_amdgcn_readfirstlane(c);
  }
  Tile tc;
  if (cur < 0 || !tile_of(cur, tc)) return;

  // activation loads: wave w fills blocks 8w .. 8w+7 of each super-stage (8 rows x 128 bytes each)
  const uint16_t* ld_ptr[kDS];
  const uint32_t a_ld_base = (uint32_t)(uintptr_t)(lds_void*)smem + wave * (kDS * 1024);
  const int KK = Kdim / 16;
  const int G = (MODE == 1) ? N / 128 : N / 256;
  const uint16_t* bptr;
  int nk16, nss, kbase;
  // source rows of the wave's activation loads (MODE 1: gathered through perm_token)
  auto rows_of = [&](const Tile& t, int (&src)[kDS]) {
#pragma unroll
    for (int b = 0; b < kDS; ++b) {
      const int r = (wave * kDS + b) * 8 + (lane >> 3);
      const int rr = r < t.rows ? r : t.rows - 1;  // padded rows repeat the last row
      const int p = min(max(t.row0 + rr, 0), TK - 1);
      src[b] = (MODE == 1) ? perm_token[p] : p;
    }
  };
  auto setup = [&](const Tile& t, const int (&src)[kDS]) {
#pragma unroll
    for (int b = 0; b < kDS; ++b) {
      const int r = (wave * kDS + b) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int row = (MODE == 1) ? min(max(src[b], 0), a_rows - 1) : src[b];
      ld_ptr[b] = A + (int64_t)row * Kdim + c * 8;
    }
    // the wave's weight stream (pair 4 nt + wave of group nt), from the tile's first k16-step
    bptr = Bp + (((int64_t)(t.e * G + t.nt) * KK + t.k0 * 2) * 4 + wave) * 1024 + lane * 8;
    nk16 = (t.k1 - t.k0) * 2;  // a multiple of PR
    nss = nk16 / 4;
    kbase = t.k0 / 2;
  };
  // Loads past the end re-load the last k-slice (into slots nobody reads
  // again), so every wave issues the same sequence and the counts hold.
  auto issue_a = [&](int stage, int b0, int nb) {
    const uint32_t dst = a_ld_base + (stage % PSA) * A_SUPER;
    const int64_t koff = (int64_t)(kbase + min(stage, nss - 1)) * 64;
#pragma unroll
    for (int b = 0; b < nb; ++b) load_lds16(ld_ptr[b0 + b] + koff, dst + (b0 + b) * 1024);
  };
  auto load_b = [&](int kk, bf16x8_t (&dst)[2]) {
    const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(bptr + (int64_t)min(kk, nk16 - 1) * 4096);
    dst[0] = src[0];
    dst[1] = src[64];
  };
  bf16x8_t br[PR][2];
  auto prologue = [&] {
#pragma unroll
    for (int st = 0; st < PSA - LAG; ++st) issue_a(st, 0, kDS);
    issue_a(PSA - LAG, 0, kDS / 4);
#pragma unroll
    for (int t = 0; t < PD; ++t) load_b(t, br[t]);
  };

  // fragment i of sub-step q (k 16 q .. +15 of a super-stage): row 32 i + l % 32, chunk 2 q + l / 32
  const int m = lane & 31;
  const int kg = lane >> 5;
  int a_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) a_off[q] = m * 128 + (((2 * q + kg) ^ ((m >> 1) & 7)) * 16);

  f32x16_t acc[8][2];
  // Writes row blocks [ib, ie) of a finished tile.  32x32 MFMA D layout: register r of lane l is
  // D row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  A padded row (past the tile's rows) was
  // computed from the tile's last row, so its values equal that row's: it is stored there again,
  // and every wave issues the same number of stores whatever the tile (the waits count on it).
  auto epilogue = [&](const Tile& t, int ib, int ie) {
    if (MODE == 1) {
      // weights as the row operand: register 4 q + c of fragment (i, j) is tile row 32 i + l % 32,
      // column 8 q + 4 (l / 32) + c of the pair's fragment j.  h: four consecutive bf16 (8 bytes)
      // per (row block, q); the 4 waves' 32-column blocks and the q groups complete each row's
      // 256 bytes in L2
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < ib || i >= ie || i >= nb_of(t)) continue;
        const int row = min(i * 32 + m, t.rows - 1);
        uint16_t* hrow = hout + (int64_t)(t.row0 + row) * N + t.nt * 128 + wave * 32 + 4 * kg;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w2[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int r0 = 4 * q + 2 * h2;
            const f32x2_t v = {silu_bf16out(agpr(acc[i][0][r0])) * agpr(acc[i][1][r0]),
                               silu_bf16out(agpr(acc[i][0][r0 + 1])) * agpr(acc[i][1][r0 + 1])};
            w2[h2] = bf16x2_rne(v);
          }
          *reinterpret_cast<u32x2_t*>(hrow + 8 * q) = u32x2_t{w2[0], w2[1]};
        }
        fence();  // one row block's values live at a time
      }
    } else {
      // o rows, or for a k-piece the whole 256 x 256 partial tile in its slot (one code
      // path, so the store count is the same either way).  Activations as the row operand:
      // register r of fragment (i, j) is tile row 32 i + 8 (r / 4) + 4 (l / 32) + r % 4,
      // column 32 j + l % 32 of the wave's 64, so each store covers two whole 128-byte row
      // pieces (first writes that cover only parts of lines were found much slower).
      const bool piece = t.slot >= 0;
      float* const base = piece ? tail_ws + (int64_t)t.slot * (BM * BN) : oout + (int64_t)t.row0 * N + t.nt * 256;
      const int64_t ld = piece ? BN : N;
      const int last = piece ? BM - 1 : t.rows - 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < ib || i >= ie || i >= nb_of(t)) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* orow = base + (int64_t)min(i * 32 + 8 * (r / 4) + 4 * kg + (r % 4), last) * ld + wave * 64 + m;
          orow[0] = acc[i][0][r];
          orow[32] = acc[i][1][r];
        }
      }
    }
  };

  {
    int src[kDS];
    rows_of(tc, src);
    setup(tc, src);
  }
  prologue();
  // wave 0: the request for the position after cur stays in flight during the
  // tile and is settled just before the tile's closing barrier
  int pending = INT32_MAX;
  if (wave == 0) pending = request();

  // Super-stage 0 of a tile has landed once at most W_FIRST of the loads issued
  // after it are outstanding, plus whatever was issued after those loads (all
  // vector memory operations of a wave complete in issue order): after a
  // previous tile, the stores of its row blocks 4 .. 7 that hold rows.
  int late_blocks = 0;
#ifdef MOE_TILE_TRACE
  int traced = 0;
  auto stamp = [&](int k) {
    const long long rt = __builtin_amdgcn_s_memrealtime();
    const long long ct = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0 && traced < kTileTraceTiles && blockIdx.x < kTileTraceWgs) {
      long long* rec = g_tile_trace[MODE - 1][blockIdx.x][traced];
      rec[k] = rt;
      rec[5 + k] = ct;
      if (k == 0) {
        rec[10] = nb_of(tc) + 16LL * (tc.k1 - tc.k0);
        rec[11] = max(2, nb_of(tc));  // row blocks the k-loop multiplies (see the switch below)
      }
    }
  };
#define MOE_STAMP(k) stamp(k)
#else
#define MOE_STAMP(k)
#endif
  for (;;) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    switch (late_blocks) {
      case 0: __builtin_amdgcn_s_waitcnt(waitcnt_imm(packed_w_late(MODE, 0), 15)); break;
      case 1: __builtin_amdgcn_s_waitcnt(waitcnt_imm(packed_w_late(MODE, 1), 15)); break;
      case 2: __builtin_amdgcn_s_waitcnt(waitcnt_imm(packed_w_late(MODE, 2), 15)); break;
      case 3: __builtin_amdgcn_s_waitcnt(waitcnt_imm(packed_w_late(MODE, 3), 15)); break;
      default: __builtin_amdgcn_s_waitcnt(waitcnt_imm(packed_w_late(MODE, 4), 15)); break;
    }
    fence();
    __builtin_amdgcn_s_barrier();
    fence();
    MOE_STAMP(0);

    // Step kk: 2 NB MFMAs on the fragments read during step kk-1, NB = the tile's
    // live 32-row blocks (rows past the tile's end are neither multiplied nor
    // stored); after each row block's two MFMAs, that block's fragment of step
    // kk+1 is read.  After the first block's turn come this step's activation
    // loads (a quarter of a super-stage, into the slot the last barrier released),
    // after the fourth's the weight loads of step kk + PD: every wave issues the
    // same loads whatever NB is.  The last step of each super-stage starts with the
    // barrier that publishes the next super-stage and releases the slot of the
    // previous one.
    auto kloop = [&](auto nb_c) {
      constexpr int NB = decltype(nb_c)::value;
      bf16x8_t a[8];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(smem + i * 4096 + a_off[0]);
        fence();  // in block order, as in the loop: the loop's first wait then covers one read
      }
      for (int base = 0; base < nk16; base += PR) {
#pragma unroll
        for (int u = 0; u < PR; ++u) {
          const int kk = base + u;
          if ((u & 3) == 3) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(W_STAGE, 15));  // own loads of super-stage kk/4 + 1 landed
            fence();
            __builtin_amdgcn_s_barrier();
            fence();
          }
          const int stn = (kk + 1) >> 2;  // super-stage of step kk+1
          const char* an = smem + (stn % PSA) * A_SUPER + a_off[(u + 1) & 3];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (i < NB) {
              if (MODE == 1) {
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(br[u][0], a[i], acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(br[u][1], a[i], acc[i][1], 0, 0, 0);
              } else {
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], br[u][0], acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], br[u][1], acc[i][1], 0, 0, 0);
              }
              a[i] = *reinterpret_cast<const bf16x8_t*>(an + i * 4096);
            }
            if (i == 0) {
              fence();
              issue_a(stn + PSA - LAG, ((u + 1) & 3) * (kDS / 4), kDS / 4);
              fence();
            }
            if (i == 3) {
              fence();
              load_b(kk + PD, br[(u + PD) % PR]);
              fence();
            }
          }
          fence();  // the next step's fragment reads stay in this step
        }
      }
    };
    // (a one-block loop would wait for its single fragment read at the head of every
    // step, a wait for every LDS read: such tiles take the two-block loop)
    switch (nb_of(tc)) {
      case 1:
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 5: kloop(std::integral_constant<int, 5>{}); break;
      case 6: kloop(std::integral_constant<int, 6>{}); break;
      case 7: kloop(std::integral_constant<int, 7>{}); break;
      default: kloop(std::integral_constant<int, 8>{}); break;
    }
    MOE_STAMP(1);
    // wave 0: the next position, handed to the other waves through handoff[1]
    // (read after the barrier; the word is written again only after the next
    // tile's first barrier, when every wave has read it)
    if (wave == 0) {
      const int nx = settle(pending);
      if (lane == 0) __hip_atomic_store(&handoff[1], nx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Every wave's loads have landed (the last, redundant ones included), its
    // LDS reads are done and wave 0's hand-over word is written: after the
    // barrier the ring may take the next tile.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    fence();
    __builtin_amdgcn_s_barrier();
    fence();
    MOE_STAMP(2);
    // The transition to the next tile is interleaved with this tile's epilogue:
    // row blocks 0-1 are written while the hand-over word comes in, 2-3 while
    // the next tile's gathered row indices come in, 4-7 while its first
    // super-stages and weight steps load.
    int c = __hip_atomic_load(&handoff[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const Tile told = tc;
    epilogue(told, 0, 2);
    fence();
    c = __builtin_amdgcn_readfirstlane(c);
    const bool more = c >= 0 && tile_of(c, tc);
    int src[kDS];
    if (more) rows_of(tc, src);
    fence();
    epilogue(told, 2, 4);
    fence();
    if (more) {
      setup(tc, src);
      prologue();
      if (wave == 0) pending = request();
    }
    fence();
    MOE_STAMP(3);
    epilogue(told, 4, 8);
    MOE_STAMP(4);
#ifdef MOE_TILE_TRACE
    ++traced;
#endif
    late_blocks = max(0, nb_of(told) - 4);
    if (!more) break;
    fence();
  }
#undef MOE_STAMP
}

// Weight streaming on packed weights, for decode-sized batches (a few rows per
// expert): every touched expert's packed stream is read once from HBM.  One
// wave (one workgroup) per (expert, two adjacent column pairs[, k-split]): it
// walks 4 KiB of weights per k16-step, SPR steps of loads in flight, and
// multiplies a 32-row pass of the expert's rows (gathered x rows, or h rows)
// with the four fragments.  The activation fragment comes straight from global
// memory (x and h are small and stay in L2); two pairs per wave keep those
// reads at a quarter of the weight bytes (one pair per wave made them half,
// and the up projection ran 6% slower; four pairs per wave left too few waves
// in flight).  Every load here is an ordinary compiler-tracked load, so the
// compiler's own waits are exact.  An expert with more than 32 rows takes
// further passes over its weights; one with none returns at once, so
// unselected experts are never read.
//   MODE 1: h rows of the pass = SiLU(a) * b (the whole reduction per wave).
//   MODE 2: o[split][row] = the split's partial sum over its k range.
constexpr int SPR = 5;  // k16-steps of loads in flight per wave
constexpr int SQ = 2;  // column pairs per wave: 4 KiB of weights per 1 KiB activation fragment per k16-step

template <int MODE>
__global__ __launch_bounds__(64) void packed_stream_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token, const uint16_t* __restrict__ Bp,
    const int* __restrict__ offsets, int n, int Kdim, int N, int a_rows, int TK, int splits,
    uint16_t* __restrict__ hout, float* __restrict__ oout) {
  const int P = (MODE == 1) ? N / 32 : N / 64;
  const int units = P / SQ;  // waves per expert and split
  const int wg = blockIdx.x;
  const int split = wg % splits;
  const int u0 = (wg / splits) % units;
  const int e = wg / (splits * units);
  if (e >= n) return;
  const int row_beg = offsets[e];
  const int rows = offsets[e + 1] - row_beg;
  if (rows <= 0) return;
  const int lane = threadIdx.x & 63;
  const int pb0 = u0 * SQ;          // first pair; pairs pb0 .. pb0 + SQ - 1 lie in group pb0 / 4
  const int g = pb0 / 4;
  const int w0 = pb0 % 4;
  const int KK = Kdim / 16;
  const int kb = (int)((int64_t)KK * split / splits);
  const int ke = (int)((int64_t)KK * (split + 1) / splits);
  const int nst = ke - kb;
  const int G = P / 4;
  const uint16_t* bptr = Bp + (((int64_t)(e * G + g) * KK + kb) * 4 + w0) * 1024 + lane * 8;
  const int m = lane & 31;
  const int kg = lane >> 5;

  for (int r0 = 0; r0 < rows; r0 += 32) {
    const int p = row_beg + min(r0 + m, rows - 1);
    const int arow = (MODE == 1) ? min(max(perm_token[p], 0), a_rows - 1) : p;
    const uint16_t* aptr = A + (int64_t)arow * Kdim + (int64_t)kb * 16 + kg * 8;
    f32x16_t acc[SQ][2];
#pragma unroll
    for (int q = 0; q < SQ; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][j][r] = 0.0f;
    bf16x8_t ra[SPR], rb[SPR][SQ][2];
    auto load = [&](int kk, int slot) {
      const int k = min(kk, nst - 1);
      ra[slot] = *reinterpret_cast<const bf16x8_t*>(aptr + (int64_t)k * 16);
      const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(bptr + (int64_t)k * 4096);
#pragma unroll
      for (int q = 0; q < SQ; ++q) {
        rb[slot][q][0] = ld_stream(src + q * 128);
        rb[slot][q][1] = ld_stream(src + q * 128 + 64);
      }
    };
#pragma unroll
    for (int t = 0; t < SPR - 1; ++t) load(t, t);
    for (int base = 0; base < nst; base += SPR) {
#pragma unroll
      for (int u = 0; u < SPR; ++u) {
        load(base + u + SPR - 1, (u + SPR - 1) % SPR);
        if (base + u < nst) {
#pragma unroll
          for (int q = 0; q < SQ; ++q) {
            acc[q][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[u], rb[u][q][0], acc[q][0], 0, 0, 0);
            acc[q][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[u], rb[u][q][1], acc[q][1], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 8 * (r >> 2) + 4 * kg + (r & 3);
      if (row >= rows) continue;
      const int64_t prow = row_beg + row;
#pragma unroll
      for (int q = 0; q < SQ; ++q) {
        const int pb = pb0 + q;
        if (MODE == 1) {
          hout[prow * N + 32 * pb + m] = f32_to_bf16_rne(silu_bf16out(acc[q][0][r]) * acc[q][1][r]);
        } else {
          float* dst = oout + ((int64_t)split * TK + prow) * N + 64 * pb + m;
          dst[0] = acc[q][0][r];
          dst[32] = acc[q][1][r];
        }
      }
    }
  }
}

// Repacks bf16 W[n][R][C] into the fragment order above (MODE 1: with the
// matching W3 as fragment j = 1).  One thread per 16-byte fragment lane
// out[e][g][kk][w][j][l][0..7]; its 8 values are one column's 8 consecutive rows.
template <int MODE>
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W, const uint16_t* __restrict__ W3,
                                                   int n, int R, int C, uint16_t* __restrict__ out) {
  const int P = (MODE == 1) ? C / 32 : C / 64;
  const int KK = R / 16;
  const int64_t total = (int64_t)n * P * KK * 2 * 64;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(g & 63);
    const int j = (int)((g >> 6) & 1);
    const int wp = (int)((g >> 7) & 3);
    int64_t t = g >> 9;
    const int kk = (int)(t % KK);
    t /= KK;
    const int grp = (int)(t % (P / 4));
    const int e = (int)(t / (P / 4));
    const int pb = 4 * grp + wp;
    const uint16_t* src = (MODE == 1 && j == 1) ? W3 : W;
    const int col = (MODE == 1) ? 32 * pb + (l & 31) : 64 * pb + 32 * j + (l & 31);
    const uint16_t* s = src + ((int64_t)e * R + 16 * kk + 8 * (l >> 5)) * C + col;
    u32x4_t w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)s[(int64_t)(2 * q) * C] | ((uint32_t)s[(int64_t)(2 * q + 1) * C] << 16);
    *reinterpret_cast<u32x4_t*>(out + g * 8) = w;
  }
}

}  // namespace

hipError_t launch_packed_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W13p,
                            const int* offsets, int64_t TK, int n, int d, int f, int cus_per_xcd, int* sched,
                            uint16_t* h, hipStream_t s) {
  if (cus_per_xcd < 1 || cus_per_xcd > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL((packed_gemm_kernel<1>), dim3(kXcds * cus_per_xcd), dim3(256), 0, s, x, perm_token, W13p,
                     offsets, n, d, f, (int)T, (int)TK, cus_per_xcd, h, (float*)nullptr, (float*)nullptr, sched,
                     sched + kPackedCounterWords);
  return hipGetLastError();
}

hipError_t launch_packed_down(const uint16_t* h, const uint16_t* W2p, const int* offsets, int64_t TK, int n, int f,
                              int d, int cus_per_xcd, int* sched, float* tail_ws, float* o, hipStream_t s) {
  if (cus_per_xcd < 1 || cus_per_xcd > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL((packed_gemm_kernel<2>), dim3(kXcds * cus_per_xcd), dim3(256), 0, s, h, (const int*)nullptr,
                     W2p, offsets, n, f, d, (int)TK, (int)TK, cus_per_xcd, (uint16_t*)nullptr, o, tail_ws,
                     sched + kXcds, sched + kPackedCounterWords + kHandoffWords);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tail_ws == nullptr || cus_per_xcd < 2) return e;  // fewer CUs never split
  return launch_tail_reduce(offsets, n, d, f / BK, cus_per_xcd, PR / 2, tail_ws, o, s);
}

int packed_stream_splits(int n, int f, int d, int cus_per_xcd) {
  // about 3 down-projection waves per compute unit (measured best at the
  // Mixtral decode shape: 3 splits of f; 2 and 4 were slower)
  const int waves = n * (d / 64) / SQ;
  const int want = (3 * 8 * cus_per_xcd + waves / 2) / waves;
  return std::max(1, std::min(std::min(want, 8), f / 128));
}

hipError_t launch_packed_stream_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W13p,
                                   const int* offsets, int64_t TK, int n, int d, int f, uint16_t* h, hipStream_t s) {
  const int units = (f / 32) / SQ;
  hipLaunchKernelGGL((packed_stream_kernel<1>), dim3(n * units), dim3(64), 0, s, x, perm_token, W13p, offsets, n, d,
                     f, (int)T, (int)TK, 1, h, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_packed_stream_down(const uint16_t* h, const uint16_t* W2p, const int* offsets, int64_t TK, int n,
                                     int f, int d, int splits, float* o, hipStream_t s) {
  const int units = (d / 64) / SQ;
  hipLaunchKernelGGL((packed_stream_kernel<2>), dim3(n * units * splits), dim3(64), 0, s, h, (const int*)nullptr,
                     W2p, offsets, n, f, d, (int)TK, (int)TK, splits, (uint16_t*)nullptr, o);
  return hipGetLastError();
}


#ifdef MOE_TILE_TRACE
hipError_t tile_trace_read(long long* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_tile_trace), sizeof(g_tile_trace), 0, hipMemcpyDeviceToHost);
}
hipError_t tile_trace_clear() {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_tile_trace));
  if (e != hipSuccess) return e;
  e = hipMemset(p, 0, sizeof(g_tile_trace));
  if (e != hipSuccess) return e;
  return hipDeviceSynchronize();
}
#endif

hipError_t launch_pack(int mode, const uint16_t* W, const uint16_t* W3, int n, int R, int C, uint16_t* out,
                       hipStream_t s) {
  if (mode == 1)
    hipLaunchKernelGGL((pack_kernel<1>), dim3(4096), dim3(256), 0, s, W, W3, n, R, C, out);
  else
    hipLaunchKernelGGL((pack_kernel<2>), dim3(4096), dim3(256), 0, s, W, W3, n, R, C, out);
  return hipGetLastError();
}

}  // namespace moe
