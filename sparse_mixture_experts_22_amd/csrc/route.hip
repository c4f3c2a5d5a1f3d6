// Router, top-K selection, softmax over the kept logits, and the integer
// dispatch that groups (token, slot) assignments by expert.
//
// Steps 1-3 of "Pip's token goes to triage" (Part 3 of "Mixture of Experts:
// Why Mixtral Only Wakes Up Two Specialists"): a bias-free linear layer scores
// the n experts, the K best are kept, a softmax over those K gives the weights.
// The dispatch realises the sparse-gating remark of "How a mixture-of-experts
// model activates only part of its parameters": experts with a zero gate are
// never evaluated, so each expert's rows are gathered into one contiguous group.
//
// Kernels (bf16 path):
//   wg_transpose_kernel  W_g [d][n] -> WgT [n_pad][d] (zero rows past n), so an
//                        MFMA B fragment (8 consecutive k of one expert) is one
//                        16-byte load.
//   router_bf16_kernel   a workgroup owns BT tokens; its W waves split the d
//                        reduction, each accumulating logits with
//                        v_mfma_f32_16x16x32_bf16 from x and WgT read straight
//                        from global memory; the W partial tiles are summed in
//                        LDS in wave order, then top-K + softmax + the block's
//                        expert histogram.  With a single routing block the
//                        same kernel also performs the scan and the scatter.
//   router_wave_kernel   many tokens and n in {32, 64, 128, 256}: one routing
//                        block per wave with the whole d reduction, W_g shared
//                        through LDS in its own layout (no transposed copy),
//                        top-K by wave-wide arg-max rounds.
//   router_split_kernel  one routing block (decode) and n <= 16: the d
//   + router_finish_kernel reduction split over workgroups, then one workgroup
//                        adds the partials and runs top-K and the dispatch.
//   scan_kernel          one workgroup: per-block bases (offsets[e] plus the
//                        assignments to e in earlier blocks), counts, offsets
//                        (scan4_kernel: the same with 16-byte rows, n % 4 == 0).
//   scatter_kernel       per block: rank of each assignment among the block's
//                        tokens that chose the same expert (LDS bitmask +
//                        popcount), position = base + rank.
// fp32 path: router_f32_kernel (fp32 FMA dot products) feeds the same scan and
// scatter.  Everything is integer or fixed-order fp32: bit-reproducible.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-K + softmax for token i of a block from logits_s[i*ld + e]: an insertion
// over the experts in index order into K slots kept in (score descending, index
// ascending) order.  The element being placed takes slot j if that slot is
// empty, holds a smaller score, or holds an equal score of a higher index (this
// last case arises only for an element pushed down from an earlier slot, whose
// index is lower than every later expert's); so ties keep the lower expert
// index, also below a larger later score.  NaN scores count as -inf, and every
// slot ends up holding a valid expert.  Returns the kept experts in id[].
__device__ void topk_softmax(const float* logits_s, int ld, int i, int n, int K, int (&id)[kMaxK],
                             float (&w)[kMaxK]) {
  if (K == 2) {
    // the same insertion with two slots, unrolled: the element pushed down
    // from slot 0 always outranks slot 1 (higher score, or an equal score of
    // a lower index), so it simply moves there
    float v0 = -INFINITY, v1 = -INFINITY;
    int i0 = -1, i1 = -1;
    for (int e = 0; e < n; ++e) {
      float cv = logits_s[i * ld + e];
      if (cv != cv) cv = -INFINITY;
      if (i0 < 0 || cv > v0) {
        v1 = v0;
        i1 = i0;
        v0 = cv;
        i0 = e;
      } else if (i1 < 0 || cv > v1) {
        v1 = cv;
        i1 = e;
      }
    }
    // the generic path's softmax, term by term (same values, same order)
    const float w0 = expf(v0 - v0);
    const float w1 = expf(v1 - v0);
    const float sum = (0.0f + w0) + w1;
    id[0] = i0;
    id[1] = i1;
    w[0] = w0 / sum;
    w[1] = w1 / sum;
    return;
  }
  float v[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    v[j] = -INFINITY;
    id[j] = -1;
  }
  for (int e = 0; e < n; ++e) {
    float cv = logits_s[i * ld + e];
    if (cv != cv) cv = -INFINITY;
    int ci = e;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < K && (id[j] < 0 || cv > v[j] || (cv == v[j] && ci < id[j]))) {
        const float tv = v[j];
        const int ti = id[j];
        v[j] = cv;
        id[j] = ci;
        cv = tv;
        ci = ti;
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      w[j] = expf(v[j] - v[0]);
      sum += w[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < K) w[j] = w[j] / sum;
}

// Shared epilogue of both routers: top-K for the block's tokens, then either
// the block histogram (multi-block) or the whole dispatch (single block).
// sel_s: [BT*K] ints, mask_s: [n] uint32 (BT <= 32), hist_s: [n] ints.
__device__ void route_epilogue(const float* logits_s, int ld, int BT, int64_t t0, int64_t T, int n,
                               int K, int* __restrict__ topk_idx, float* __restrict__ topk_w,
                               int* __restrict__ hist, bool fused, int* __restrict__ counts,
                               int* __restrict__ offsets, int* __restrict__ perm_token,
                               int* __restrict__ slot_pos, int* sel_s, uint32_t* mask_s,
                               int* hist_s, float* __restrict__ probsum, int cap,
                               float* __restrict__ ec_probs) {
  const int tid = threadIdx.x;
  const int cnt = (int)((T - t0) < BT ? (T - t0) : BT);
  __shared__ float tmax_s[32], tsum_s[32];
  if (ec_probs != nullptr) {
    // expert-choice scores: each token's full softmax over the n experts
    if (tid < cnt) {
      float mx = -INFINITY;
      for (int e = 0; e < n; ++e) mx = fmaxf(mx, logits_s[tid * ld + e]);
      float sm = 0.0f;
      for (int e = 0; e < n; ++e) sm += expf(logits_s[tid * ld + e] - mx);
      tmax_s[tid] = mx;
      tsum_s[tid] = sm;
    }
    __syncthreads();
    for (int idx = tid; idx < cnt * n; idx += blockDim.x) {
      const int i = idx / n;
      const int e = idx % n;
      ec_probs[(t0 + i) * n + e] = expf(logits_s[i * ld + e] - tmax_s[i]) / tsum_s[i];
      slot_pos[(t0 + i) * n + e] = -1;  // the selection writes only the chosen slots
    }
    return;
  }
  for (int e = tid; e < n; e += blockDim.x) {
    hist_s[e] = 0;
    mask_s[e] = 0u;
  }
  __syncthreads();
  if (tid < cnt) {
    int id[kMaxK];
    float w[kMaxK];
    topk_softmax(logits_s, ld, tid, n, K, id, w);
    const int64_t t = t0 + tid;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < K) {
        topk_idx[t * K + j] = id[j];
        topk_w[t * K + j] = w[j];
        sel_s[tid * K + j] = id[j];
        atomicAdd(&hist_s[id[j]], 1);          // integer: order-independent
        atomicOr(&mask_s[id[j]], 1u << tid);   // token tid chose expert id[j]
      }
    }
    if (probsum != nullptr) {
      // full n-way softmax of the token (router statistics): max, then the
      // sum of exponentials in expert order
      float mx = -INFINITY;
      for (int e = 0; e < n; ++e) mx = fmaxf(mx, logits_s[tid * ld + e]);
      float sm = 0.0f;
      for (int e = 0; e < n; ++e) sm += expf(logits_s[tid * ld + e] - mx);
      tmax_s[tid] = mx;
      tsum_s[tid] = sm;
    }
  }
  __syncthreads();
  if (probsum != nullptr) {
    // this block's sum over its tokens (in token order) of each expert's probability
    for (int e = tid; e < n; e += blockDim.x) {
      float acc = 0.0f;
      for (int i = 0; i < cnt; ++i) acc += expf(logits_s[i * ld + e] - tmax_s[i]) / tsum_s[i];
      probsum[(int64_t)blockIdx.x * n + e] = acc;
    }
  }
  if (!fused) {
    for (int e = tid; e < n; e += blockDim.x) hist[(int64_t)blockIdx.x * n + e] = hist_s[e];
    return;
  }
  // single routing block: offsets = exclusive scan of the block histogram,
  // each expert keeping at most `cap` assignments (the earliest tokens)
  __shared__ int base_s[kMaxN + 1];
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < n; ++e) {
      base_s[e] = run;
      run += min(hist_s[e], cap);
    }
    base_s[n] = run;
  }
  __syncthreads();
  for (int e = tid; e <= n; e += blockDim.x) {
    offsets[e] = base_s[e];
    if (e < n) counts[e] = min(hist_s[e], cap);
  }
  if (tid < cnt) {
    for (int j = 0; j < K; ++j) {
      const int e = sel_s[tid * K + j];
      const int rank = __popc(mask_s[e] & ((1u << tid) - 1u));  // earlier tokens of e
      int pos = -1;
      if (rank < cap) {
        pos = base_s[e] + rank;
        perm_token[pos] = (int)(t0 + tid);
      }
      slot_pos[(t0 + tid) * K + j] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
// W_g [d][n] -> WgT [NP][d], rows n..NP-1 zero.  64 (k) x 64 (e) tiles via LDS.
__global__ __launch_bounds__(256) void wg_transpose_kernel(const uint16_t* __restrict__ Wg, int d,
                                                           int n, int NP,
                                                           uint16_t* __restrict__ WgT) {
  __shared__ uint16_t tile[64][65];
  const int k0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int kk = idx / 64, ee = idx % 64;
    const int k = k0 + kk, e = e0 + ee;
    tile[kk][ee] = (k < d && e < n) ? Wg[(int64_t)k * n + e] : (uint16_t)0;
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int ee = idx / 64, kk = idx % 64;
    const int k = k0 + kk, e = e0 + ee;
    if (k < d && e < NP) WgT[(int64_t)e * d + k] = tile[kk][ee];
  }
}

// ---------------------------------------------------------------------------
// bf16 router.  NE expert tiles of 16, TT token tiles of 16 (BT = 16*TT), W
// waves splitting the reduction over d in steps of 32.  Lane (r = l%16,
// g = l/16) supplies A = x[token r][k + 8g ..] and B = WgT[expert r][k + 8g ..].
// DIRECT (n <= 16): B is gathered from W_g [d][n] itself
// (8 two-byte loads per fragment), so no transposed copy has to be made first.
template <int NE, int TT, int W, bool DIRECT = false>
__global__ __launch_bounds__(W * 64) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ WgT, int64_t T, int d, int n, int K,
    int* __restrict__ topk_idx, float* __restrict__ topk_w, int* __restrict__ hist, int fused,
    int* __restrict__ counts, int* __restrict__ offsets, int* __restrict__ perm_token,
    int* __restrict__ slot_pos, float* __restrict__ probsum, int cap, float* __restrict__ ec_probs,
    int* __restrict__ zero, int n_zero) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  constexpr int BT = 16 * TT;
  constexpr int NP = 16 * NE;
  constexpr int LDL = NP + 1;
  __shared__ float part_s[W * BT * NP];
  __shared__ float logits_s[BT * LDL];
  __shared__ int sel_s[32 * kMaxK];
  __shared__ uint32_t mask_s[kMaxN];
  __shared__ int hist_s[kMaxN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BT;

  const uint16_t* ap[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int64_t tok = t0 + tt * 16 + r;
    if (tok >= T) tok = T - 1;  // rows past the end are computed, never stored
    ap[tt] = x + tok * (int64_t)d + g * 8;
  }
  const uint16_t* bp[NE];
#pragma unroll
  for (int et = 0; et < NE; ++et) bp[et] = WgT + (int64_t)(et * 16 + r) * d + g * 8;
  // DIRECT: WgT is W_g [d][n]; lane r < n reads column r, rows k + 8g + i
  const bool b_col = !DIRECT || r < n;
  const uint16_t* bcol = WgT + (int64_t)(g * 8) * n + (b_col ? r : 0);
  auto load_b = [&](int et, int kc) -> bf16x8_t {
    if (!DIRECT) return *reinterpret_cast<const bf16x8_t*>(bp[et] + kc * 32);
    typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
    u16x8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = b_col ? bcol[(int64_t)(kc * 32 + i) * n] : (uint16_t)0;
    return *reinterpret_cast<bf16x8_t*>(&v);
  };

  f32x4_t acc[TT][NE];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < NE; ++et) acc[tt][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nkc = d / 32;
  const int kc0 = wave * nkc / W;
  const int kc1 = (wave + 1) * nkc / W;
  constexpr int U = 4;  // k-steps whose loads are issued together
  int kc = kc0;
  for (; kc + U <= kc1; kc += U) {
    bf16x8_t a[U][TT], b[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        a[u][tt] = *reinterpret_cast<const bf16x8_t*>(ap[tt] + (kc + u) * 32);
#pragma unroll
      for (int et = 0; et < NE; ++et) b[u][et] = load_b(et, kc + u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int et = 0; et < NE; ++et)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[tt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][tt], b[u][et], acc[tt][et], 0, 0, 0);
  }
  for (; kc < kc1; ++kc) {
#pragma unroll
    for (int et = 0; et < NE; ++et) {
      const bf16x8_t b = load_b(et, kc);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ap[tt] + kc * 32);
        acc[tt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[tt][et], 0, 0, 0);
      }
    }
  }
  // D layout of the 16x16 MFMA: lane holds rows (tokens) 4g + j, column (expert) r.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < NE; ++et)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part_s[(wave * BT + tt * 16 + 4 * g + j) * NP + et * 16 + r] = acc[tt][et][j];
  __syncthreads();
  for (int idx = tid; idx < BT * NP; idx += W * 64) {
    float s = part_s[idx];
#pragma unroll
    for (int w2 = 1; w2 < W; ++w2) s += part_s[w2 * BT * NP + idx];  // fixed wave order
    logits_s[(idx / NP) * LDL + (idx % NP)] = s;
  }
  __syncthreads();
  route_epilogue(logits_s, LDL, BT, t0, T, n, K, topk_idx, topk_w, hist, fused != 0, counts, offsets,
                 perm_token, slot_pos, sel_s, mask_s, hist_s, probsum, cap, ec_probs);
}

// ---------------------------------------------------------------------------
// bf16 router for many tokens and n % 16 == 0 experts.  Each wave owns one
// routing block of 16*TT tokens and the whole reduction over d, so its logits
// stay in registers; the workgroup's 4 waves share W_g, streamed through LDS in
// chunks of KC rows in its own [d][n] layout (a contiguous copy) and read as
// MFMA B fragments with transposing LDS reads (ds_read_b64_tr_b16: when lane
// q + 4j of a 16-lane group points at W[k + j][e0 + 4q ..], lane i of the
// group receives W[k .. k+3][e0 + i]).  x rows are read once, straight into
// registers, DA chunks ahead.  Top-K runs across the 16 lanes that hold a
// token's logits: K rounds of a butterfly arg-max (larger score, then lower
// expert index; NaN as -inf), the winner's lane retiring it; the softmax over
// the kept scores is the same expression as topk_softmax.
template <int NE, int TT>
__global__ __launch_bounds__(256) void router_wave_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ Wg, int64_t T, int d,
                                                          int K, int* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w, int* __restrict__ hist,
                                                          float* __restrict__ probsum, int* __restrict__ zero,
                                                          int n_zero) {
  constexpr int n = 16 * NE;
  constexpr int BTW = 16 * TT;              // tokens per wave (one routing block)
  constexpr int KC = n <= 64 ? 64 : 32;     // W_g rows per LDS chunk
  constexpr int NBUF = 3;                   // LDS chunk buffers
  constexpr int RS = n * 2 + 16;            // LDS row stride (bytes): padded against bank conflicts
  constexpr int CH = KC * n * 2;            // bytes per chunk in W_g
  constexpr int PIECES = CH / (16 * 256);   // 16-byte pieces per thread per chunk
  static_assert(PIECES >= 1 && CH % (16 * 256) == 0, "chunk copy");
  constexpr int DA = 4;                     // chunks of x and of W_g in flight
  static_assert(DA % 2 == 0, "fragment buffers alternate by k-step");
  constexpr int KS = KC / 32;               // MFMA k-steps per chunk
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  __shared__ __attribute__((aligned(16))) char wg_s[NBUF][KC * RS];
  __shared__ int hist_s[4][n];

  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t nb = (T + BTW - 1) / BTW;
  const int64_t blk = (int64_t)blockIdx.x * 4 + wave;
  const int64_t t0 = blk * BTW;

  const uint16_t* ap[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int64_t tok = t0 + tt * 16 + r;
    if (tok >= T) tok = T - 1;  // rows past the end are computed, never stored
    ap[tt] = x + tok * (int64_t)d + g * 8;
  }
  const int nch = d / KC;
  // Loads past the last chunk re-read it (never used), so every iteration issues the
  // same loads.  Each iteration issues W_g before x: the wait for a W_g chunk then
  // covers only x chunks that are already needed (a wave's loads complete in order).
  const u32x4_t* wsrc = reinterpret_cast<const u32x4_t*>(Wg);
  u32x4_t rb[DA][PIECES];
  auto load_b = [&](int c, u32x4_t (&dst)[PIECES]) {
    const int64_t cc = min(c, nch - 1);
#pragma unroll
    for (int i = 0; i < PIECES; ++i) dst[i] = wsrc[cc * (CH / 16) + i * 256 + tid];
  };
  auto store_b = [&](int c, const u32x4_t (&src)[PIECES]) {
    char* dst = wg_s[c % NBUF];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int byte = (i * 256 + tid) * 16;  // of the chunk in W_g's layout
      *reinterpret_cast<u32x4_t*>(dst + (byte / (n * 2)) * RS + byte % (n * 2)) = src[i];
    }
  };
  bf16x8_t ra[DA][TT][KS];
  auto load_a = [&](int c, bf16x8_t (&dst)[TT][KS]) {
    const int cc = min(c, nch - 1);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        dst[tt][ks] = *reinterpret_cast<const bf16x8_t*>(ap[tt] + cc * KC + ks * 32);
  };
  // B fragments of experts 16 et .. +15 at k-step ks of a chunk: two transposing reads each
  const int lq = r & 3, lj = r >> 2;
  bf16x8_t fb[2][NE];
  auto read_b = [&](int c, int ks, bf16x8_t (&dst)[NE]) {
    const char* row = wg_s[c % NBUF] + (ks * 32 + 8 * g + lj) * RS + 8 * lq;
#pragma unroll
    for (int et = 0; et < NE; ++et) {
      const char* p0 = row + et * 32;
      const i16x4_t both[2] = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0)),
                               __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * RS))};
      dst[et] = *reinterpret_cast<const bf16x8_t*>(both);
    }
  };

  f32x4_t acc[TT][NE];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < NE; ++et) acc[tt][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < DA; ++c) {
    load_b(c, rb[c]);
    load_a(c, ra[c]);
  }
  store_b(0, rb[0]);
  __syncthreads();
  read_b(0, 0, fb[0]);
  // Iteration c: chunk c+1 goes to LDS and is published by the barrier, so the
  // fragments of the next k-step can always be read while the MFMAs of the
  // current one run (the buffer written in iteration c last held chunk c-2,
  // whose reads every wave finished before the barrier of iteration c-1).
  // nch is a multiple of DA: every iteration issues the same loads, so the
  // compiler's own waits stay exact around the loop.
  for (int c0 = 0; c0 < nch; c0 += DA) {
#pragma unroll
    for (int u = 0; u < DA; ++u) {
      const int c = c0 + u;
      store_b(c + 1, rb[(u + 1) % DA]);  // chunk c+1 (past the end: a copy of the last, unread)
      __syncthreads();
      load_b(c + DA, rb[u]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = (u * KS + ks) & 1;  // k-steps alternate fragment buffers (DA is even)
        // next k-step's fragments (the first of chunk c+1 after the last of chunk c)
        if (ks + 1 < KS)
          read_b(c, ks + 1, fb[cur ^ 1]);
        else
          read_b(c + 1, 0, fb[cur ^ 1]);
#pragma unroll
        for (int et = 0; et < NE; ++et)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            acc[tt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[u][tt][ks], fb[cur][et], acc[tt][et], 0, 0, 0);
      }
      load_a(c + DA, ra[u]);
    }
  }

  // top-K per token; lane (r, g) holds experts 16 et + r of tokens 4 g + j of each token tile
  for (int e = lane; e < n; e += 64) hist_s[wave][e] = 0;
  float psum[NE];  // router statistics: this lane's sum of its experts' probabilities
#pragma unroll
  for (int et = 0; et < NE; ++et) psum[et] = 0.0f;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + tt * 16 + 4 * g + j;
      uint32_t taken = 0;
      float sv[kMaxK];
      int si[kMaxK];
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        sv[k] = -INFINITY;
        si[k] = 0;
        if (k < K) {
          float bv = -INFINITY;
          int bi = INT32_MAX;
#pragma unroll
          for (int et = 0; et < NE; ++et) {
            float v = acc[tt][et][j];
            if (v != v) v = -INFINITY;
            const int idx = et * 16 + r;
            if (!((taken >> et) & 1u) && (v > bv || (v == bv && idx < bi))) {
              bv = v;
              bi = idx;
            }
          }
#pragma unroll
          for (int mk = 1; mk < 16; mk <<= 1) {
            const float ov = __shfl_xor(bv, mk, 16);
            const int oi = __shfl_xor(bi, mk, 16);
            if (ov > bv || (ov == bv && oi < bi)) {
              bv = ov;
              bi = oi;
            }
          }
          if ((bi & 15) == r) taken |= 1u << (bi >> 4);
          sv[k] = bv;
          si[k] = bi;
        }
      }
      // the softmax over the kept scores, term by term as topk_softmax
      float w[kMaxK];
      float sum = 0.0f;
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < K) {
          w[k] = expf(sv[k] - sv[0]);
          sum += w[k];
        }
      if (t < T) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
          if (k < K && r == k) {
            topk_idx[t * K + k] = si[k];
            topk_w[t * K + k] = w[k] / sum;
            atomicAdd(&hist_s[wave][si[k]], 1);
          }
      }
      if (probsum != nullptr && t < T) {
        // the token's full n-way softmax: max (NaN ignored) and sum of exponentials over its 16 lanes
        float mx = -INFINITY;
#pragma unroll
        for (int et = 0; et < NE; ++et) mx = fmaxf(mx, acc[tt][et][j]);
#pragma unroll
        for (int mk = 1; mk < 16; mk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, mk, 16));
        float ex[NE], sm = 0.0f;
#pragma unroll
        for (int et = 0; et < NE; ++et) {
          ex[et] = expf(acc[tt][et][j] - mx);
          sm += ex[et];
        }
#pragma unroll
        for (int mk = 1; mk < 16; mk <<= 1) sm += __shfl_xor(sm, mk, 16);
#pragma unroll
        for (int et = 0; et < NE; ++et) psum[et] += ex[et] / sm;
      }
    }
  if (blk < nb)
    for (int e = lane; e < n; e += 64) hist[blk * n + e] = hist_s[wave][e];
  if (probsum != nullptr) {
    // the routing block's sum over its tokens: the lanes of the four token groups, then written by group 0
#pragma unroll
    for (int et = 0; et < NE; ++et) {
      float v = psum[et];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (blk < nb && g == 0) probsum[blk * n + et * 16 + r] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// One routing block (T <= 32 tokens) and n <= 16 experts: the decode case.  A
// single workgroup would pull all of x through one compute unit, so the d
// reduction is split over `nsplit` workgroups first: workgroup b sums its k
// range (its 4 waves a quarter each, W_g's columns gathered in place) and
// stores the block's [32][16] partial logits; one workgroup then adds the
// partials in b order and runs top-K, softmax and the whole dispatch.
constexpr int kDecodeSplitK = 256;  // k per workgroup of the split

__global__ __launch_bounds__(256) void router_split_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ Wg, int64_t T, int d,
                                                           int n, float* __restrict__ part,
                                                           int* __restrict__ zero, int n_zero) {
  __shared__ float wp_s[4][32 * 16];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  constexpr int KW = kDecodeSplitK / 4;  // k per wave: 2 MFMA k-steps
  const int k0 = blockIdx.x * kDecodeSplitK + wave * KW;
  const bool b_col = r < n;
  bf16x8_t a[2][KW / 32], b[KW / 32];
#pragma unroll
  for (int ks = 0; ks < KW / 32; ++ks) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t tok = min<int64_t>(tt * 16 + r, T - 1);  // rows past T are computed, never used
      a[tt][ks] = *reinterpret_cast<const bf16x8_t*>(x + tok * d + k0 + ks * 32 + g * 8);
    }
    typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
    u16x8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = b_col ? Wg[(int64_t)(k0 + ks * 32 + g * 8 + i) * n + r] : (uint16_t)0;
    b[ks] = *reinterpret_cast<bf16x8_t*>(&v);
  }
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < KW / 32; ++ks)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt][ks], b[ks], acc[tt], 0, 0, 0);
  // D layout: lane (r, g) holds tokens 16 tt + 4 g + j, expert r
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) wp_s[wave][(tt * 16 + 4 * g + j) * 16 + r] = acc[tt][j];
  __syncthreads();
  for (int i = tid; i < 32 * 16; i += 256) {
    float s = wp_s[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) s += wp_s[w][i];  // fixed wave order
    part[(int64_t)blockIdx.x * 32 * 16 + i] = s;
  }
}

__global__ __launch_bounds__(256) void router_finish_kernel(const float* __restrict__ part, int nsplit, int64_t T,
                                                            int n, int K, int* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w, int* __restrict__ counts,
                                                            int* __restrict__ offsets, int* __restrict__ perm_token,
                                                            int* __restrict__ slot_pos, int cap) {
  constexpr int LDL = 17;
  __shared__ float logits_s[32 * LDL];
  __shared__ int sel_s[32 * kMaxK];
  __shared__ uint32_t mask_s[kMaxN];
  __shared__ int hist_s[kMaxN];
  for (int i = threadIdx.x; i < 32 * 16; i += 256) {
    // in split order; each run of 16 partials is loaded at once (a chain of
    // dependent-looking loads would wait for each in turn)
    float s = 0.0f;
    for (int b0 = 0; b0 < nsplit; b0 += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = b0 + j < nsplit ? part[(int64_t)(b0 + j) * 32 * 16 + i] : 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (b0 + j < nsplit) s += v[j];
    }
    logits_s[(i / 16) * LDL + i % 16] = s;
  }
  __syncthreads();
  route_epilogue(logits_s, LDL, 32, 0, T, n, K, topk_idx, topk_w, nullptr, true, counts, offsets, perm_token,
                 slot_pos, sel_s, mask_s, hist_s, nullptr, cap, nullptr);
}

// ---------------------------------------------------------------------------
// fp32 router: one dot product per (token, expert), sequential in j.
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ Wg, int64_t T,
                                                         int64_t d, int n, int K, int BT,
                                                         int* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int* __restrict__ hist,
                                                         float* __restrict__ probsum) {
  __shared__ float logits_s[32 * (kMaxN + 1)];
  __shared__ int sel_s[32 * kMaxK];
  __shared__ uint32_t mask_s[kMaxN];
  __shared__ int hist_s[kMaxN];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int ld = n + 1;
  for (int idx = tid; idx < BT * n; idx += 256) {
    const int i = idx / n;
    const int e = idx % n;
    int64_t tok = t0 + i;
    if (tok >= T) tok = T - 1;
    const float* xr = x + tok * d;
    float s = 0.0f;
    for (int64_t j = 0; j < d; ++j) s = fmaf(xr[j], Wg[j * n + e], s);
    logits_s[i * ld + e] = s;
  }
  __syncthreads();
  route_epilogue(logits_s, ld, BT, t0, T, n, K, topk_idx, topk_w, hist, false, nullptr, nullptr,
                 nullptr, nullptr, sel_s, mask_s, hist_s, probsum, INT32_MAX, nullptr);
}

// ---------------------------------------------------------------------------
// Scan over the block histograms hist[nb][n] (one workgroup of 1024 threads).
// Thread (e, p) owns a contiguous range of blocks for expert e.  Each expert
// keeps at most `cap` assignments (INT32_MAX: all).  Writes counts[e] =
// min(total_e, cap), offsets = their exclusive scan, and bases[b][e] =
// offsets[e] + sum_{b' < b} hist[b'][e] (an assignment whose position minus
// offsets[e] reaches cap is dropped by the scatter).
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ hist, int nb, int n, int cap,
                                                    int* __restrict__ bases,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offsets) {
  __shared__ int psum[1024];
  __shared__ int tot_s[kMaxN];
  __shared__ int off_s[kMaxN + 1];
  const int tid = threadIdx.x;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  const int P = 1024 / np2;  // threads per expert
  const int e = tid % np2;
  const int p = tid / np2;
  const int b0 = (int)((int64_t)p * nb / P);
  const int b1 = (int)((int64_t)(p + 1) * nb / P);
  int s = 0;
  if (e < n)
    for (int b = b0; b < b1; ++b) s += hist[(int64_t)b * n + e];
  psum[tid] = s;
  __syncthreads();
  if (tid < n) {
    int run = 0;
    for (int q = 0; q < P; ++q) {
      const int v = psum[q * np2 + tid];
      psum[q * np2 + tid] = run;  // exclusive prefix over the chunks of expert tid
      run += v;
    }
    tot_s[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < n; ++i) {
      off_s[i] = run;
      run += min(tot_s[i], cap);
    }
    off_s[n] = run;
  }
  __syncthreads();
  for (int i = tid; i <= n; i += 1024) {
    offsets[i] = off_s[i];
    if (i < n) counts[i] = min(tot_s[i], cap);
  }
  if (e < n) {
    int run = off_s[e] + psum[tid];
    for (int b = b0; b < b1; ++b) {
      bases[(int64_t)b * n + e] = run;
      run += hist[(int64_t)b * n + e];
    }
  }
}

// The same scan when n % 4 == 0, four experts per thread with 16-byte loads:
// thread (quad q, part p) holds its part's histogram rows in registers (at
// most kScanRows per pass; longer parts take more passes), so every load of a
// pass is in flight at once.  The parts' sums are scanned across the
// workgroup in LDS (Hillis-Steele over p), the experts' offsets by one thread.
constexpr int kScanRows = 16;

__global__ __launch_bounds__(1024) void scan4_kernel(const int* __restrict__ hist, int nb, int n, int cap,
                                                     int* __restrict__ bases, int* __restrict__ counts,
                                                     int* __restrict__ offsets) {
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  __shared__ i32x4_t part_s[2][1024];
  __shared__ int tot_s[kMaxN];
  __shared__ int off_s[kMaxN + 1];
  const int tid = threadIdx.x;
  const int nq = n / 4;
  const int P = 1024 / nq;  // parts (n <= 256: at least 16)
  const int q = tid % nq;
  const int p = tid / nq;
  const bool active = p < P;
  const int b0 = active ? (int)((int64_t)p * nb / P) : 0;
  const int b1 = active ? (int)((int64_t)(p + 1) * nb / P) : 0;
  const i32x4_t* h4 = reinterpret_cast<const i32x4_t*>(hist);
  i32x4_t s = {0, 0, 0, 0};
  for (int c0 = b0; c0 < b1; c0 += kScanRows) {
    i32x4_t v[kScanRows];
#pragma unroll
    for (int j = 0; j < kScanRows; ++j)
      if (c0 + j < b1) v[j] = h4[(int64_t)(c0 + j) * nq + q];
#pragma unroll
    for (int j = 0; j < kScanRows; ++j)
      if (c0 + j < b1) s += v[j];
  }
  // inclusive scan of the parts' sums over p (same q), ping-pong buffers
  int cur = 0;
  part_s[0][tid] = s;
  __syncthreads();
  for (int d = 1; d < P; d <<= 1) {
    i32x4_t t = part_s[cur][tid];
    if (active && p >= d) t += part_s[cur][tid - d * nq];
    part_s[cur ^ 1][tid] = t;
    cur ^= 1;
    __syncthreads();
  }
  if (tid < nq) {
    const i32x4_t t = part_s[cur][(P - 1) * nq + tid];
    tot_s[4 * tid] = t[0];
    tot_s[4 * tid + 1] = t[1];
    tot_s[4 * tid + 2] = t[2];
    tot_s[4 * tid + 3] = t[3];
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < n; ++i) {
      off_s[i] = run;
      run += min(tot_s[i], cap);
    }
    off_s[n] = run;
  }
  __syncthreads();
  for (int i = tid; i <= n; i += 1024) {
    offsets[i] = off_s[i];
    if (i < n) counts[i] = min(tot_s[i], cap);
  }
  if (!active) return;
  // bases of the part's rows: offsets plus everything before (exclusive over parts, then rows)
  i32x4_t run = i32x4_t{off_s[4 * q], off_s[4 * q + 1], off_s[4 * q + 2], off_s[4 * q + 3]} + part_s[cur][tid] - s;
  i32x4_t* bases4 = reinterpret_cast<i32x4_t*>(bases);
  for (int c0 = b0; c0 < b1; c0 += kScanRows) {
    i32x4_t v[kScanRows];
#pragma unroll
    for (int j = 0; j < kScanRows; ++j)
      if (c0 + j < b1) v[j] = h4[(int64_t)(c0 + j) * nq + q];
#pragma unroll
    for (int j = 0; j < kScanRows; ++j)
      if (c0 + j < b1) {
        bases4[(int64_t)(c0 + j) * nq + q] = run;
        run += v[j];
      }
  }
}

// Scatter of one routing block (BT <= 32 tokens): positions are
// expert-contiguous and ascending in token index within an expert.
__global__ __launch_bounds__(64) void scatter_kernel(const int* __restrict__ topk_idx,
                                                     const int* __restrict__ bases,
                                                     const int* __restrict__ offsets, int cap, int64_t T,
                                                     int n, int K, int BT, int* __restrict__ perm_token,
                                                     int* __restrict__ slot_pos) {
  __shared__ uint32_t mask_s[kMaxN];
  __shared__ int sel_s[32 * kMaxK];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int cnt = (int)((T - t0) < BT ? (T - t0) : BT);
  for (int e = tid; e < n; e += 64) mask_s[e] = 0u;
  __syncthreads();
  if (tid < cnt) {
    for (int j = 0; j < K; ++j) {
      const int e = min(max(topk_idx[(t0 + tid) * K + j], 0), n - 1);
      sel_s[tid * K + j] = e;
      atomicOr(&mask_s[e], 1u << tid);
    }
  }
  __syncthreads();
  if (tid < cnt) {
    for (int j = 0; j < K; ++j) {
      const int e = sel_s[tid * K + j];
      int pos = bases[(int64_t)blockIdx.x * n + e] + __popc(mask_s[e] & ((1u << tid) - 1u));
      if (pos - offsets[e] < cap)
        perm_token[pos] = (int)(t0 + tid);
      else
        pos = -1;  // the expert is full: this assignment is dropped
      slot_pos[(t0 + tid) * K + j] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
namespace {

template <int NE, int TT, int W, bool DIRECT = false>
void launch_router_t(const uint16_t* x, const uint16_t* WgT, int64_t T, int64_t d, int n, int K,
                     const RouteBuffers& rb, bool fused, float* probsum, int cap, float* ec_probs,
                     hipStream_t s) {
  constexpr int BT = 16 * TT;
  const int64_t nb = (T + BT - 1) / BT;
  hipLaunchKernelGGL((router_bf16_kernel<NE, TT, W, DIRECT>), dim3((unsigned)nb), dim3(W * 64), 0, s, x, WgT,
                     T, (int)d, n, K, rb.topk_idx, rb.topk_w, rb.hist, fused ? 1 : 0, rb.counts,
                     rb.offsets, rb.perm_token, rb.slot_pos, probsum, cap, ec_probs, rb.zero, rb.n_zero);
}

// Router statistics from the per-block histograms and probability sums
// (summed in double):
//   frac[e] = counts[e] / (T*K), prob[e] = sum_t p_t[e] / T,
//   aux_loss = alpha * n * sum_e frac[e] * prob[e]   (summed in expert order).
// One workgroup of 1024 threads.  Thread (part p, expert e), e fastest, sums
// the routing blocks [p*nb/P, (p+1)*nb/P) of expert e in block order
// (consecutive threads read consecutive experts of a block), and the parts
// are then added in part order, so the result is deterministic.  P gives each
// part about 8 blocks, within the 1024/n parts the workgroup holds.
constexpr int kStatsThreads = 1024;
__global__ __launch_bounds__(kStatsThreads) void route_stats_kernel(const int* __restrict__ hist,
                                                                    const float* __restrict__ probsum, int nb,
                                                                    int64_t T, int n, int K, float alpha,
                                                                    float* __restrict__ frac,
                                                                    float* __restrict__ prob,
                                                                    float* __restrict__ aux_loss) {
  __shared__ long long cnt_s[kStatsThreads];
  __shared__ double p_s[kStatsThreads];
  __shared__ double fp_s[kMaxN];
  const int tid = threadIdx.x;
  const int P = max(1, min(kStatsThreads / n, nb / 8));  // n <= kMaxN = 256
  const int e = tid % n;
  const int part = tid / n;
  if (part < P) {
    const int b0 = (int)((int64_t)part * nb / P);
    const int b1 = (int)((int64_t)(part + 1) * nb / P);
    long long c = 0;
    double p = 0.0;
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      c += hist[(int64_t)b * n + e];
      p += (double)probsum[(int64_t)b * n + e];
    }
    cnt_s[tid] = c;
    p_s[tid] = p;
  }
  __syncthreads();
  if (tid < n) {
    long long c = 0;
    double p = 0.0;
    for (int q = 0; q < P; ++q) {
      c += cnt_s[q * n + tid];
      p += p_s[q * n + tid];
    }
    const double fe = (double)c / ((double)T * K);
    const double pe = p / (double)T;
    if (frac != nullptr) frac[tid] = (float)fe;
    if (prob != nullptr) prob[tid] = (float)pe;
    fp_s[tid] = fe * pe;
  }
  __syncthreads();
  if (tid == 0 && aux_loss != nullptr) {
    double acc = 0.0;
    for (int q = 0; q < n; ++q) acc += fp_s[q];
    aux_loss[0] = (float)((double)alpha * n * acc);
  }
}

// Picks the router configuration for the expert count (WgT rows padded to 16).
void launch_router_bf16(const uint16_t* x, int64_t T, int64_t d, int n, int K, const RouteBuffers& rb,
                        bool fused, float* probsum, int cap, hipStream_t s, float* ec_probs = nullptr) {
  const int ne = route_padded_experts(n) / 16;
  if (ne <= 1)
    launch_router_t<1, 2, 16>(x, rb.wgT, T, d, n, K, rb, fused, probsum, cap, ec_probs, s);
  else if (ne <= 2)
    launch_router_t<2, 2, 8>(x, rb.wgT, T, d, n, K, rb, fused, probsum, cap, ec_probs, s);
  else if (ne <= 4)
    launch_router_t<4, 2, 8>(x, rb.wgT, T, d, n, K, rb, fused, probsum, cap, ec_probs, s);
  else if (ne <= 8)
    launch_router_t<8, 1, 8>(x, rb.wgT, T, d, n, K, rb, fused, probsum, cap, ec_probs, s);
  else
    launch_router_t<16, 1, 4>(x, rb.wgT, T, d, n, K, rb, fused, probsum, cap, ec_probs, s);
}

// Expert-choice selection: workgroup e finds the C-th largest score of column
// e of probs [T][n] by a 4-pass 8-bit radix select on the float bit patterns
// (scores are >= 0, so their bits order like their values), then keeps every
// token above that threshold and the earliest tokens equal to it.  Rows go to
// e*C + j in ascending token order; slot_pos was set to -1 by the router, so
// only the chosen slots are written.  The column is staged in LDS when it fits.
// Scores cluster near 1/n, so most keys share their upper digits: each wave
// keeps its own histogram and adds a run of equal digits with one atomic.
// The compaction gives each wave a contiguous token range and ranks within it
// by ballot, so LDS reads are consecutive and the order is the token order.
constexpr int kEcLdsKeys = 32768;  // 128 KiB of keys
constexpr int kEcWaves = 16;
__global__ __launch_bounds__(kEcWaves * 64) void expert_choice_kernel(const float* __restrict__ probs, int64_t T,
                                                                      int n, int C, int* __restrict__ perm_token,
                                                                      int* __restrict__ slot_pos,
                                                                      int* __restrict__ counts,
                                                                      int* __restrict__ offsets) {
  __shared__ uint32_t keys_s[kEcLdsKeys];
  __shared__ int hist_s[kEcWaves][256];
  __shared__ int suffix[256];
  __shared__ uint32_t prefix_s;
  __shared__ int need_s;
  __shared__ int wcnt_s[kEcWaves][2];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1;  // lanes before this one
  const float* col = probs + e;
  const bool staged = T <= kEcLdsKeys;
  if (staged)
    for (int64_t t = tid; t < T; t += kEcWaves * 64) keys_s[t] = __float_as_uint(col[t * n]);
  auto key = [&](int64_t t) -> uint32_t { return staged ? keys_s[t] : __float_as_uint(col[t * n]); };
  if (tid == 0) {
    prefix_s = 0u;
    need_s = C;
    counts[e] = C;
    offsets[e] = e * C;
    if (e == n - 1) offsets[n] = n * C;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t himask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < kEcWaves * 256; i += kEcWaves * 64) (&hist_s[0][0])[i] = 0;
    __syncthreads();
    const uint32_t prefix = prefix_s;
    const int need = need_s;
    for (int64_t t = tid; t < T; t += kEcWaves * 64) {
      const uint32_t k = key(t);
      const bool match = (k & himask) == prefix;
      const int dg = (int)((k >> shift) & 255u);
      const unsigned long long act = __ballot(match);
      if (act != 0ull) {
        const int lead = __ffsll((long long)act) - 1;
        const int dl = __shfl(dg, lead);
        const unsigned long long same = __ballot(match && dg == dl);
        if (lane == lead)
          atomicAdd(&hist_s[wave][dl], __popcll(same));
        else if (match && dg != dl)
          atomicAdd(&hist_s[wave][dg], 1);
      }
    }
    __syncthreads();
    // suffix[dg] = number of candidates with digit >= dg (inclusive scan from the top)
    if (tid < 256) {
      int h = 0;
#pragma unroll
      for (int w = 0; w < kEcWaves; ++w) h += hist_s[w][tid];
      suffix[tid] = h;
    }
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = (tid < 256 && tid + off < 256) ? suffix[tid + off] : 0;
      __syncthreads();
      if (tid < 256) suffix[tid] += v;
      __syncthreads();
    }
    // the selected digit: its suffix reaches `need`, the next one's does not
    if (tid < 256) {
      const int above = tid < 255 ? suffix[tid + 1] : 0;
      if (suffix[tid] >= need && above < need) {
        need_s = need - above;
        prefix_s = prefix | ((uint32_t)tid << shift);
      }
    }
    __syncthreads();
  }
  const uint32_t thr = prefix_s;  // the C-th largest key
  const int need = need_s;        // tokens equal to it that are taken (earliest first)
  // wave w ranks tokens [w*span, (w+1)*span), span a multiple of 64
  const int64_t span = ((T + kEcWaves - 1) / kEcWaves + 63) / 64 * 64;
  const int64_t wb0 = min<int64_t>(T, wave * span);
  const int64_t wb1 = min<int64_t>(T, wb0 + span);
  int n_gt = 0, n_eq = 0;
  for (int64_t t0 = wb0; t0 < wb1; t0 += 64) {
    const int64_t t = t0 + lane;
    const bool in = t < wb1;
    const uint32_t k = in ? key(t) : 0u;
    n_gt += __popcll(__ballot(in && k > thr));
    n_eq += __popcll(__ballot(in && k == thr));
  }
  if (lane == 0) {
    wcnt_s[wave][0] = n_gt;
    wcnt_s[wave][1] = n_eq;
  }
  __syncthreads();
  // tokens equal to the threshold and tokens chosen in the ranges before this wave's
  int eq_seen = 0, pos = e * C;
  for (int w = 0; w < wave; ++w) {
    const int gt_w = wcnt_s[w][0];
    const int eq_w = wcnt_s[w][1];
    pos += gt_w + min(max(need - eq_seen, 0), eq_w);
    eq_seen += eq_w;
  }
  for (int64_t t0 = wb0; t0 < wb1; t0 += 64) {
    const int64_t t = t0 + lane;
    const bool in = t < wb1;
    const uint32_t k = in ? key(t) : 0u;
    const bool eq = in && k == thr;
    const unsigned long long eqm = __ballot(eq);
    const bool sel = in && (k > thr || (eq && eq_seen + __popcll(eqm & below) < need));
    const unsigned long long selm = __ballot(sel);
    if (sel) {
      const int p = pos + __popcll(selm & below);
      perm_token[p] = (int)t;
      slot_pos[t * n + e] = p;
    }
    eq_seen += __popcll(eqm);
    pos += __popcll(selm);
  }
}

}  // namespace

int route_block_tokens(int n) { return n <= 64 ? 32 : 16; }

// Many tokens (more than one routing block) and n in {32, 64, 128, 256}: the
// wave-per-routing-block router.  Routing and router statistics take the same
// kernel, so both see the same selection.
bool use_wave_router(int64_t T, int64_t d, int n) {
  return T > route_block_tokens(n) && (n == 32 || n == 64 || n == 128 || n == 256) && d % 256 == 0;
}

void launch_router_wave(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n, int K,
                        const RouteBuffers& rb, float* probsum, hipStream_t s) {
  const int64_t nb = (T + route_block_tokens(n) - 1) / route_block_tokens(n);
  const dim3 grid((unsigned)((nb + 3) / 4)), block(256);
  if (n == 32)
    hipLaunchKernelGGL((router_wave_kernel<2, 2>), grid, block, 0, s, x, Wg, T, (int)d, K, rb.topk_idx, rb.topk_w,
                       rb.hist, probsum, rb.zero, rb.n_zero);
  else if (n == 64)
    hipLaunchKernelGGL((router_wave_kernel<4, 2>), grid, block, 0, s, x, Wg, T, (int)d, K, rb.topk_idx, rb.topk_w,
                       rb.hist, probsum, rb.zero, rb.n_zero);
  else if (n == 128)
    hipLaunchKernelGGL((router_wave_kernel<8, 1>), grid, block, 0, s, x, Wg, T, (int)d, K, rb.topk_idx, rb.topk_w,
                       rb.hist, probsum, rb.zero, rb.n_zero);
  else
    hipLaunchKernelGGL((router_wave_kernel<16, 1>), grid, block, 0, s, x, Wg, T, (int)d, K, rb.topk_idx, rb.topk_w,
                       rb.hist, probsum, rb.zero, rb.n_zero);
}

int route_padded_experts(int n) { return (n + 15) / 16 * 16; }

hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                             int K, const RouteBuffers& rb, hipStream_t s, hipEvent_t after_router,
                             int cap) {
  const int BT = route_block_tokens(n);
  const int64_t nb = (T + BT - 1) / BT;
  const bool fused = nb == 1;
  hipError_t e;
  if (n <= 16 && fused && route_block_tokens(n) == 32 && d % kDecodeSplitK == 0 && rb.split != nullptr) {
    // one routing block: the reduction over d split over workgroups, then one
    // workgroup for top-K and the dispatch
    const int nsplit = (int)(d / kDecodeSplitK);
    hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)nsplit), dim3(256), 0, s, x, Wg, T, (int)d, n, rb.split,
                       rb.zero, rb.n_zero);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(router_finish_kernel, dim3(1), dim3(256), 0, s, rb.split, nsplit, T, n, K, rb.topk_idx,
                       rb.topk_w, rb.counts, rb.offsets, rb.perm_token, rb.slot_pos, cap);
  } else if (n <= 16) {
    // up to 16 experts: gather W_g's columns in place instead of launching a
    // transposed copy first (7 us at the Mixtral shape); the whole dispatch
    // runs in the router when one routing block covers T
    launch_router_t<1, 2, 16, true>(x, Wg, T, d, n, K, rb, fused, nullptr, cap, nullptr, s);
  } else if (use_wave_router(T, d, n)) {
    launch_router_wave(x, Wg, T, d, n, K, rb, nullptr, s);
  } else {
    const int NP = route_padded_experts(n);
    hipLaunchKernelGGL(wg_transpose_kernel, dim3((unsigned)((d + 63) / 64), (unsigned)((NP + 63) / 64)),
                       dim3(256), 0, s, Wg, (int)d, n, NP, rb.wgT);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_router_bf16(x, T, d, n, K, rb, fused, nullptr, cap, s);
  }
  e = hipGetLastError();
  if (e == hipSuccess && after_router != nullptr) e = hipEventRecord(after_router, s);
  if (e != hipSuccess || fused) return e;
  return launch_dispatch(T, n, K, rb, s, cap);
}

hipError_t launch_route_stats_bf16(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                                   int K, float alpha, const RouteBuffers& rb, float* probsum,
                                   float* frac, float* prob, float* aux_loss, hipStream_t s) {
  hipError_t e;
  if (use_wave_router(T, d, n)) {
    launch_router_wave(x, Wg, T, d, n, K, rb, probsum, s);
  } else {
    const int NP = route_padded_experts(n);
    hipLaunchKernelGGL(wg_transpose_kernel, dim3((unsigned)((d + 63) / 64), (unsigned)((NP + 63) / 64)),
                       dim3(256), 0, s, Wg, (int)d, n, NP, rb.wgT);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_router_bf16(x, T, d, n, K, rb, false, probsum, INT32_MAX, s);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int BT = route_block_tokens(n);
  const int nb = (int)((T + BT - 1) / BT);
  hipLaunchKernelGGL(route_stats_kernel, dim3(1), dim3(kStatsThreads), 0, s, rb.hist, probsum, nb, T, n, K, alpha,
                     frac, prob, aux_loss);
  return hipGetLastError();
}

hipError_t launch_route_expert_choice(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                                     int C, const RouteBuffers& rb, hipStream_t s) {
  const int NP = route_padded_experts(n);
  hipLaunchKernelGGL(wg_transpose_kernel, dim3((unsigned)((d + 63) / 64), (unsigned)((NP + 63) / 64)),
                     dim3(256), 0, s, Wg, (int)d, n, NP, rb.wgT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_router_bf16(x, T, d, n, 1, rb, false, nullptr, INT32_MAX, s, rb.topk_w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(expert_choice_kernel, dim3((unsigned)n), dim3(kEcWaves * 64), 0, s, rb.topk_w, T, n, C,
                     rb.perm_token, rb.slot_pos, rb.counts, rb.offsets);
  return hipGetLastError();
}

hipError_t launch_route_f32(const float* x, const float* Wg, int64_t T, int64_t d, int n, int K,
                            const RouteBuffers& rb, hipStream_t s) {
  const int BT = route_block_tokens(n);
  const int64_t nb = (T + BT - 1) / BT;
  hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)nb), dim3(256), 0, s, x, Wg, T, d, n, K, BT,
                     rb.topk_idx, rb.topk_w, rb.hist, (float*)nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dispatch(T, n, K, rb, s);
}

hipError_t launch_route_stats_f32(const float* x, const float* Wg, int64_t T, int64_t d, int n, int K,
                                  float alpha, const RouteBuffers& rb, float* probsum, float* frac,
                                  float* prob, float* aux_loss, hipStream_t s) {
  const int BT = route_block_tokens(n);
  const int64_t nb = (T + BT - 1) / BT;
  hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)nb), dim3(256), 0, s, x, Wg, T, d, n, K, BT,
                     rb.topk_idx, rb.topk_w, rb.hist, probsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_stats_kernel, dim3(1), dim3(kStatsThreads), 0, s, rb.hist, probsum, (int)nb, T, n, K,
                     alpha, frac, prob, aux_loss);
  return hipGetLastError();
}

hipError_t launch_dispatch(int64_t T, int n, int K, const RouteBuffers& rb, hipStream_t s, int cap) {
  const int BT = route_block_tokens(n);
  const int nb = (int)((T + BT - 1) / BT);
  if (n % 4 == 0)
    hipLaunchKernelGGL(scan4_kernel, dim3(1), dim3(1024), 0, s, rb.hist, nb, n, cap, rb.bases, rb.counts,
                       rb.offsets);
  else
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, rb.hist, nb, n, cap, rb.bases, rb.counts,
                       rb.offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nb), dim3(64), 0, s, rb.topk_idx, rb.bases, rb.offsets,
                     cap, T, n, K, BT, rb.perm_token, rb.slot_pos);
  return hipGetLastError();
}

}  // namespace moe
