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
// Kernels:
//   router_bf16_kernel  logits on bf16 MFMA (16x16x32), fp32 accumulation,
//                       then top-K + softmax + per-block expert histogram.
//   router_f32_kernel   same epilogue, fp32 FMA dot products.
//   scatter_kernel      per-block bases from the histograms, ranks within the
//                       block, writes counts/offsets/perm_token/slot_pos.
// Everything is integer or fixed-order fp32: results are bit-reproducible.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-K + softmax + histogram for the tokens of one block; logits_s[i*ld + e].
// Thread i handles token t0 + i.  Ties keep the lower expert index first
// (a later expert only displaces a strictly smaller score); an empty slot takes
// any score, so every slot ends up holding a valid expert even for NaN input.
__device__ void topk_softmax_epilogue(const float* logits_s, int ld, int BT, int64_t t0,
                                      int64_t T, int n, int K, int* __restrict__ topk_idx,
                                      float* __restrict__ topk_w, int* hist_s) {
  const int i = threadIdx.x;
  if (i >= BT || t0 + i >= T) return;
  float v[kMaxK];
  int id[kMaxK];
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
      if (j < K && (id[j] < 0 || cv > v[j])) {
        const float tv = v[j];
        const int ti = id[j];
        v[j] = cv;
        id[j] = ci;
        cv = tv;
        ci = ti;
      }
    }
  }
  float z[kMaxK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      z[j] = expf(v[j] - v[0]);
      sum += z[j];
    }
  }
  const int64_t t = t0 + i;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      topk_idx[t * K + j] = id[j];
      topk_w[t * K + j] = z[j] / sum;
      atomicAdd(&hist_s[id[j]], 1);  // integer: order-independent
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 router.  A workgroup (4 waves) owns BT = 64*TT tokens; wave w owns TT
// tiles of 16 tokens.  W_g is staged through LDS transposed to [expert][k] in
// chunks of 64 rows so MFMA B fragments are single 16-byte LDS reads.  The K
// index inside an MFMA step is permuted (lane group g covers k = g*16 + s*8 ..
// of the 64-chunk in step s) identically for both operands, which leaves the
// dot products unchanged and makes each lane read 32 contiguous bytes of x.
template <int NE, int TT>
__global__ __launch_bounds__(256) void router_bf16_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ Wg,
                                                          int64_t T, int d, int n, int K,
                                                          int* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          int* __restrict__ hist) {
  constexpr int BT = 64 * TT;
  constexpr int NP = NE * 16;
  constexpr int DK = 64;
  constexpr int LDW = DK + 8;  // padded row: consecutive experts shift by 16 B
  constexpr int LDL = NP + 1;
  __shared__ __attribute__((aligned(16))) uint16_t wgT[NP * LDW];
  __shared__ float logits_s[BT * LDL];
  __shared__ int hist_s[NP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BT;

  for (int e = tid; e < NP; e += 256) hist_s[e] = 0;

  const uint16_t* xrow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int64_t tok = t0 + wave * 16 * TT + tt * 16 + r;
    if (tok >= T) tok = T - 1;  // rows past the end are computed, never stored
    xrow[tt] = x + tok * (int64_t)d;
  }
  f32x4_t acc[TT][NE];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < NE; ++et) acc[tt][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool vec_ok = (n % 8) == 0;
  for (int k0 = 0; k0 < d; k0 += DK) {
    __syncthreads();  // previous chunk consumed
    constexpr int NC = NP / 8;
    for (int idx = tid; idx < DK * NC; idx += 256) {
      const int kk = idx / NC;
      const int e0 = (idx % NC) * 8;
      uint16_t v[8];
      const uint16_t* src = Wg + (int64_t)(k0 + kk) * n + e0;
      if (vec_ok && e0 < n) {
        const uint4 q = *reinterpret_cast<const uint4*>(src);
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = (uint16_t)(w4[j] & 0xFFFFu);
          v[2 * j + 1] = (uint16_t)(w4[j] >> 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (e0 + j < n) ? src[j] : (uint16_t)0;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) wgT[(e0 + j) * LDW + kk] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = g * 16 + s * 8;
      bf16x8_t a[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        a[tt] = *reinterpret_cast<const bf16x8_t*>(xrow[tt] + k0 + kk);
#pragma unroll
      for (int et = 0; et < NE; ++et) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&wgT[(et * 16 + r) * LDW + kk]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[tt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt], b, acc[tt][et], 0, 0, 0);
      }
    }
  }
  // D layout of 16x16 MFMA: lane holds rows 4*g + j, column r.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < NE; ++et)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tl = wave * 16 * TT + tt * 16 + 4 * g + j;
        logits_s[tl * LDL + et * 16 + r] = acc[tt][et][j];
      }
  __syncthreads();
  topk_softmax_epilogue(logits_s, LDL, BT, t0, T, n, K, topk_idx, topk_w, hist_s);
  __syncthreads();
  for (int e = tid; e < n; e += 256) hist[(int64_t)blockIdx.x * n + e] = hist_s[e];
}

// ---------------------------------------------------------------------------
// fp32 router: one dot product per (token, expert), sequential in j.
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ Wg, int64_t T,
                                                         int64_t d, int n, int K, int BT,
                                                         int* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int* __restrict__ hist) {
  __shared__ float logits_s[128 * 129];  // BT*(n+1) <= 128*129 for both block sizes
  __shared__ int hist_s[kMaxN];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int ld = n + 1;
  for (int e = tid; e < n; e += 256) hist_s[e] = 0;
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
  topk_softmax_epilogue(logits_s, ld, BT, t0, T, n, K, topk_idx, topk_w, hist_s);
  __syncthreads();
  for (int e = tid; e < n; e += 256) hist[(int64_t)blockIdx.x * n + e] = hist_s[e];
}

// ---------------------------------------------------------------------------
// Scatter: block b places its assignments.  The base of expert e for block b
// is offsets[e] + (assignments to e in blocks before b); the rank of token i's
// assignment to e inside the block counts earlier tokens of the block that
// also chose e.  Positions are therefore expert-contiguous and ascending in
// token index within an expert (a stable counting sort).
__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ topk_idx,
                                                      const int* __restrict__ hist, int64_t T,
                                                      int n, int K, int BT, int nb,
                                                      int* __restrict__ counts,
                                                      int* __restrict__ offsets,
                                                      int* __restrict__ perm_token,
                                                      int* __restrict__ slot_pos) {
  __shared__ int tot[kMaxN];
  __shared__ int pre[kMaxN];
  __shared__ int base[kMaxN + 1];
  __shared__ int sel_s[128 * kMaxK];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = tid; e < n; e += 256) {
    tot[e] = 0;
    pre[e] = 0;
  }
  __syncthreads();
  const int64_t nh = (int64_t)nb * n;
  for (int64_t idx = tid; idx < nh; idx += 256) {
    const int bb = (int)(idx / n);
    const int e = (int)(idx % n);
    const int h = hist[idx];
    atomicAdd(&tot[e], h);
    if (bb < b) atomicAdd(&pre[e], h);
  }
  const int64_t t0 = (int64_t)b * BT;
  const int cnt = (int)((T - t0) < BT ? (T - t0) : BT);
  for (int idx = tid; idx < cnt * K; idx += 256) sel_s[idx] = topk_idx[t0 * K + idx];
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < n; ++e) {
      base[e] = run;
      run += tot[e];
    }
    base[n] = run;
  }
  __syncthreads();
  if (b == 0) {
    for (int e = tid; e <= n; e += 256) {
      offsets[e] = base[e];
      if (e < n) counts[e] = tot[e];
    }
  }
  if (tid < cnt) {
    for (int k = 0; k < K; ++k) {
      const int e = sel_s[tid * K + k];
      int rank = 0;
      for (int i2 = 0; i2 < tid; ++i2)
        for (int k2 = 0; k2 < K; ++k2) rank += (sel_s[i2 * K + k2] == e) ? 1 : 0;
      const int pos = base[e] + pre[e] + rank;
      perm_token[pos] = (int)(t0 + tid);
      slot_pos[(t0 + tid) * K + k] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
template <int NE, int TT>
static void launch_router_bf16_t(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d,
                                 int n, int K, int* topk_idx, float* topk_w, int* hist,
                                 hipStream_t s) {
  const int BT = 64 * TT;
  const int64_t nb = (T + BT - 1) / BT;
  hipLaunchKernelGGL((router_bf16_kernel<NE, TT>), dim3((unsigned)nb), dim3(256), 0, s, x, Wg, T,
                     (int)d, n, K, topk_idx, topk_w, hist);
}

hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                              int K, int* topk_idx, float* topk_w, int* hist, hipStream_t s) {
  const int ne = (n + 15) / 16;
  if (ne <= 1)
    launch_router_bf16_t<1, 2>(x, Wg, T, d, n, K, topk_idx, topk_w, hist, s);
  else if (ne <= 2)
    launch_router_bf16_t<2, 2>(x, Wg, T, d, n, K, topk_idx, topk_w, hist, s);
  else if (ne <= 4)
    launch_router_bf16_t<4, 2>(x, Wg, T, d, n, K, topk_idx, topk_w, hist, s);
  else if (ne <= 8)
    launch_router_bf16_t<8, 2>(x, Wg, T, d, n, K, topk_idx, topk_w, hist, s);
  else
    launch_router_bf16_t<16, 1>(x, Wg, T, d, n, K, topk_idx, topk_w, hist, s);
  return hipGetLastError();
}

hipError_t launch_router_f32(const float* x, const float* Wg, int64_t T, int64_t d, int n, int K,
                             int* topk_idx, float* topk_w, int* hist, hipStream_t s) {
  const int BT = route_block_tokens(n);
  const int64_t nb = (T + BT - 1) / BT;
  hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)nb), dim3(256), 0, s, x, Wg, T, d, n, K, BT,
                     topk_idx, topk_w, hist);
  return hipGetLastError();
}

hipError_t launch_scatter(const int* topk_idx, const int* hist, int64_t T, int n, int K,
                          int* counts, int* offsets, int* perm_token, int* slot_pos, hipStream_t s) {
  const int BT = route_block_tokens(n);
  const int nb = (int)((T + BT - 1) / BT);
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nb), dim3(256), 0, s, topk_idx, hist, T, n, K,
                     BT, nb, counts, offsets, perm_token, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
