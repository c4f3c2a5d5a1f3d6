// Weighted combine, and the fp32 expert projections.
//
// Combine: step 4 of "Pip's token goes to triage" (Part 3 of "Mixture of
// Experts: Why Mixtral Only Wakes Up Two Specialists"): each chosen expert's
// output is scaled by its gate weight and the results are added; the general
// token-choice form sum_j alpha_{i_j} E_{i_j}(x) is in "How Experts Are Chosen
// (Routing Methods)" of "Mixtral of Experts? Mixture of Experts? Try to
// explain Mixtral 8x7B".  Here it is a gather-sum over the K slots of each
// token in slot order (one writer per output element, no atomics).
//
// fp32 projections: plain 16x16 LDS-tiled FMA kernels over the same grouped
// layout (expert-contiguous rows); they serve the fp32 entry point.
#include "moe_internal.h"

namespace moe {

namespace {

template <int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o, int splits,
                                                      int64_t TK, const float* __restrict__ topk_w,
                                                      const int* __restrict__ slot_pos, int64_t T,
                                                      int64_t d, int K, float* __restrict__ y) {
  const int64_t dv = d / VEC;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * dv) return;
  const int64_t t = idx / dv;
  const int64_t c = (idx % dv) * VEC;
  float acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.0f;
  for (int k = 0; k < K; ++k) {
    const int sp = slot_pos[t * K + k];
    if (sp < 0) continue;  // an assignment dropped by a full expert contributes nothing
    const int64_t pos = min<int64_t>(sp, TK - 1);
    const float w = topk_w[t * K + k];
    float v[VEC];
    if (VEC == 4) {
      const float4 q = *reinterpret_cast<const float4*>(o + pos * d + c);
      v[0] = q.x;
      v[1 % VEC] = q.y;
      v[2 % VEC] = q.z;
      v[3 % VEC] = q.w;
    } else {
      v[0] = o[pos * d + c];
    }
    for (int s = 1; s < splits; ++s) {
      const float* os = o + ((int64_t)s * TK + pos) * d + c;
#pragma unroll
      for (int j = 0; j < VEC; ++j) v[j] += os[j];
    }
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = acc[j] + w * v[j];
  }
  if (VEC == 4) {
    *reinterpret_cast<float4*>(y + t * d + c) = make_float4(acc[0], acc[1 % VEC], acc[2 % VEC], acc[3 % VEC]);
  } else {
    y[t * d + c] = acc[0];
  }
}

// Locate 16-row tile `L` of the fp32 grouped GEMM: its expert, first row and height.
__device__ bool f32_tile(const int* __restrict__ offsets, int n, int L, int& e_out, int& row0,
                         int& rows) {
  for (int e = 0; e < n; ++e) {
    const int c = offsets[e + 1] - offsets[e];
    const int mt = (c + 15) / 16;
    if (L < mt) {
      e_out = e;
      row0 = offsets[e] + L * 16;
      rows = offsets[e + 1] - row0;
      if (rows > 16) rows = 16;
      return true;
    }
    L -= mt;
  }
  return false;
}

template <int MODE>
__global__ __launch_bounds__(256) void f32_gemm_kernel(const float* __restrict__ A,
                                                       const int* __restrict__ perm_token,
                                                       const float* __restrict__ B1,
                                                       const float* __restrict__ B3,
                                                       const int* __restrict__ offsets, int n,
                                                       int64_t Kdim, int64_t N, int64_t a_rows,
                                                       int64_t TK, float* __restrict__ hout,
                                                       float* __restrict__ oout) {
  __shared__ float As[16][17];
  __shared__ float B1s[16][17];
  __shared__ float B3s[16][17];
  // blockIdx.x = row tile * ncol_tiles + column tile
  const int64_t nct = (N + 15) / 16;
  const int64_t ct = blockIdx.x % nct;
  int e, row0, rows;
  if (!f32_tile(offsets, n, (int)(blockIdx.x / nct), e, row0, rows)) return;
  const int tx = threadIdx.x & 15;
  const int ty = threadIdx.x >> 4;
  const int64_t col = ct * 16 + tx;
  const int ra = ty < rows ? ty : rows - 1;
  const int64_t p = min<int64_t>(max<int64_t>(row0 + ra, 0), TK - 1);
  const int64_t arow = (MODE == 1) ? min<int64_t>(max(perm_token[p], 0), a_rows - 1) : p;
  const int64_t e_off = (int64_t)e * Kdim * N;
  float acc1 = 0.0f, acc3 = 0.0f;
  for (int64_t k0 = 0; k0 < Kdim; k0 += 16) {
    As[ty][tx] = (k0 + tx < Kdim) ? A[arow * Kdim + k0 + tx] : 0.0f;
    const int64_t bcol = col;
    const bool bok = (k0 + ty < Kdim) && (bcol < N);
    B1s[ty][tx] = bok ? B1[e_off + (k0 + ty) * N + bcol] : 0.0f;
    if (MODE == 1) B3s[ty][tx] = bok ? B3[e_off + (k0 + ty) * N + bcol] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      acc1 = fmaf(As[ty][kk], B1s[kk][tx], acc1);
      if (MODE == 1) acc3 = fmaf(As[ty][kk], B3s[kk][tx], acc3);
    }
    __syncthreads();
  }
  if (ty < rows && col < N && row0 + ty < TK) {
    if (MODE == 1)
      hout[(int64_t)(row0 + ty) * N + col] = silu_f32(acc1) * acc3;
    else
      oout[(int64_t)(row0 + ty) * N + col] = acc1;
  }
}

// The same sum when a token has many slots of which few are set (expert-choice
// routing passes one slot per expert).  A workgroup takes 1024 columns of one
// token; wave 0 reads the token's K slots in parallel and lists the set ones in
// slot order, then every thread adds only those, in that order, so the result
// equals combine_kernel's bit for bit.
constexpr int kSparseCombineMinK = 8;
__global__ __launch_bounds__(256) void combine_sparse_kernel(const float* __restrict__ o, int splits,
                                                             int64_t TK, const float* __restrict__ topk_w,
                                                             const int* __restrict__ slot_pos, int64_t d,
                                                             int K, float* __restrict__ y) {
  __shared__ int pos_s[kMaxN];
  __shared__ float w_s[kMaxN];
  __shared__ int cnt_s;
  const int64_t chunks = (d + 1023) / 1024;
  const int64_t t = blockIdx.x / chunks;
  const int64_t c = (blockIdx.x % chunks) * 1024 + threadIdx.x * 4;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int cnt = 0;
    for (int base = 0; base < K; base += 64) {
      const int k = base + lane;
      const int sp = k < K ? slot_pos[t * K + k] : -1;
      const unsigned long long set = __ballot(sp >= 0);
      if (sp >= 0) {
        const int r = cnt + __popcll(set & ((1ull << lane) - 1));
        pos_s[r] = (int)min<int64_t>(sp, TK - 1);
        w_s[r] = topk_w[t * K + k];
      }
      cnt += __popcll(set);
    }
    if (lane == 0) cnt_s = cnt;
  }
  __syncthreads();
  if (c >= d) return;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int cnt = cnt_s;
  for (int r = 0; r < cnt; ++r) {
    const int64_t pos = pos_s[r];
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(o + pos * d + c);
    for (int sidx = 1; sidx < splits; ++sidx) {
      const f32x4_t q = *reinterpret_cast<const f32x4_t*>(o + ((int64_t)sidx * TK + pos) * d + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += q[j];
    }
    const float w = w_s[r];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = acc[j] + w * v[j];
  }
  *reinterpret_cast<f32x4_t*>(y + t * d + c) = acc;
}

}  // namespace

hipError_t launch_combine(const float* o, int splits, int64_t TK, const float* topk_w,
                          const int* slot_pos, int64_t T, int64_t d, int K, float* y, hipStream_t s) {
  const bool vec = (d % 4) == 0 && (reinterpret_cast<uintptr_t>(o) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) % 16) == 0;
  if (vec && K >= kSparseCombineMinK && K <= kMaxN && T * ((d + 1023) / 1024) <= INT32_MAX) {
    const int64_t blocks = T * ((d + 1023) / 1024);
    hipLaunchKernelGGL(combine_sparse_kernel, dim3((unsigned)blocks), dim3(256), 0, s, o, splits, TK, topk_w,
                       slot_pos, d, K, y);
    return hipGetLastError();
  }
  const int64_t items = T * (vec ? d / 4 : d);
  const unsigned blocks = (unsigned)((items + 255) / 256);
  if (vec)
    hipLaunchKernelGGL(combine_kernel<4>, dim3(blocks), dim3(256), 0, s, o, splits, TK, topk_w,
                       slot_pos, T, d, K, y);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(blocks), dim3(256), 0, s, o, splits, TK, topk_w,
                       slot_pos, T, d, K, y);
  return hipGetLastError();
}

hipError_t launch_f32_up(const float* x, int64_t T, const int* perm_token, const float* W1, const float* W3,
                         const int* offsets, int64_t TK, int n, int d, int f, float* h, hipStream_t s) {
  const unsigned grid = (unsigned)(((TK + 15) / 16 + n) * ((f + 15) / 16));
  hipLaunchKernelGGL((f32_gemm_kernel<1>), dim3(grid), dim3(256), 0, s, x,
                     perm_token, W1, W3, offsets, n, (int64_t)d, (int64_t)f, T, TK, h,
                     (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_f32_down(const float* h, const float* W2, const int* offsets, int64_t TK, int n,
                           int f, int d, float* o, hipStream_t s) {
  const unsigned grid = (unsigned)(((TK + 15) / 16 + n) * ((d + 15) / 16));
  hipLaunchKernelGGL((f32_gemm_kernel<2>), dim3(grid), dim3(256), 0, s, h,
                     (const int*)nullptr, W2, (const float*)nullptr, offsets, n, (int64_t)f,
                     (int64_t)d, TK, TK, (float*)nullptr, o);
  return hipGetLastError();
}

}  // namespace moe
