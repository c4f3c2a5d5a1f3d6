// Dispatch invariants, checked on the device.
//
// The grouping of assignments by expert (moe_route) is defined by the token
// choice it follows (Part 3 of "Mixture of Experts: Why Mixtral Only Wakes Up
// Two Specialists", step 2: each token keeps its K highest-scoring experts):
// every kept assignment (t, k) of expert e = topk_idx[t][k] owns exactly one
// position p = slot_pos[t][k] of e's segment [offsets[e], offsets[e+1]), with
// perm_token[p] = t, and each segment lists its tokens in ascending order.
// This kernel checks those properties (and counts/offsets consistency) and
// reports violations as bit flags; it never writes anything else.
#include <algorithm>

#include "moe_internal.h"

namespace moe {

namespace {

// expert whose segment holds position p (offsets ascending, n <= 256)
__device__ int segment_of(const int* __restrict__ offsets, int n, int p) {
  int lo = 0, hi = n;  // offsets[lo] <= p < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ void flag(int* err, int bit, int64_t where) {
  atomicOr(&err[0], bit);
  atomicMin(&err[1], (int)min<int64_t>(where, INT32_MAX));
}

__global__ __launch_bounds__(256) void validate_kernel(const int* __restrict__ topk_idx,
                                                       const int* __restrict__ counts,
                                                       const int* __restrict__ offsets,
                                                       const int* __restrict__ perm_token,
                                                       const int* __restrict__ slot_pos, int64_t T, int n, int K,
                                                       int cap, int* __restrict__ err) {
  const int64_t TK = T * K;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // counts and offsets
  for (int64_t e = gid; e <= n; e += stride) {
    if (e == 0 && offsets[0] != 0) flag(err, kValidateOffsets, 0);
    if (e < n) {
      const int c = counts[e];
      if (c < 0 || c > cap || offsets[e + 1] - offsets[e] != c) flag(err, kValidateOffsets, e);
    } else {
      const int total = offsets[n];
      if (total < 0 || total > TK || (cap == INT32_MAX && total != TK)) flag(err, kValidateTotal, e);
    }
  }
  const int total = offsets[n];
  if (total < 0 || total > TK) return;  // flagged above; positions below would be out of range
  // assignments: index in range and distinct within the token, slot in the expert's segment, back-pointer
  for (int64_t a = gid; a < TK; a += stride) {
    const int64_t t = a / K;
    const int k = (int)(a % K);
    const int e = topk_idx[a];
    if (e < 0 || e >= n) {
      flag(err, kValidateIndex, a);
      continue;
    }
    for (int j = 0; j < k; ++j)
      if (topk_idx[t * K + j] == e) flag(err, kValidateIndex, a);
    const int sp = slot_pos[a];
    if (sp == -1 && cap != INT32_MAX) continue;  // dropped by a full expert
    if (sp < 0 || sp >= total || sp < offsets[e] || sp >= offsets[e + 1]) {  // caller data: every read in range
      flag(err, kValidateSlot, a);
      continue;
    }
    if (perm_token[sp] != t) flag(err, kValidatePerm, a);
  }
  // positions: a token of the batch, ascending within a segment, and owned by
  // the assignment that points back to it
  for (int64_t p = gid; p < total; p += stride) {
    const int t = perm_token[p];
    if (t < 0 || t >= T) {
      flag(err, kValidatePerm, p);
      continue;
    }
    const int e = segment_of(offsets, n, (int)p);
    if (p + 1 < total && p + 1 < offsets[e + 1] && perm_token[p + 1] <= t) flag(err, kValidateOrder, p);
    int owner = -1;
    for (int j = 0; j < K; ++j)
      if (topk_idx[(int64_t)t * K + j] == e) owner = j;
    if (owner < 0 || slot_pos[(int64_t)t * K + owner] != (int)p) flag(err, kValidatePerm, p);
  }
}

__global__ void validate_clear(int* err) {
  err[0] = 0;
  err[1] = INT32_MAX;
}

}  // namespace

hipError_t launch_validate(const int* topk_idx, const int* counts, const int* offsets, const int* perm_token,
                           const int* slot_pos, int64_t T, int n, int K, int cap, int* err, hipStream_t s) {
  hipLaunchKernelGGL(validate_clear, dim3(1), dim3(1), 0, s, err);
  const int64_t work = std::max<int64_t>(T * K, n + 1);
  const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 4096);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(256), 0, s, topk_idx, counts, offsets, perm_token, slot_pos,
                     T, n, K, cap, err);
  return hipGetLastError();
}

}  // namespace moe
