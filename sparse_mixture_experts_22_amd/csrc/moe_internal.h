// Internal interface between the C-ABI host layer (api.hip) and the kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace moe {

constexpr int kMaxN = 256;  // experts per layer
constexpr int kMaxK = 8;    // experts kept per token

// Native clang vectors (not HIP's struct vector types): plain loads/stores,
// so staging arrays of them stay in registers.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Load of expert weights that a decode-size call reads exactly once: marked
// non-temporal, so the stream does not displace cached lines on its way (the
// Mixtral decode layer reads its 2.8 GB of weights 10-12% faster this way).
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
  return __builtin_nontemporal_load(p);
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Tokens per routing block (the router, scan and scatter agree on it; <= 32).
int route_block_tokens(int n);
// Experts rounded up to a multiple of 16 (rows of the transposed router).
int route_padded_experts(int n);

// Device buffers of the routing stage (all in the library workspace except
// where a caller of moe_route supplies its own outputs).
struct RouteBuffers {
  int* topk_idx;    // [T][K]
  float* topk_w;    // [T][K]
  int* hist;        // [nb][n] per-block expert histograms
  int* bases;       // [nb][n] per-block first positions
  int* counts;      // [n]
  int* offsets;     // [n+1]
  int* perm_token;  // [T*K]
  int* slot_pos;    // [T][K]
  uint16_t* wgT;    // [n_pad][d] transposed router (bf16 path)
  float* split = nullptr;  // [d / 256][32][16] partial logits of the split single-block router
  int* zero = nullptr;  // words the router sets to zero (the packed GEMMs' work counters)
  int n_zero = 0;
};

// Rows of an expert handled by one prefill tile.
constexpr int kPrefillBM = 256;

// Average assignments per expert at or below which the weight-streaming
// ("skinny") expert kernels are used instead of the tiled grouped GEMM.
constexpr int kSkinnyMaxAvgRows = 24;
// Split of the down projection's reduction in the skinny path.  Two splits
// (each wave streams half of its split's rows) beat four at the Mixtral decode
// shape: longer weight streams per wave, and half the partial sums to combine.
constexpr int kSkinnyDownSplits = 2;

// ---------------------------------------------------------------- routing
// Router + top-K + softmax + dispatch; fills every RouteBuffers output.
// `after_router` (optional) is recorded between the router and the dispatch.
// `cap`: each expert keeps its first `cap` assignments in token order, the
// rest get slot_pos -1 and no row (counts/offsets/perm_token cover the kept).
hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                             int K, const RouteBuffers& rb, hipStream_t s,
                             hipEvent_t after_router = nullptr, int cap = INT32_MAX);
hipError_t launch_route_f32(const float* x, const float* Wg, int64_t T, int64_t d, int n, int K,
                            const RouteBuffers& rb, hipStream_t s);
// Router statistics: frac[e] = counts[e]/(T*K), prob[e] = mean over tokens of
// the full n-way softmax, aux_loss = alpha*n*sum_e frac[e]*prob[e] (each
// output optional).  Fills topk_idx, topk_w and hist of rb; probsum holds
// [blocks][n] floats.
hipError_t launch_route_stats_bf16(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                                   int K, float alpha, const RouteBuffers& rb, float* probsum,
                                   float* frac, float* prob, float* aux_loss, hipStream_t s);
hipError_t launch_route_stats_f32(const float* x, const float* Wg, int64_t T, int64_t d, int n, int K,
                                  float alpha, const RouteBuffers& rb, float* probsum, float* frac,
                                  float* prob, float* aux_loss, hipStream_t s);
// Expert-choice routing: topk_w receives the scores [T][n] (each token's
// softmax over the experts); expert e takes its C best tokens (ties to the
// lower token index) into rows e*C .. e*C+C-1 in ascending token order:
// perm_token [n*C], slot_pos [T][n] (-1 where e did not choose t),
// counts[e] = C, offsets[e] = e*C.  1 <= C <= T.
hipError_t launch_route_expert_choice(const uint16_t* x, const uint16_t* Wg, int64_t T, int64_t d, int n,
                                     int C, const RouteBuffers& rb, hipStream_t s);
// Scan + scatter from topk_idx and hist (used after a multi-block router).
hipError_t launch_dispatch(int64_t T, int n, int K, const RouteBuffers& rb, hipStream_t s,
                           int cap = INT32_MAX);

// ------------------------------------------------------ expert projections
// Gate/up: h[p][:] = SiLU(x[perm_token[p]] W1_e) * (x[perm_token[p]] W3_e), bf16 out.
// `cus_per_xcd`: compute units per XCD of the device (tile scheduling).
hipError_t launch_prefill_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W1,
                             const uint16_t* W3, const int* offsets, int64_t TK, int n, int d, int f,
                             int cus_per_xcd, uint16_t* h, hipStream_t s);
// Down: o[p][:] = h[p] W2_e, fp32 out.  With `tail_ws` (prefill_tail_bytes
// bytes, 1 <= cus_per_xcd <= 64) the tiles left over after the last full wave
// are split over k and their pieces summed by a second kernel; with nullptr
// every tile runs whole.
hipError_t launch_prefill_down(const uint16_t* h, const uint16_t* W2, const int* offsets, int64_t TK,
                               int n, int f, int d, int cus_per_xcd, float* tail_ws, float* o,
                               hipStream_t s);
size_t prefill_tail_bytes(int cus_per_xcd);
// Sums the k-pieces of the split leftover tiles of a tiled down projection
// (N output columns, nk k-steps of 32, pieces multiples of `gran` k-steps) into o.
hipError_t launch_tail_reduce(const int* offsets, int n, int N, int nk, int cus_per_xcd, int gran,
                              const float* tail_ws, float* o, hipStream_t s);
// Packed weights (fragment order, see gemm_packed.hip): W13p from W1, W3
// [n][d][f] (d % 128 == 0, f % 128 == 0); W2p from W2 [n][f][d] (f % 128 == 0,
// d % 256 == 0).  mode 1 packs (W, W3) as the up pair, mode 2 packs W alone.
hipError_t launch_pack(int mode, const uint16_t* W, const uint16_t* W3, int n, int R, int C, uint16_t* out,
                       hipStream_t s);
// The tiled packed projections run one workgroup per compute unit, each taking
// tiles from a work list until it is empty (1 <= cus_per_xcd <= 64).  `sched`:
// kPackedSchedWords int32 of device memory whose first kPackedCounterWords
// words are zero at the up projection's launch (the router clears them).
constexpr int kPackedCounterWords = 16;
// Tile-trace build: records per projection, workgroup and tile (see gemm_packed.hip).
constexpr int kTileTraceWgs = 512, kTileTraceTiles = 64, kTileTraceFields = 12;
constexpr int kPackedSchedWords = kPackedCounterWords + 2 * 2 * 8 * 64;
hipError_t launch_packed_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W13p,
                            const int* offsets, int64_t TK, int n, int d, int f, int cus_per_xcd, int* sched,
                            uint16_t* h, hipStream_t s);
hipError_t launch_packed_down(const uint16_t* h, const uint16_t* W2p, const int* offsets, int64_t TK, int n, int f,
                              int d, int cus_per_xcd, int* sched, float* tail_ws, float* o, hipStream_t s);
// Weight streaming on packed weights (decode-sized batches): the up projection
// streams each touched expert's pairs once; the down projection splits the
// reduction over f into `splits` parts (o[split][p][:] partial sums).
int packed_stream_splits(int n, int f, int d, int cus_per_xcd);
hipError_t launch_packed_stream_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W13p,
                                   const int* offsets, int64_t TK, int n, int d, int f, uint16_t* h, hipStream_t s);
hipError_t launch_packed_stream_down(const uint16_t* h, const uint16_t* W2p, const int* offsets, int64_t TK, int n,
                                     int f, int d, int splits, float* o, hipStream_t s);
hipError_t launch_skinny_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W1,
                            const uint16_t* W3, const int* offsets, int64_t TK, int n, int d, int f,
                            uint16_t* h, hipStream_t s);
// Down with the reduction over f split in `splits` parts: o[s][p][:] partial sums.
hipError_t launch_skinny_down(const uint16_t* h, const uint16_t* W2, const int* offsets, int64_t TK,
                              int n, int f, int d, int splits, float* o, hipStream_t s);
hipError_t launch_f32_up(const float* x, int64_t T, const int* perm_token, const float* W1, const float* W3,
                         const int* offsets, int64_t TK, int n, int d, int f, float* h, hipStream_t s);
hipError_t launch_f32_down(const float* h, const float* W2, const int* offsets, int64_t TK, int n,
                           int f, int d, float* o, hipStream_t s);

// ------------------------------------------------------- 4-bit weights
// Quantize W bf16 [n][R][C] (R % 128 == 0, C % 2 == 0) into codes
// (n*R*C/2 bytes, 16-byte aligned) and bf16 scales [n][R/128][C].
hipError_t launch_quantize_q4(const uint16_t* W, int n, int R, int C, uint8_t* codes, uint16_t* scales,
                              hipStream_t s);
// Decode-size projections on 4-bit weights (same row layout as the bf16 ones).
hipError_t launch_q4_up(const uint16_t* x, int64_t T, const int* perm_token, const uint8_t* Q1,
                        const uint16_t* S1, const uint8_t* Q3, const uint16_t* S3, const int* offsets,
                        int64_t TK, int n, int d, int f, int cus, uint16_t* h, hipStream_t s);
hipError_t launch_q4_down(const uint16_t* h, const uint8_t* Q2, const uint16_t* S2, const int* offsets,
                          int64_t TK, int n, int f, int d, int splits, int cus, float* o, hipStream_t s);

// ------------------------------------------------------------ validation
// Dispatch invariants, as bit flags in err[0] (err[1]: smallest offending index).
constexpr int kValidateOffsets = 1;  // offsets[0] != 0, a count negative, above the capacity or != its segment
constexpr int kValidateTotal = 2;    // offsets[n] != T*K (dropless) or outside [0, T*K]
constexpr int kValidateIndex = 4;    // an expert index out of range or repeated within a token
constexpr int kValidateSlot = 8;     // slot_pos outside its expert's segment (or -1 without a capacity)
constexpr int kValidatePerm = 16;    // perm_token and slot_pos do not point at each other
constexpr int kValidateOrder = 32;   // tokens not ascending within an expert's segment
// Clears err and checks the arrays; err is 2 ints of device memory.  cap = INT32_MAX: dropless.
hipError_t launch_validate(const int* topk_idx, const int* counts, const int* offsets, const int* perm_token,
                           const int* slot_pos, int64_t T, int n, int K, int cap, int* err, hipStream_t s);

// ----------------------------------------------------------------- combine
// y[t][:] = sum_k topk_w[t][k] * (sum_s o[s][slot_pos[t][k]][:]), k and s ascending.
hipError_t launch_combine(const float* o, int splits, int64_t TK, const float* topk_w,
                          const int* slot_pos, int64_t T, int64_t d, int K, float* y, hipStream_t s);

// bf16 round-to-nearest-even of a finite float.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// The same rounding for two values at once (the hardware's packed conversion,
// round to nearest even; its low half is v[0]).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(f32x2_t v) {
  const bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return *reinterpret_cast<const uint32_t*>(&b);
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + expf(-a)); }

// SiLU for outputs that are rounded to bf16 right away: a * 1/(1 + 2^(-a*log2 e))
// with the hardware base-2 exponential and reciprocal (about 1 ulp each, a few
// 1e-7 relative after the argument's rounding), far below bf16's 2^-9 step.
// Saturates like the exact form: 2^(large) = inf gives 1/inf = 0, so -0.
__device__ __forceinline__ float silu_bf16out(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.44269504088896341f));
}

}  // namespace moe
