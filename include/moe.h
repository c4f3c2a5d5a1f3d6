/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts layer.
 *
 * The layer (card 2.1 "Sparse Mixture of Experts" of the "Mixtral of Experts"
 * study deck, Jiang et al. 2024):
 *
 *     y = sum_{i=0}^{n-1} Softmax(TopK(x . W_g))_i * SwiGLU_i(x)
 *
 * A bias-free linear router scores the n experts of every token, the K largest
 * scores are kept (ties to the lower expert index, kept slots in descending
 * score order), a softmax over the kept scores gives the gate weights, only the
 * chosen experts run, and their outputs are summed with those weights (Part 3,
 * "Pip's token goes to triage", steps 1-4, of "Mixture of Experts: Why Mixtral
 * Only Wakes Up Two Specialists").  SwiGLU_i(z) = (SiLU(z W1_i) * (z W3_i)) W2_i,
 * SiLU(u) = u / (1 + e^-u); no biases anywhere.  Expert indices are 0-based.
 *
 * Conventions shared by every entry point:
 *   - Tensors are DEVICE pointers, row-major, contiguous, owned by the caller.
 *     The library keeps no pointer after a call returns.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *     caller keeps buffers alive until that work completes.
 *   - Every argument is validated before anything is enqueued; on an error
 *     nothing is enqueued and the status says why (moe_last_error() has the
 *     detail).  T == 0 is a valid no-op; then the per-token arrays (x, y and
 *     the per-token routing outputs) may be null, since none of them is
 *     accessed.  No C++ exception crosses the ABI.
 *   - Layouts: x[T][d], W_g[d][n] (so logits = x . W_g; a PyTorch nn.Linear
 *     router weight [n][d] is passed transposed), W1[n][d][f], W3[n][d][f],
 *     W2[n][f][d].  bf16 entry points take bf16 storage (uint16 bit patterns).
 *   - Limits: 1 <= K <= n <= 256, K <= 8, T*K < 2^31.  bf16 entry points need
 *     d % 64 == 0, f % 64 == 0 and 16-byte aligned tensors (MOE_ERR_UNSUPPORTED).
 *   - The library owns a per-device workspace (routing arrays, the
 *     intermediate h and o buffers and partial sums of split tiles;
 *     moe_workspace_bytes() gives what one call needs).  It is allocated on the
 *     first call on a device and grown on demand, at least doubling; an
 *     outgrown buffer is not freed but kept until moe_release(), so work
 *     already enqueued and HIP graphs captured over earlier calls keep valid
 *     addresses.  moe_release() frees every buffer: a graph captured over any
 *     call must not be replayed after it.  Capture a call only after a call
 *     of the same or a larger shape has run uncaptured (a growing call
 *     allocates).  Calls that share a device's workspace must not run
 *     concurrently on different streams.
 *   - Results are deterministic: no float atomics; every output element has a
 *     single writer and a fixed summation order.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, K < 1, K > n, n < 1, d/f < 1, T < 0 */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside this library's limits (see above) */
  MOE_ERR_HIP = 3,         /* a HIP call or kernel launch failed */
  MOE_ERR_NO_MEMORY = 4,   /* workspace allocation failed */
  MOE_ERR_VALIDATION = 5   /* a dispatch check failed (moe_check_dispatch, MOE_VALIDATE=1) */
} moe_status_t;

/* Opaque HIP stream handle (hipStream_t). */
typedef struct ihipStream_t* moe_stream_t;

/*
 * moe_forward -- the whole layer, bf16 storage, fp32 accumulation.
 *   x[T][d], Wg[d][n], W1[n][d][f], W3[n][d][f], W2[n][f][d]: bf16.
 *   y[T][d]: fp32, fully overwritten (the caller adds the residual).
 * Routing is computed exactly as moe_route does (same kernels).  The SwiGLU
 * hidden activation is rounded once to bf16 (round-to-nearest-even) before
 * the down projection; everything else accumulates and is stored in fp32.
 * The combine sums the K expert outputs in slot order.
 */
moe_status_t moe_forward(const void* x, const void* Wg, const void* W1, const void* W3,
                         const void* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                         int32_t K, float* y, moe_stream_t stream);

/*
 * moe_forward_traced -- moe_forward that also records caller-created HIP events
 * (hipEvent_t, passed as void*) on `stream` between its stages, for timing:
 *   stage_events[0] before the router      [1] after the router
 *   stage_events[2] after the dispatch     [3] after the gate/up projection
 *   stage_events[4] after the down proj.   [5] after the combine
 * When a batch fits one routing block the router kernel also performs the
 * dispatch, and [1] is recorded right after it.
 * Same kernels and results as moe_forward; all six events are required.
 */
moe_status_t moe_forward_traced(const void* x, const void* Wg, const void* W1, const void* W3,
                                const void* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                                int32_t K, float* y, moe_stream_t stream, void* const* stage_events);

/*
 * Packed expert weights: the same bf16 values in the order the matrix cores
 * consume them, written once (at weight-load time) and then read by
 * moe_forward_packed on every call.  The layer is the one moe_forward computes
 * (card 2.1 "Sparse Mixture of Experts" of the "Mixtral of Experts" study
 * deck): only the storage order of W1, W3 and W2 differs.
 * Format, for a stack with reduction index k and columns c:
 *     P[e][g][kk][w][j][l][i]  bf16, kk = k / 16, w = 0..3, j = 0..1, l = 0..63,
 *     i = 0..7, holds W[e][16 kk + 8 (l / 32) + i][column of (pb, j, l % 32)]
 *     with the column pair pb = 4 g + w
 *   up pair  (moe_pack_up, from W1 and W3 [n][d][f], 2*n*d*f values):
 *            pb < f / 32; j = 0 takes W1, j = 1 takes W3, column 32 pb + l % 32
 *   down     (moe_pack_down, from W2 [n][f][d], n*f*d values):
 *            pb < d / 64; column 64 pb + 32 j + l % 32
 * (one 1 KiB unit per (pb, kk, j) is one MFMA operand; four adjacent pairs'
 * whole reduction is one contiguous stream of 8 KiB per kk).  Both need d % 256 == 0, f % 128 == 0,
 * n <= 256 and 16-byte aligned tensors (MOE_ERR_UNSUPPORTED otherwise); the
 * output buffers are caller-allocated, not overlapping the inputs.
 *
 * moe_forward_packed -- moe_forward on packed weights: x[T][d], Wg[d][n] bf16,
 *   W13p from moe_pack_up, W2p from moe_pack_down, y[T][d] fp32.  Routing,
 *   SwiGLU, bf16 rounding of h and the combine are those of moe_forward; the
 *   expert projections multiply in the same order, so y equals moe_forward's
 *   bit for bit on the tiled path except where the last tiles of the down
 *   projection are split over the reduction (then to fp32 summation order).
 * moe_forward_packed_traced -- the same with the six stage events of
 *   moe_forward_traced.
 */
moe_status_t moe_pack_up(const void* W1, const void* W3, int32_t n, int64_t d, int64_t f, void* W13p,
                         moe_stream_t stream);
moe_status_t moe_pack_down(const void* W2, int32_t n, int64_t f, int64_t d, void* W2p, moe_stream_t stream);
moe_status_t moe_forward_packed(const void* x, const void* Wg, const void* W13p, const void* W2p, int64_t T,
                                int64_t d, int64_t f, int32_t n, int32_t K, float* y, moe_stream_t stream);
moe_status_t moe_forward_packed_traced(const void* x, const void* Wg, const void* W13p, const void* W2p, int64_t T,
                                       int64_t d, int64_t f, int32_t n, int32_t K, float* y, moe_stream_t stream,
                                       void* const* stage_events);

/*
 * moe_forward_noalloc -- moe_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, validation and routing; it calls no
 * hipMalloc/hipFree and no allocating library routine.  Its intermediates live
 * in a fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends.
 *   - A shape whose intermediates exceed that size returns MOE_ERR_UNSUPPORTED
 *     before anything is enqueued; moe_noalloc_scratch_bytes() gives the need
 *     (Mixtral decode batches, T = 32, d = 4096, f = 14336, n = 8, K = 2, need
 *     about 4 MiB; the weight-streaming path covers T*K <= 24*n).
 *   - Weight-streaming shapes (T*K <= 24*n) give results bitwise equal to
 *     moe_forward.  On the tiled path every down-projection tile runs whole
 *     (moe_forward may split the last tiles over the reduction), so results
 *     agree to fp32 summation order.
 *   - Every call on a device shares that device's scratch, which keeps the last
 *     call's contents (each call writes everything it reads, nothing needs to
 *     start at zero).  Calls that overlap on one device race: serialise them
 *     on one stream.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

moe_status_t moe_forward_noalloc(const void* x, const void* Wg, const void* W1, const void* W3,
                                 const void* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                                 int32_t K, float* y, moe_stream_t stream);

/* Scratch bytes moe_forward_noalloc needs for this shape (0 on invalid shapes). */
size_t moe_noalloc_scratch_bytes(int64_t T, int64_t d, int64_t f, int32_t n, int32_t K);

/*
 * moe_forward_f32 -- the same layer with every input in fp32 (the hidden
 * activation stays fp32).  No alignment or divisibility requirement.
 */
moe_status_t moe_forward_f32(const float* x, const float* Wg, const float* W1, const float* W3,
                             const float* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                             int32_t K, float* y, moe_stream_t stream);

/*
 * moe_route -- router, top-K, softmax over the kept K, and the integer dispatch
 * (steps 1-3 of the walk-through plus the grouping of assignments by expert that
 * lets each chosen expert run once on its rows; unselected experts are never
 * evaluated, per the sparse-gating passage of "How a mixture-of-experts model
 * activates only part of its parameters").  x[T][d], Wg[d][n]: bf16.
 * Every output is optional (NULL = not written); at least one must be given.
 *   topk_idx[T][K]  int32  kept experts, descending logit, ties -> lower index
 *   topk_w[T][K]    fp32   softmax over the kept logits (sums to 1 per token)
 *   counts[n]       int32  number of assignments per expert
 *   offsets[n+1]    int32  exclusive prefix sum of counts; offsets[n] = T*K
 *   perm_token[T*K] int32  token at each position, expert-contiguous, tokens
 *                          ascending within an expert
 *   slot_pos[T][K]  int32  position of assignment (t, k): perm_token[slot_pos] = t
 * The integer outputs are a pure function of the logits' fp32 values.
 */
moe_status_t moe_route(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n,
                       int32_t K, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* slot_pos,
                       moe_stream_t stream);

/* moe_route_f32 -- moe_route with fp32 x and Wg. */
moe_status_t moe_route_f32(const float* x, const float* Wg, int64_t T, int64_t d, int32_t n,
                           int32_t K, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* perm_token, int32_t* slot_pos,
                           moe_stream_t stream);

/*
 * moe_route_stats -- router statistics and the load-balancing loss of the
 * Switch design described in Part 5 of "Mixture of Experts: Why Mixtral Only
 * Wakes Up Two Specialists" ("The favourite expert problem", tool 2), for the
 * top-K routing of moe_route.  x[T][d], Wg[d][n]: bf16; T >= 1.
 *   frac[n]     fp32  share of the T*K assignments sent to each expert,
 *                     counts[e] / (T*K) (sums to 1)
 *   prob[n]     fp32  mean over the tokens of the router's full n-way softmax
 *                     probability of each expert (sums to 1)
 *   aux_loss[1] fp32  alpha * n * sum_e frac[e] * prob[e]; equals alpha when
 *                     either share is uniform (1/n each)
 * Each output is optional (NULL = not written); at least one must be given.
 * The selection is the one moe_route makes (same kernels); sums over tokens
 * run in a fixed order, so results are reproducible.  T == 0 or a NaN alpha
 * -> MOE_ERR_INVALID_ARG.
 */
moe_status_t moe_route_stats(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n,
                             int32_t K, float alpha, float* frac, float* prob, float* aux_loss,
                             moe_stream_t stream);

/* moe_route_stats_f32 -- moe_route_stats with fp32 x and Wg. */
moe_status_t moe_route_stats_f32(const float* x, const float* Wg, int64_t T, int64_t d, int32_t n,
                                 int32_t K, float alpha, float* frac, float* prob, float* aux_loss,
                                 moe_stream_t stream);

/*
 * Capacity-limited routing: the expert capacity of the Switch design described
 * in Part 5 of "Mixture of Experts: Why Mixtral Only Wakes Up Two Specialists"
 * ("What happens when an expert is full"): the tokens of the batch divided by
 * the number of experts, times a capacity factor; with K assignments per token
 * it is C = ceil(capacity_factor * T * K / n).  Each expert keeps its first C
 * assignments in token order; the others are dropped: they get no row, no
 * computation and contribute nothing to y (the token passes on through the
 * caller's residual add; the kept gate weights are not renormalised, so a
 * token whose K assignments are all dropped gets y = 0).
 *   moe_expert_capacity  returns C (0 if capacity_factor is not positive and
 *                        finite or C does not fit an int32).
 *   moe_route_capacity   moe_route with the limit: counts[e] = kept
 *                        assignments (<= C), offsets their exclusive scan,
 *                        perm_token[0 .. offsets[n]) the kept rows, and
 *                        slot_pos[t][k] = -1 for a dropped assignment.
 *                        topk_idx / topk_w are those of moe_route.
 *   moe_forward_capacity moe_forward with the limit.
 * A capacity of at least the largest expert load gives moe_route / moe_forward
 * exactly.  Invalid capacity_factor -> MOE_ERR_INVALID_ARG.
 */
int64_t moe_expert_capacity(int64_t T, int32_t n, int32_t K, double capacity_factor);

moe_status_t moe_route_capacity(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n,
                                int32_t K, double capacity_factor, int32_t* topk_idx, float* topk_w,
                                int32_t* counts, int32_t* offsets, int32_t* perm_token,
                                int32_t* slot_pos, moe_stream_t stream);

moe_status_t moe_forward_capacity(const void* x, const void* Wg, const void* W1, const void* W3,
                                  const void* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                                  int32_t K, double capacity_factor, float* y, moe_stream_t stream);

/*
 * Expert-choice routing: the second routing method of "How Experts Are Chosen
 * (Routing Methods)" in "Mixtral of Experts? Mixture of Experts? Try to
 * explain Mixtral 8x7B": instead of tokens choosing experts, each expert
 * chooses the tokens it processes, with a fixed capacity.  Reading used here:
 * the score of (t, e) is the router's probability S[t][e] (softmax of the
 * token's n logits, fp32); expert e takes the C = min(T, ceil(cf * T / n))
 * tokens with the largest S[t][e] (ties to the lower token index); a chosen
 * pair adds S[t][e] * SwiGLU_e(x_t) to y_t, so a token may use 0 .. n experts
 * and one that no expert chose gets y = 0.  With cf = K the experts do the
 * same work as top-K token choice.
 *   moe_expert_choice_capacity  returns C (0 if invalid).
 *   moe_route_expert_choice     scores[T][n] fp32 (S), perm_token[n*C] int32
 *                               (rows e*C .. e*C+C-1: expert e's tokens,
 *                               ascending), slot_pos[T][n] int32 (row of (t, e)
 *                               or -1); each optional, at least one given.
 *   moe_forward_expert_choice   the layer (bf16 inputs, fp32 y).
 * Limits as moe_forward, plus T*n < 2^31; invalid capacity_factor ->
 * MOE_ERR_INVALID_ARG.
 */
int64_t moe_expert_choice_capacity(int64_t T, int32_t n, double capacity_factor);

moe_status_t moe_route_expert_choice(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n,
                                     double capacity_factor, float* scores, int32_t* perm_token,
                                     int32_t* slot_pos, moe_stream_t stream);

moe_status_t moe_forward_expert_choice(const void* x, const void* Wg, const void* W1, const void* W3,
                                       const void* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                                       double capacity_factor, float* y, moe_stream_t stream);

/*
 * 4-bit expert weights.  The explainer sizes the model at 16 and at 4 bits per
 * parameter ("Why total and active both matter", Part 4 of "Mixture of
 * Experts: Why Mixtral Only Wakes Up Two Specialists") but gives no format;
 * this library's format, for a weight stack W[n][R][C] (R = reduction index):
 *   scales [n][R/128][C] bf16: s = bf16_rne(max |W| over 128 consecutive r of
 *           a column / 7), computed in fp32;
 *   codes   n*R*C/2 bytes: q = clamp(rint(W / s), -7, 7) (fp32 division, q = 0
 *           where s = 0), nibble q + 8; per expert, by group b = r/128, then
 *           column tile c/16, then chunk g = (r%128)/32, then column c%16,
 *           16 bytes = 4 little-endian words, word m holding
 *           r = 128b + 32g + 8m + i with element i = 2t in bits 4t..4t+3 and
 *           element 2t+1 in bits 16+4t..16+4t+3 (a 16-column tile of a group
 *           is one contiguous kilobyte).
 * The dequantised weight is q * s.
 *
 * moe_quantize_q4 -- W bf16 [n][R][C] (R % 128 == 0, C % 16 == 0; W and codes
 *   16-byte aligned) -> codes, scales.  Deterministic, bit-exact to the format.
 * moe_forward_q4  -- the layer with 4-bit W1, W3 (R = d, C = f) and W2 (R = f,
 *   C = d) given as (codes, scales) pairs; x, Wg bf16, y fp32.  Needs d % 128
 *   == 0 and f % 128 == 0.  Routing, SwiGLU, bf16 rounding of h and the
 *   combine are as in moe_forward; every projection uses the weight-streaming
 *   kernels, which suit decode batches (a few rows per expert) - larger
 *   batches are correct but re-stream the weights per 16 rows of an expert.
 */
moe_status_t moe_quantize_q4(const void* W, int32_t n, int64_t R, int64_t C, void* codes, void* scales,
                             moe_stream_t stream);

moe_status_t moe_forward_q4(const void* x, const void* Wg, const void* W1q, const void* W1s,
                            const void* W3q, const void* W3s, const void* W2q, const void* W2s,
                            int64_t T, int64_t d, int64_t f, int32_t n, int32_t K, float* y,
                            moe_stream_t stream);

/*
 * moe_check_dispatch -- checks routing arrays on the device against the
 * definition of the dispatch (moe_route above): counts[e] = offsets[e+1] -
 * offsets[e] <= capacity, offsets[0] = 0, offsets[n] = T*K without a capacity;
 * every expert index in [0, n) and distinct within its token; every kept
 * assignment (t, k) at a position slot_pos[t][k] inside its expert's segment
 * with perm_token[slot_pos[t][k]] = t; every position owned by exactly such an
 * assignment; tokens ascending within each segment.  capacity = 0: dropless
 * (slot_pos = -1 is then an error); capacity > 0: moe_route_capacity's arrays,
 * where -1 marks a dropped assignment.  All arrays are device int32 in the
 * layouts of moe_route.  The call waits for the verdict on `stream` (it
 * synchronises that stream): MOE_OK, or MOE_ERR_VALIDATION with the failed
 * properties and the first offending index in moe_last_error().
 * With MOE_VALIDATE=1 in the environment, moe_route, moe_route_capacity and
 * every bf16 forward entry point run the same check after routing (and so
 * synchronise their stream; not for use under graph capture).
 */
moe_status_t moe_check_dispatch(const int32_t* topk_idx, const int32_t* counts, const int32_t* offsets,
                                const int32_t* perm_token, const int32_t* slot_pos, int64_t T, int32_t n, int32_t K,
                                int64_t capacity, moe_stream_t stream);

/* Bytes of library workspace a call of this shape needs on any supported
 * device, for every entry point that takes (T, d, f, n, K) (an upper bound:
 * the prefill path's leftover-tile buffer scales with the device's compute
 * units per XCD).  For the expert-choice entry points pass K = n (K may
 * exceed the per-call limit of 8 here).  0 on invalid shapes. */
size_t moe_workspace_bytes(int64_t T, int64_t d, int64_t f, int32_t n, int32_t K);

/* Frees the workspace of every device (synchronises each device first). */
moe_status_t moe_release(void);

/* Static text for a status code. */
const char* moe_status_string(moe_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
