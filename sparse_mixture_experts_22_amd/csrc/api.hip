// C ABI of the sparse MoE layer: argument validation, the per-device
// workspace, and the launch sequence on the caller's stream.
//
//   route:   router (+top-K, softmax, block histograms) -> scatter
//   forward: route -> expert up projection (SwiGLU) -> down projection -> combine
//
// The host never reads device data back: all scheduling decisions that depend
// on the routing (which tiles exist, which rows they hold) are taken on the
// device from `offsets`.  The only host-side choice is between the tiled
// grouped GEMM and the weight-streaming kernels, made from the shape alone.
#include <mutex>
#include <string>
#include <vector>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <utility>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr int kMaxDevices = 64;
struct DeviceWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  int cus_per_xcd = 0;  // compute units per XCD, queried on first use
  // Outgrown workspaces: a HIP graph captured over an earlier call still
  // addresses them, so they stay allocated until moe_release.
  std::vector<void*> retired;
  char* scratch = nullptr;  // this device's address of `scratch` (below)
};
std::mutex g_ws_mutex;
DeviceWorkspace g_ws[kMaxDevices];

}  // namespace

// Fixed scratch of moe_forward_noalloc: one copy per device, held until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in symbol): it takes the device address from
// hipGetSymbolAddress once per device and passes that.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

enum class Path { kRouteOnly, kStats, kBf16, kPacked, kF32 };

struct Plan {
  size_t topk_idx = 0, topk_w = 0, hist = 0, bases = 0, wgT = 0, counts = 0, offsets = 0,
         perm_token = 0, slot_pos = 0;
  size_t h = 0, o = 0, tail = 0, probsum = 0, verr = 0, sched = 0, total = 0;
  bool skinny = false;
  int splits = 1;
};

// `rows`: expert rows of the projections (T*K unless given).
Plan make_plan(int64_t T, int64_t d, int64_t f, int n, int K, Path path, int cus_per_xcd = 0,
               bool force_skinny = false, int64_t rows = -1) {
  Plan p;
  const int64_t TK = T * K;
  const int64_t R = rows >= 0 ? rows : TK;
  const int BT = moe::route_block_tokens(n);
  const int64_t nb = (T + BT - 1) / BT;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.topk_idx = take((size_t)TK * 4);
  p.topk_w = take((size_t)TK * 4);
  p.hist = take((size_t)nb * n * 4);
  p.bases = take((size_t)nb * n * 4);
  p.wgT = take((size_t)moe::route_padded_experts(n) * d * 2);
  p.counts = take((size_t)n * 4);
  p.offsets = take((size_t)(n + 1) * 4);
  p.perm_token = take((size_t)TK * 4);
  p.slot_pos = take((size_t)TK * 4);
  p.verr = take(8);
  if (path == Path::kStats) p.probsum = take((size_t)nb * n * 4);
  if (path == Path::kBf16 || path == Path::kPacked) {
    p.skinny = force_skinny || R <= (int64_t)moe::kSkinnyMaxAvgRows * n;
    if (path == Path::kPacked)  // cus_per_xcd == 0 (a size query): the largest split count
      p.splits = p.skinny ? (cus_per_xcd > 0 ? moe::packed_stream_splits(n, (int)f, (int)d, cus_per_xcd) : 8) : 1;
    else
      p.splits = p.skinny ? moe::kSkinnyDownSplits : 1;
    p.h = take((size_t)R * f * 2);
    p.o = take((size_t)p.splits * R * d * 4);
    if (!p.skinny && cus_per_xcd >= 1 && cus_per_xcd <= 64) p.tail = take(moe::prefill_tail_bytes(cus_per_xcd));
    if (path == Path::kPacked && !p.skinny) p.sched = take((size_t)moe::kPackedSchedWords * 4);
  } else if (path == Path::kF32) {
    p.h = take((size_t)TK * f * 4);
    p.o = take((size_t)TK * d * 4);
  }
  p.total = off;
  return p;
}

// Validation shared by every entry point; nothing here touches the GPU.
moe_status_t check_shape(int64_t T, int64_t d, int64_t f, int32_t n, int32_t K, bool need_f) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  if (d < 1) return fail(MOE_ERR_INVALID_ARG, "d must be >= 1");
  if (need_f && f < 1) return fail(MOE_ERR_INVALID_ARG, "f must be >= 1");
  if (n < 1) return fail(MOE_ERR_INVALID_ARG, "n must be >= 1");
  if (K < 1 || K > n) return fail(MOE_ERR_INVALID_ARG, "K must satisfy 1 <= K <= n");
  if (n > moe::kMaxN) return fail(MOE_ERR_UNSUPPORTED, "n > 256 experts is not supported");
  if (K > moe::kMaxK) return fail(MOE_ERR_UNSUPPORTED, "K > 8 is not supported");
  if (T * (int64_t)K > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "T*K must be < 2^31");
  if (d > INT32_MAX || f > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "d and f must be < 2^31");
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status_t check_bf16(int64_t d, int64_t f, bool need_f, std::initializer_list<const void*> ptrs) {
  if (d % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs d % 64 == 0");
  if (need_f && f % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs f % 64 == 0");
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensors");
  return MOE_OK;
}

moe_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// MOE_VALIDATE=1 in the environment: every routing is followed by the
// dispatch checks on the device, and the call waits for their verdict.
bool validate_enabled() {
  const char* v = std::getenv("MOE_VALIDATE");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

moe_status_t validation_verdict(const int* topk_idx, const int* counts, const int* offsets, const int* perm_token,
                                const int* slot_pos, int64_t T, int n, int K, int cap, int* err, hipStream_t stream) {
  hipError_t e = moe::launch_validate(topk_idx, counts, offsets, perm_token, slot_pos, T, n, K, cap, err, stream);
  if (e != hipSuccess) return hip_fail(e, "validation kernel launch");
  int host[2] = {0, 0};
  e = hipMemcpyAsync(host, err, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "validation read-back");
  if (host[0] == 0) return MOE_OK;
  std::string what;
  const std::pair<int, const char*> names[] = {
      {moe::kValidateOffsets, "counts/offsets"}, {moe::kValidateTotal, "total assignments"},
      {moe::kValidateIndex, "expert index"}, {moe::kValidateSlot, "slot_pos segment"},
      {moe::kValidatePerm, "perm_token/slot_pos back-pointer"}, {moe::kValidateOrder, "token order in a segment"}};
  for (const auto& nm : names)
    if (host[0] & nm.first) what += std::string(what.empty() ? "" : ", ") + nm.second;
  return fail(MOE_ERR_VALIDATION, "dispatch check failed (" + what + "), first at index " + std::to_string(host[1]));
}

// Returns the current device's workspace, grown to at least `bytes`.
moe_status_t get_workspace(size_t bytes, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace& ws = g_ws[dev];
  if (ws.bytes < bytes) {
    // Grow at least 2x, so the outgrown buffers kept alive (retired) total
    // less than the live one.  Nothing is freed here: work already enqueued,
    // or a graph captured over an earlier call, may still use the old buffer.
    const size_t want = std::max(bytes, 2 * ws.bytes);
    void* p = nullptr;
    e = hipMalloc(&p, want);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MOE_ERR_NO_MEMORY, std::string("hipMalloc of workspace failed: ") + hipGetErrorString(e));
    }
    if (ws.ptr != nullptr) ws.retired.push_back(ws.ptr);
    ws.ptr = p;
    ws.bytes = want;
  }
  *out = static_cast<char*>(ws.ptr);
  return MOE_OK;
}

// Device address of the current device's fixed scratch, looked up once per
// device (with that device current) and kept.
moe_status_t get_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace& ws = g_ws[dev];
  if (ws.scratch == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    ws.scratch = static_cast<char*>(p);
  }
  *out = ws.scratch;
  return MOE_OK;
}

// Compute units per XCD of the current device (the tile scheduler assumes 8
// XCDs, the layout of the CDNA4 parts), queried once per device.
moe_status_t cus_per_xcd(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace& ws = g_ws[dev];
  if (ws.cus_per_xcd == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    ws.cus_per_xcd = cus >= 8 ? cus / 8 : 1;
  }
  *out = ws.cus_per_xcd;
  return MOE_OK;
}

#define MOE_LAUNCH(call, what)                  \
  do {                                          \
    hipError_t err_ = (call);                   \
    if (err_ != hipSuccess) return hip_fail(err_, what); \
  } while (0)

template <typename T>
T* at(char* base, size_t off) {
  return reinterpret_cast<T*>(base + off);
}

struct RouteOut {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_token;
  int32_t* slot_pos;
};

moe::RouteBuffers route_buffers(char* ws, const Plan& p, const RouteOut& user) {
  moe::RouteBuffers r;
  r.topk_idx = user.topk_idx ? user.topk_idx : at<int32_t>(ws, p.topk_idx);
  r.topk_w = user.topk_w ? user.topk_w : at<float>(ws, p.topk_w);
  r.counts = user.counts ? user.counts : at<int32_t>(ws, p.counts);
  r.offsets = user.offsets ? user.offsets : at<int32_t>(ws, p.offsets);
  r.perm_token = user.perm_token ? user.perm_token : at<int32_t>(ws, p.perm_token);
  r.slot_pos = user.slot_pos ? user.slot_pos : at<int32_t>(ws, p.slot_pos);
  r.hist = at<int>(ws, p.hist);
  r.bases = at<int>(ws, p.bases);
  r.wgT = at<uint16_t>(ws, p.wgT);
  r.split = at<float>(ws, p.wgT);  // the transposed copy is unused where the split router runs
  return r;
}

template <bool BF16>
moe_status_t route_impl(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n, int32_t K,
                        const RouteOut& user, hipStream_t stream, int cap = INT32_MAX) {
  moe_status_t st = check_shape(T, d, 1, n, K, false);
  if (st != MOE_OK) return st;
  if ((!x && T > 0) || !Wg) return fail(MOE_ERR_INVALID_ARG, "x and Wg must be non-null");
  if (T > 0 && !user.topk_idx && !user.topk_w && !user.counts && !user.offsets && !user.perm_token &&
      !user.slot_pos)
    return fail(MOE_ERR_INVALID_ARG, "at least one routing output must be non-null");
  if (BF16) {
    st = check_bf16(d, 0, false, {x, Wg});
    if (st != MOE_OK) return st;
  }
  if (T == 0) return MOE_OK;  // nothing is written
  const Plan p = make_plan(T, d, 0, n, K, Path::kRouteOnly);
  char* ws = nullptr;
  st = get_workspace(p.total, &ws);
  if (st != MOE_OK) return st;
  const moe::RouteBuffers r = route_buffers(ws, p, user);
  if (BF16)
    MOE_LAUNCH(moe::launch_route_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wg),
                                      T, d, n, K, r, stream, nullptr, cap),
               "routing kernel launch");
  else
    MOE_LAUNCH(moe::launch_route_f32(static_cast<const float*>(x), static_cast<const float*>(Wg), T, d, n,
                                     K, r, stream),
               "routing kernel launch");
  if (validate_enabled())
    return validation_verdict(r.topk_idx, r.counts, r.offsets, r.perm_token, r.slot_pos, T, n, K, cap,
                              at<int>(ws, p.verr), stream);
  return MOE_OK;
}

// x and y hold T rows: with T == 0 they may be null (an empty array).
moe_status_t check_forward_ptrs(int64_t T, const void* x, const void* Wg, const void* W1, const void* W3,
                                const void* W2, const void* y) {
  if (!Wg || !W1 || !W3 || !W2 || (T > 0 && (!x || !y)))
    return fail(MOE_ERR_INVALID_ARG, "x, Wg, W1, W3, W2 and y must be non-null");
  return MOE_OK;
}

}  // namespace

namespace {

// `fixed`: run in the fixed scratch instead of the growable workspace (no
// allocation; the tiled path then runs every down-projection tile whole).
// `packed`: W1 is the packed up pair (moe_pack_up), W3 is unused, W2 the packed
// down stack (moe_pack_down).
moe_status_t forward_bf16(const void* x, const void* Wg, const void* W1, const void* W3, const void* W2,
                          int64_t T, int64_t d, int64_t f, int32_t n, int32_t K, float* y,
                          hipStream_t stream, void* const* ev, int cap = INT32_MAX, bool fixed = false,
                          bool packed = false) {
  g_last_error.clear();
  moe_status_t st = check_shape(T, d, f, n, K, true);
  if (st != MOE_OK) return st;
  st = check_forward_ptrs(T, x, Wg, W1, packed ? W1 : W3, W2, y);
  if (st != MOE_OK) return st;
  st = check_bf16(d, f, true, {x, Wg, W1, packed ? W1 : W3, W2, y});
  if (st != MOE_OK) return st;
  if (packed && (d % 256 != 0 || f % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "packed weights need d % 256 == 0 and f % 128 == 0");
  if (ev != nullptr)
    for (int i = 0; i < 6; ++i)
      if (ev[i] == nullptr) return fail(MOE_ERR_INVALID_ARG, "stage_events must hold 6 events");
  if (T == 0) return MOE_OK;
  int cus = 0;
  st = cus_per_xcd(&cus);
  if (st != MOE_OK) return st;
  const Plan p = packed ? make_plan(T, d, f, n, K, Path::kPacked, cus)
                        : make_plan(T, d, f, n, K, Path::kBf16, fixed ? 0 : cus);
  char* ws = nullptr;
  if (fixed) {
    if (p.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ERR_UNSUPPORTED, "this shape needs " + std::to_string(p.total) +
                                           " bytes of scratch; the fixed scratch holds " +
                                           std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES));
    st = get_scratch(&ws);
  } else {
    st = get_workspace(p.total, &ws);
  }
  if (st != MOE_OK) return st;
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), stream) : hipSuccess;
  };
  moe::RouteBuffers r = route_buffers(ws, p, RouteOut{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr});
  int* sched = nullptr;
  if (packed && !p.skinny) {
    if (cus < 1 || cus > 64) return fail(MOE_ERR_UNSUPPORTED, "packed tiled path needs 1..64 compute units per XCD");
    sched = at<int>(ws, p.sched);
    r.zero = sched;  // the router clears the work counters of the two projections
    r.n_zero = moe::kPackedCounterWords;
  }
  uint16_t* h = at<uint16_t>(ws, p.h);
  float* o = at<float>(ws, p.o);
  const auto* xb = static_cast<const uint16_t*>(x);
  const int64_t TK = T * K;
  MOE_LAUNCH(mark(0), "hipEventRecord");
  MOE_LAUNCH(moe::launch_route_bf16(xb, static_cast<const uint16_t*>(Wg), T, d, n, K, r, stream,
                                    ev ? static_cast<hipEvent_t>(ev[1]) : nullptr, cap),
             "routing kernel launch");
  if (validate_enabled()) {
    st = validation_verdict(r.topk_idx, r.counts, r.offsets, r.perm_token, r.slot_pos, T, n, K, cap,
                            at<int>(ws, p.verr), stream);
    if (st != MOE_OK) return st;
  }
  MOE_LAUNCH(mark(2), "hipEventRecord");
  const auto* w1 = static_cast<const uint16_t*>(W1);
  const auto* w3 = static_cast<const uint16_t*>(W3);
  const auto* w2 = static_cast<const uint16_t*>(W2);
  if (packed && p.skinny) {
    MOE_LAUNCH(moe::launch_packed_stream_up(xb, T, r.perm_token, w1, r.offsets, TK, n, (int)d, (int)f, h, stream),
               "up-projection kernel launch");
    MOE_LAUNCH(mark(3), "hipEventRecord");
    MOE_LAUNCH(moe::launch_packed_stream_down(h, w2, r.offsets, TK, n, (int)f, (int)d, p.splits, o, stream),
               "down-projection kernel launch");
  } else if (packed) {
    MOE_LAUNCH(moe::launch_packed_up(xb, T, r.perm_token, w1, r.offsets, TK, n, (int)d, (int)f, cus, sched, h, stream),
               "up-projection kernel launch");
    MOE_LAUNCH(mark(3), "hipEventRecord");
    float* tail = p.tail ? at<float>(ws, p.tail) : nullptr;
    MOE_LAUNCH(moe::launch_packed_down(h, w2, r.offsets, TK, n, (int)f, (int)d, cus, sched, tail, o, stream),
               "down-projection kernel launch");
  } else if (p.skinny) {
    MOE_LAUNCH(moe::launch_skinny_up(xb, T, r.perm_token, w1, w3, r.offsets, TK, n, (int)d, (int)f, h, stream),
               "up-projection kernel launch");
    MOE_LAUNCH(mark(3), "hipEventRecord");
    MOE_LAUNCH(moe::launch_skinny_down(h, w2, r.offsets, TK, n, (int)f, (int)d, p.splits, o, stream),
               "down-projection kernel launch");
  } else {
    MOE_LAUNCH(moe::launch_prefill_up(xb, T, r.perm_token, w1, w3, r.offsets, TK, n, (int)d, (int)f, cus,
                                      h, stream),
               "up-projection kernel launch");
    MOE_LAUNCH(mark(3), "hipEventRecord");
    float* tail = p.tail ? at<float>(ws, p.tail) : nullptr;
    MOE_LAUNCH(moe::launch_prefill_down(h, w2, r.offsets, TK, n, (int)f, (int)d, cus, tail, o, stream),
               "down-projection kernel launch");
  }
  MOE_LAUNCH(mark(4), "hipEventRecord");
  MOE_LAUNCH(moe::launch_combine(o, p.splits, TK, r.topk_w, r.slot_pos, T, d, K, y, stream),
             "combine kernel launch");
  MOE_LAUNCH(mark(5), "hipEventRecord");
  return MOE_OK;
}

template <bool BF16>
moe_status_t route_stats_impl(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n, int32_t K,
                              float alpha, float* frac, float* prob, float* aux_loss, hipStream_t stream) {
  g_last_error.clear();
  moe_status_t st = check_shape(T, d, 1, n, K, false);
  if (st != MOE_OK) return st;
  if (!x || !Wg) return fail(MOE_ERR_INVALID_ARG, "x and Wg must be non-null");
  if (!frac && !prob && !aux_loss) return fail(MOE_ERR_INVALID_ARG, "at least one statistics output must be non-null");
  if (!(alpha == alpha)) return fail(MOE_ERR_INVALID_ARG, "alpha must not be NaN");
  if (T == 0) return fail(MOE_ERR_INVALID_ARG, "router statistics need T >= 1");
  if (BF16) {
    st = check_bf16(d, 0, false, {x, Wg});
    if (st != MOE_OK) return st;
  }
  const Plan p = make_plan(T, d, 0, n, K, Path::kStats);
  char* ws = nullptr;
  st = get_workspace(p.total, &ws);
  if (st != MOE_OK) return st;
  const moe::RouteBuffers r =
      route_buffers(ws, p, RouteOut{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr});
  float* probsum = at<float>(ws, p.probsum);
  if (BF16)
    MOE_LAUNCH(moe::launch_route_stats_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wg),
                                            T, d, n, K, alpha, r, probsum, frac, prob, aux_loss, stream),
               "router statistics launch");
  else
    MOE_LAUNCH(moe::launch_route_stats_f32(static_cast<const float*>(x), static_cast<const float*>(Wg), T, d,
                                           n, K, alpha, r, probsum, frac, prob, aux_loss, stream),
               "router statistics launch");
  return MOE_OK;
}

moe_status_t forward_q4(const void* x, const void* Wg, const void* W1q, const void* W1s, const void* W3q,
                        const void* W3s, const void* W2q, const void* W2s, int64_t T, int64_t d, int64_t f,
                        int32_t n, int32_t K, float* y, hipStream_t stream) {
  g_last_error.clear();
  moe_status_t st = check_shape(T, d, f, n, K, true);
  if (st != MOE_OK) return st;
  if (!Wg || !W1q || !W1s || !W3q || !W3s || !W2q || !W2s || (T > 0 && (!x || !y)))
    return fail(MOE_ERR_INVALID_ARG, "null tensor pointer");
  if (d % 128 != 0 || f % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "4-bit path needs d % 128 == 0 and f % 128 == 0");
  st = check_bf16(d, f, true, {x, Wg, W1q, W3q, W2q, y});
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  int cus = 0;
  st = cus_per_xcd(&cus);
  if (st != MOE_OK) return st;
  const Plan p = make_plan(T, d, f, n, K, Path::kBf16, 0, true);
  char* ws = nullptr;
  st = get_workspace(p.total, &ws);
  if (st != MOE_OK) return st;
  const moe::RouteBuffers r =
      route_buffers(ws, p, RouteOut{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr});
  uint16_t* h = at<uint16_t>(ws, p.h);
  float* o = at<float>(ws, p.o);
  const auto* xb = static_cast<const uint16_t*>(x);
  const int64_t TK = T * K;
  MOE_LAUNCH(moe::launch_route_bf16(xb, static_cast<const uint16_t*>(Wg), T, d, n, K, r, stream),
             "routing kernel launch");
  MOE_LAUNCH(moe::launch_q4_up(xb, T, r.perm_token, static_cast<const uint8_t*>(W1q),
                               static_cast<const uint16_t*>(W1s), static_cast<const uint8_t*>(W3q),
                               static_cast<const uint16_t*>(W3s), r.offsets, TK, n, (int)d, (int)f, 8 * cus, h,
                               stream),
             "up-projection kernel launch");
  MOE_LAUNCH(moe::launch_q4_down(h, static_cast<const uint8_t*>(W2q), static_cast<const uint16_t*>(W2s),
                                 r.offsets, TK, n, (int)f, (int)d, p.splits, 8 * cus, o, stream),
             "down-projection kernel launch");
  MOE_LAUNCH(moe::launch_combine(o, p.splits, TK, r.topk_w, r.slot_pos, T, d, K, y, stream),
             "combine kernel launch");
  return MOE_OK;
}

// Tokens per expert of expert-choice routing, min(T, ceil(cf * T / n)), or -1.
int64_t ec_capacity_of(int64_t T, int32_t n, double cf) {
  if (!(cf > 0.0) || !std::isfinite(cf) || n < 1 || T < 1) return -1;
  const double c = std::ceil(cf * (double)T / (double)n);
  if (c > (double)INT32_MAX) return -1;
  return std::min<int64_t>(T, (int64_t)c);
}

moe_status_t check_ec(int64_t T, int64_t d, int64_t f, int32_t n, bool need_f, double cf, int64_t* C) {
  moe_status_t st = check_shape(T, d, f, n, 1, need_f);
  if (st != MOE_OK) return st;
  if (T * (int64_t)n > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "T*n must be < 2^31");
  if (T == 0) {
    *C = 0;
    return MOE_OK;
  }
  *C = ec_capacity_of(T, n, cf);
  if (*C < 1) return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be positive and finite");
  return MOE_OK;
}

// Expert capacity ceil(cf * T * K / n), or -1 if cf is not a positive finite
// number or the capacity does not fit an int.
int64_t capacity_of(int64_t T, int32_t n, int32_t K, double cf) {
  if (!(cf > 0.0) || !std::isfinite(cf) || n < 1 || K < 1 || T < 0) return -1;
  const double c = std::ceil(cf * (double)T * (double)K / (double)n);
  if (c > (double)INT32_MAX) return -1;
  return (int64_t)c;
}

}  // namespace

#ifdef MOE_TILE_TRACE
#include "moe_tile_trace.h"
namespace moe {
hipError_t tile_trace_read(long long* host);
hipError_t tile_trace_clear();
}
static_assert(MOE_TILE_TRACE_WGS == moe::kTileTraceWgs && MOE_TILE_TRACE_TILES == moe::kTileTraceTiles &&
                  MOE_TILE_TRACE_FIELDS == moe::kTileTraceFields,
              "trace layout");
extern "C" int moe_tile_trace_read(long long* host) {
  return host ? (int)moe::tile_trace_read(host) : (int)hipErrorInvalidValue;
}
extern "C" int moe_tile_trace_clear(void) { return (int)moe::tile_trace_clear(); }
#endif

extern "C" {

moe_status_t moe_forward(const void* x, const void* Wg, const void* W1, const void* W3, const void* W2,
                         int64_t T, int64_t d, int64_t f, int32_t n, int32_t K, float* y,
                         moe_stream_t stream) {
  return forward_bf16(x, Wg, W1, W3, W2, T, d, f, n, K, y, reinterpret_cast<hipStream_t>(stream),
                      nullptr);
}

moe_status_t moe_pack_up(const void* W1, const void* W3, int32_t n, int64_t d, int64_t f, void* W13p,
                         moe_stream_t stream) {
  g_last_error.clear();
  if (!W1 || !W3 || !W13p) return fail(MOE_ERR_INVALID_ARG, "null tensor pointer");
  if (n < 1 || d < 1 || f < 1) return fail(MOE_ERR_INVALID_ARG, "n, d and f must be >= 1");
  if (n > moe::kMaxN) return fail(MOE_ERR_UNSUPPORTED, "n > 256 experts is not supported");
  if (d % 256 != 0 || f % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "packed weights need d % 256 == 0 and f % 128 == 0");
  if (d > INT32_MAX || f > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "d and f must be < 2^31");
  if (!aligned16(W1) || !aligned16(W3) || !aligned16(W13p))
    return fail(MOE_ERR_UNSUPPORTED, "packed weights need 16-byte aligned tensors");
  MOE_LAUNCH(moe::launch_pack(1, static_cast<const uint16_t*>(W1), static_cast<const uint16_t*>(W3), n, (int)d,
                              (int)f, static_cast<uint16_t*>(W13p), reinterpret_cast<hipStream_t>(stream)),
             "pack kernel launch");
  return MOE_OK;
}

moe_status_t moe_pack_down(const void* W2, int32_t n, int64_t f, int64_t d, void* W2p, moe_stream_t stream) {
  g_last_error.clear();
  if (!W2 || !W2p) return fail(MOE_ERR_INVALID_ARG, "null tensor pointer");
  if (n < 1 || d < 1 || f < 1) return fail(MOE_ERR_INVALID_ARG, "n, d and f must be >= 1");
  if (n > moe::kMaxN) return fail(MOE_ERR_UNSUPPORTED, "n > 256 experts is not supported");
  if (d % 256 != 0 || f % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "packed weights need d % 256 == 0 and f % 128 == 0");
  if (d > INT32_MAX || f > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "d and f must be < 2^31");
  if (!aligned16(W2) || !aligned16(W2p)) return fail(MOE_ERR_UNSUPPORTED, "packed weights need 16-byte aligned tensors");
  MOE_LAUNCH(moe::launch_pack(2, static_cast<const uint16_t*>(W2), nullptr, n, (int)f, (int)d,
                              static_cast<uint16_t*>(W2p), reinterpret_cast<hipStream_t>(stream)),
             "pack kernel launch");
  return MOE_OK;
}

moe_status_t moe_forward_packed(const void* x, const void* Wg, const void* W13p, const void* W2p, int64_t T,
                                int64_t d, int64_t f, int32_t n, int32_t K, float* y, moe_stream_t stream) {
  return forward_bf16(x, Wg, W13p, nullptr, W2p, T, d, f, n, K, y, reinterpret_cast<hipStream_t>(stream), nullptr,
                      INT32_MAX, false, true);
}

moe_status_t moe_forward_packed_traced(const void* x, const void* Wg, const void* W13p, const void* W2p, int64_t T,
                                       int64_t d, int64_t f, int32_t n, int32_t K, float* y, moe_stream_t stream,
                                       void* const* stage_events) {
  if (stage_events == nullptr) return fail(MOE_ERR_INVALID_ARG, "stage_events must be non-null");
  return forward_bf16(x, Wg, W13p, nullptr, W2p, T, d, f, n, K, y, reinterpret_cast<hipStream_t>(stream),
                      stage_events, INT32_MAX, false, true);
}

moe_status_t moe_check_dispatch(const int32_t* topk_idx, const int32_t* counts, const int32_t* offsets,
                                const int32_t* perm_token, const int32_t* slot_pos, int64_t T, int32_t n, int32_t K,
                                int64_t capacity, moe_stream_t stream) {
  g_last_error.clear();
  moe_status_t st = check_shape(T, 1, 1, n, K, false);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || (T > 0 && (!topk_idx || !perm_token || !slot_pos)))
    return fail(MOE_ERR_INVALID_ARG, "null routing array");
  if (capacity < 0 || capacity > INT32_MAX) return fail(MOE_ERR_INVALID_ARG, "capacity must be in [0, 2^31)");
  char* ws = nullptr;
  st = get_workspace(256, &ws);
  if (st != MOE_OK) return st;
  return validation_verdict(topk_idx, counts, offsets, perm_token, slot_pos, T, n, K,
                            capacity == 0 ? INT32_MAX : (int)capacity, reinterpret_cast<int*>(ws),
                            reinterpret_cast<hipStream_t>(stream));
}

moe_status_t moe_forward_noalloc(const void* x, const void* Wg, const void* W1, const void* W3,
                                 const void* W2, int64_t T, int64_t d, int64_t f, int32_t n, int32_t K,
                                 float* y, moe_stream_t stream) {
  return forward_bf16(x, Wg, W1, W3, W2, T, d, f, n, K, y, reinterpret_cast<hipStream_t>(stream), nullptr,
                      INT32_MAX, true);
}

size_t moe_noalloc_scratch_bytes(int64_t T, int64_t d, int64_t f, int32_t n, int32_t K) {
  if (T < 0 || d < 1 || f < 1 || n < 1 || n > moe::kMaxN || K < 1 || K > n || K > moe::kMaxK) return 0;
  if (T * (int64_t)K > INT32_MAX || d > INT32_MAX || f > INT32_MAX) return 0;
  return make_plan(T, d, f, n, K, Path::kBf16, 0).total;
}

moe_status_t moe_forward_traced(const void* x, const void* Wg, const void* W1, const void* W3,
                                const void* W2, int64_t T, int64_t d, int64_t f, int32_t n, int32_t K,
                                float* y, moe_stream_t stream, void* const* stage_events) {
  if (stage_events == nullptr) return fail(MOE_ERR_INVALID_ARG, "stage_events must be non-null");
  return forward_bf16(x, Wg, W1, W3, W2, T, d, f, n, K, y, reinterpret_cast<hipStream_t>(stream),
                      stage_events);
}

moe_status_t moe_forward_f32(const float* x, const float* Wg, const float* W1, const float* W3,
                             const float* W2, int64_t T, int64_t d, int64_t f, int32_t n, int32_t K,
                             float* y, moe_stream_t stream_) {
  g_last_error.clear();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  moe_status_t st = check_shape(T, d, f, n, K, true);
  if (st != MOE_OK) return st;
  st = check_forward_ptrs(T, x, Wg, W1, W3, W2, y);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const Plan p = make_plan(T, d, f, n, K, Path::kF32);
  char* ws = nullptr;
  st = get_workspace(p.total, &ws);
  if (st != MOE_OK) return st;
  const moe::RouteBuffers r =
      route_buffers(ws, p, RouteOut{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr});
  float* h = at<float>(ws, p.h);
  float* o = at<float>(ws, p.o);
  const int64_t TK = T * K;
  MOE_LAUNCH(moe::launch_route_f32(x, Wg, T, d, n, K, r, stream), "routing kernel launch");
  MOE_LAUNCH(moe::launch_f32_up(x, T, r.perm_token, W1, W3, r.offsets, TK, n, (int)d, (int)f, h, stream),
             "up-projection kernel launch");
  MOE_LAUNCH(moe::launch_f32_down(h, W2, r.offsets, TK, n, (int)f, (int)d, o, stream),
             "down-projection kernel launch");
  MOE_LAUNCH(moe::launch_combine(o, 1, TK, r.topk_w, r.slot_pos, T, d, K, y, stream),
             "combine kernel launch");
  return MOE_OK;
}

moe_status_t moe_route(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n, int32_t K,
                       int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                       int32_t* perm_token, int32_t* slot_pos, moe_stream_t stream) {
  g_last_error.clear();
  return route_impl<true>(x, Wg, T, d, n, K,
                          RouteOut{topk_idx, topk_w, counts, offsets, perm_token, slot_pos},
                          reinterpret_cast<hipStream_t>(stream));
}

moe_status_t moe_route_f32(const float* x, const float* Wg, int64_t T, int64_t d, int32_t n, int32_t K,
                           int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                           int32_t* perm_token, int32_t* slot_pos, moe_stream_t stream) {
  g_last_error.clear();
  return route_impl<false>(x, Wg, T, d, n, K,
                           RouteOut{topk_idx, topk_w, counts, offsets, perm_token, slot_pos},
                           reinterpret_cast<hipStream_t>(stream));
}

size_t moe_workspace_bytes(int64_t T, int64_t d, int64_t f, int32_t n, int32_t K) {
  // a size query: K may exceed the per-call limit kMaxK (K = n sizes the
  // expert-choice entry points, whose rows never exceed T*n)
  if (T < 0 || d < 1 || f < 1 || n < 1 || n > moe::kMaxN || K < 1 || K > n) return 0;
  if (T * (int64_t)K > INT32_MAX || d > INT32_MAX || f > INT32_MAX) return 0;
  // the largest of: the tiled plan on the largest device layout the tile
  // scheduler uses (64 CUs per XCD), the weight-streaming plan (4-bit path
  // and few rows per expert), and the fp32 plan
  const Plan a = make_plan(T, d, f, n, K, Path::kBf16, 64);
  const Plan b = make_plan(T, d, f, n, K, Path::kBf16, 0, true);
  const Plan c = make_plan(T, d, f, n, K, Path::kF32);
  const Plan e = make_plan(T, d, f, n, K, Path::kPacked, 64);
  const Plan g = make_plan(T, d, f, n, K, Path::kPacked, 0);
  return std::max(std::max(a.total, std::max(b.total, c.total)), std::max(e.total, g.total));
}

moe_status_t moe_release(void) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) cur = 0;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    DeviceWorkspace& ws = g_ws[dev];
    if (ws.ptr == nullptr) continue;
    hipError_t e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    for (void* old : ws.retired)
      if (e == hipSuccess) e = hipFree(old);
    ws.retired.clear();
    if (e == hipSuccess) e = hipFree(ws.ptr);
    ws.ptr = nullptr;
    ws.bytes = 0;
    if (e != hipSuccess) {
      (void)hipSetDevice(cur);
      return hip_fail(e, "moe_release");
    }
  }
  (void)hipSetDevice(cur);
  return MOE_OK;
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_NO_MEMORY: return "MOE_ERR_NO_MEMORY";
    case MOE_ERR_VALIDATION: return "MOE_ERR_VALIDATION";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1.0 (gfx950)"; }

moe_status_t moe_route_stats(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n, int32_t K,
                             float alpha, float* frac, float* prob, float* aux_loss, moe_stream_t stream) {
  return route_stats_impl<true>(x, Wg, T, d, n, K, alpha, frac, prob, aux_loss,
                                reinterpret_cast<hipStream_t>(stream));
}

moe_status_t moe_route_stats_f32(const float* x, const float* Wg, int64_t T, int64_t d, int32_t n,
                                 int32_t K, float alpha, float* frac, float* prob, float* aux_loss,
                                 moe_stream_t stream) {
  return route_stats_impl<false>(x, Wg, T, d, n, K, alpha, frac, prob, aux_loss,
                                 reinterpret_cast<hipStream_t>(stream));
}

int64_t moe_expert_capacity(int64_t T, int32_t n, int32_t K, double capacity_factor) {
  const int64_t c = capacity_of(T, n, K, capacity_factor);
  return c < 0 ? 0 : c;
}

moe_status_t moe_forward_capacity(const void* x, const void* Wg, const void* W1, const void* W3,
                                  const void* W2, int64_t T, int64_t d, int64_t f, int32_t n, int32_t K,
                                  double capacity_factor, float* y, moe_stream_t stream) {
  g_last_error.clear();
  moe_status_t st = check_shape(T, d, f, n, K, true);
  if (st != MOE_OK) return st;
  const int64_t cap = capacity_of(T, n, K, capacity_factor);
  if (cap < 0) return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be positive and finite");
  return forward_bf16(x, Wg, W1, W3, W2, T, d, f, n, K, y, reinterpret_cast<hipStream_t>(stream), nullptr,
                      (int)cap);
}

moe_status_t moe_route_capacity(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n, int32_t K,
                                double capacity_factor, int32_t* topk_idx, float* topk_w, int32_t* counts,
                                int32_t* offsets, int32_t* perm_token, int32_t* slot_pos,
                                moe_stream_t stream) {
  g_last_error.clear();
  moe_status_t st = check_shape(T, d, 1, n, K, false);
  if (st != MOE_OK) return st;
  const int64_t cap = capacity_of(T, n, K, capacity_factor);
  if (cap < 0) return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be positive and finite");
  return route_impl<true>(x, Wg, T, d, n, K,
                          RouteOut{topk_idx, topk_w, counts, offsets, perm_token, slot_pos},
                          reinterpret_cast<hipStream_t>(stream), (int)cap);
}

moe_status_t moe_quantize_q4(const void* W, int32_t n, int64_t R, int64_t C, void* codes, void* scales,
                             moe_stream_t stream) {
  g_last_error.clear();
  if (!W || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "null tensor pointer");
  if (n < 1 || R < 1 || C < 1) return fail(MOE_ERR_INVALID_ARG, "n, R and C must be >= 1");
  if (R % 128 != 0 || C % 16 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "4-bit format needs R % 128 == 0 and C % 16 == 0");
  if (R > INT32_MAX || C > INT32_MAX || (int64_t)n * R * C / 2 > ((int64_t)1 << 40))
    return fail(MOE_ERR_UNSUPPORTED, "weight stack too large");
  if (!aligned16(W) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 1u) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "W and codes must be 16-byte aligned, scales 2-byte aligned");
  MOE_LAUNCH(moe::launch_quantize_q4(static_cast<const uint16_t*>(W), n, (int)R, (int)C,
                                     static_cast<uint8_t*>(codes), static_cast<uint16_t*>(scales),
                                     reinterpret_cast<hipStream_t>(stream)),
             "quantize kernel launch");
  return MOE_OK;
}

moe_status_t moe_forward_q4(const void* x, const void* Wg, const void* W1q, const void* W1s, const void* W3q,
                            const void* W3s, const void* W2q, const void* W2s, int64_t T, int64_t d,
                            int64_t f, int32_t n, int32_t K, float* y, moe_stream_t stream) {
  return forward_q4(x, Wg, W1q, W1s, W3q, W3s, W2q, W2s, T, d, f, n, K, y,
                    reinterpret_cast<hipStream_t>(stream));
}

int64_t moe_expert_choice_capacity(int64_t T, int32_t n, double capacity_factor) {
  const int64_t c = ec_capacity_of(T, n, capacity_factor);
  return c < 0 ? 0 : c;
}

moe_status_t moe_route_expert_choice(const void* x, const void* Wg, int64_t T, int64_t d, int32_t n,
                                     double capacity_factor, float* scores, int32_t* perm_token,
                                     int32_t* slot_pos, moe_stream_t stream_) {
  g_last_error.clear();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int64_t C = 0;
  moe_status_t st = check_ec(T, d, 1, n, false, capacity_factor, &C);
  if (st != MOE_OK) return st;
  if ((!x && T > 0) || !Wg) return fail(MOE_ERR_INVALID_ARG, "x and Wg must be non-null");
  if (T > 0 && !scores && !perm_token && !slot_pos)
    return fail(MOE_ERR_INVALID_ARG, "at least one output must be non-null");
  st = check_bf16(d, 0, false, {x, Wg});
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const Plan p = make_plan(T, d, 0, n, n, Path::kRouteOnly);
  char* ws = nullptr;
  st = get_workspace(p.total, &ws);
  if (st != MOE_OK) return st;
  const moe::RouteBuffers r = route_buffers(ws, p, RouteOut{nullptr, scores, nullptr, nullptr, perm_token, slot_pos});
  MOE_LAUNCH(moe::launch_route_expert_choice(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wg),
                                             T, d, n, (int)C, r, stream),
             "expert-choice routing launch");
  return MOE_OK;
}

moe_status_t moe_forward_expert_choice(const void* x, const void* Wg, const void* W1, const void* W3,
                                       const void* W2, int64_t T, int64_t d, int64_t f, int32_t n,
                                       double capacity_factor, float* y, moe_stream_t stream_) {
  g_last_error.clear();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int64_t C = 0;
  moe_status_t st = check_ec(T, d, f, n, true, capacity_factor, &C);
  if (st != MOE_OK) return st;
  st = check_forward_ptrs(T, x, Wg, W1, W3, W2, y);
  if (st != MOE_OK) return st;
  st = check_bf16(d, f, true, {x, Wg, W1, W3, W2, y});
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  int cus = 0;
  st = cus_per_xcd(&cus);
  if (st != MOE_OK) return st;
  const int64_t rows = (int64_t)n * C;
  const Plan p = make_plan(T, d, f, n, n, Path::kBf16, cus, false, rows);
  char* ws = nullptr;
  st = get_workspace(p.total, &ws);
  if (st != MOE_OK) return st;
  const moe::RouteBuffers r =
      route_buffers(ws, p, RouteOut{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr});
  uint16_t* h = at<uint16_t>(ws, p.h);
  float* o = at<float>(ws, p.o);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* w1 = static_cast<const uint16_t*>(W1);
  const auto* w3 = static_cast<const uint16_t*>(W3);
  const auto* w2 = static_cast<const uint16_t*>(W2);
  MOE_LAUNCH(moe::launch_route_expert_choice(xb, static_cast<const uint16_t*>(Wg), T, d, n, (int)C, r, stream),
             "expert-choice routing launch");
  if (p.skinny) {
    MOE_LAUNCH(moe::launch_skinny_up(xb, T, r.perm_token, w1, w3, r.offsets, rows, n, (int)d, (int)f, h, stream),
               "up-projection kernel launch");
    MOE_LAUNCH(moe::launch_skinny_down(h, w2, r.offsets, rows, n, (int)f, (int)d, p.splits, o, stream),
               "down-projection kernel launch");
  } else {
    MOE_LAUNCH(moe::launch_prefill_up(xb, T, r.perm_token, w1, w3, r.offsets, rows, n, (int)d, (int)f, cus, h,
                                      stream),
               "up-projection kernel launch");
    float* tail = p.tail ? at<float>(ws, p.tail) : nullptr;
    MOE_LAUNCH(moe::launch_prefill_down(h, w2, r.offsets, rows, n, (int)f, (int)d, cus, tail, o, stream),
               "down-projection kernel launch");
  }
  // combine over the n (token, expert) slots: scores as weights, -1 = not chosen
  MOE_LAUNCH(moe::launch_combine(o, p.splits, rows, r.topk_w, r.slot_pos, T, d, n, y, stream),
             "combine kernel launch");
  return MOE_OK;
}

}  // extern "C"
