"""ctypes binding of include/moe.h.  Same names as the C entry points, minus
the ``moe_`` prefix; tensors are torch CUDA(HIP) tensors, the stream is
torch's current stream unless one is given."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_HIP",
          4: "MOE_ERR_NO_MEMORY", 5: "MOE_ERR_VALIDATION"}

EXPORTS = ["moe_forward", "moe_forward_traced", "moe_forward_noalloc", "moe_noalloc_scratch_bytes",
           "moe_pack_up", "moe_pack_down", "moe_forward_packed", "moe_forward_packed_traced",
           "moe_forward_f32", "moe_route", "moe_route_f32",
           "moe_route_stats", "moe_route_stats_f32", "moe_expert_capacity", "moe_route_capacity",
           "moe_forward_capacity", "moe_quantize_q4", "moe_forward_q4",
           "moe_expert_choice_capacity", "moe_route_expert_choice", "moe_forward_expert_choice",
           "moe_check_dispatch", "moe_workspace_bytes",
           "moe_release", "moe_status_string", "moe_last_error", "moe_version"]


class MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def lib_path() -> str:
    """The in-tree libmoe.so, or the build named by MOE_LIBRARY (for instance the
    host-sanitized build that tests/test_abi_sanitized.py makes)."""
    return os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by __graft_entry__.build()).  Raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    try:
        # bind to the HIP runtime torch already carries, so tensors, streams and
        # events from torch and this library share one runtime instance
        import torch  # noqa: F401
    except ImportError:
        pass
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m sparse_mixture_experts_22_amd.build)")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.moe_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp]
    L.moe_forward.restype = ctypes.c_int
    L.moe_forward_traced.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp]
    L.moe_forward_traced.restype = ctypes.c_int
    L.moe_check_dispatch.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, vp]
    L.moe_check_dispatch.restype = ctypes.c_int
    L.moe_pack_up.argtypes = [vp, vp, i32, i64, i64, vp, vp]
    L.moe_pack_up.restype = ctypes.c_int
    L.moe_pack_down.argtypes = [vp, i32, i64, i64, vp, vp]
    L.moe_pack_down.restype = ctypes.c_int
    L.moe_forward_packed.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp]
    L.moe_forward_packed.restype = ctypes.c_int
    L.moe_forward_packed_traced.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp]
    L.moe_forward_packed_traced.restype = ctypes.c_int
    L.moe_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp]
    L.moe_forward_noalloc.restype = ctypes.c_int
    L.moe_noalloc_scratch_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.moe_forward_f32.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp]
    L.moe_forward_f32.restype = ctypes.c_int
    L.moe_route.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_route.restype = ctypes.c_int
    L.moe_route_f32.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_route_f32.restype = ctypes.c_int
    f32 = ctypes.c_float
    L.moe_route_stats.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp]
    L.moe_route_stats.restype = ctypes.c_int
    L.moe_route_stats_f32.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp]
    L.moe_route_stats_f32.restype = ctypes.c_int
    f64 = ctypes.c_double
    L.moe_expert_capacity.argtypes = [i64, i32, i32, f64]
    L.moe_expert_capacity.restype = i64
    L.moe_route_capacity.argtypes = [vp, vp, i64, i64, i32, i32, f64, vp, vp, vp, vp, vp, vp, vp]
    L.moe_route_capacity.restype = ctypes.c_int
    L.moe_forward_capacity.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, f64, vp, vp]
    L.moe_forward_capacity.restype = ctypes.c_int
    L.moe_quantize_q4.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.moe_quantize_q4.restype = ctypes.c_int
    L.moe_forward_q4.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp]
    L.moe_forward_q4.restype = ctypes.c_int
    L.moe_expert_choice_capacity.argtypes = [i64, i32, f64]
    L.moe_expert_choice_capacity.restype = i64
    L.moe_route_expert_choice.argtypes = [vp, vp, i64, i64, i32, f64, vp, vp, vp, vp]
    L.moe_route_expert_choice.restype = ctypes.c_int
    L.moe_forward_expert_choice.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, f64, vp, vp]
    L.moe_forward_expert_choice.restype = ctypes.c_int
    L.moe_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.moe_workspace_bytes.restype = ctypes.c_size_t
    L.moe_release.argtypes = []
    L.moe_release.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_version.argtypes = []
    L.moe_version.restype = ctypes.c_char_p
    _LIB = L
    return L


def last_error() -> str:
    return lib().moe_last_error().decode()


def version() -> str:
    return lib().moe_version().decode()


def _check(status: int) -> None:
    if status != 0:
        raise MoEError(status, last_error())


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _expect(t, dtype, name, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _forward(fn, dtype, x, Wg, W1, W3, W2, K, y, stream, extra=(), mid=()):
    import torch
    for t, name, nd in ((x, "x", 2), (Wg, "Wg", 2), (W1, "W1", 3), (W3, "W3", 3), (W2, "W2", 3)):
        _expect(t, dtype, name, nd)
    T, d = x.shape
    n = Wg.shape[1]
    f = W1.shape[2]
    if Wg.shape != (d, n) or W1.shape != (n, d, f) or W3.shape != (n, d, f) or W2.shape != (n, f, d):
        raise ValueError("shapes must be x[T][d], Wg[d][n], W1/W3[n][d][f], W2[n][f][d]")
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=x.device)
    else:
        _expect(y, torch.float32, "y", 2)
        if tuple(y.shape) != (T, d):
            raise ValueError("y must be [T][d]")
    _check(fn(_ptr(x), _ptr(Wg), _ptr(W1), _ptr(W3), _ptr(W2), T, d, f, n, int(K), *mid, _ptr(y),
              _stream(stream), *extra))
    return y


def forward(x, Wg, W1, W3, W2, K, y=None, stream=None):
    """moe_forward: bf16 x[T][d], Wg[d][n], W1/W3[n][d][f], W2[n][f][d] -> fp32 y[T][d]."""
    import torch
    return _forward(lib().moe_forward, torch.bfloat16, x, Wg, W1, W3, W2, K, y, stream)


def forward_traced(x, Wg, W1, W3, W2, K, stage_events, y=None, stream=None):
    """moe_forward_traced: as forward(), recording six caller-created hipEvent_t
    handles (integers) between the stages on the stream."""
    import torch
    if len(stage_events) != 6:
        raise ValueError("need 6 events")
    arr = (ctypes.c_void_p * 6)(*stage_events)
    return _forward(lib().moe_forward_traced, torch.bfloat16, x, Wg, W1, W3, W2, K, y, stream,
                    extra=(ctypes.cast(arr, ctypes.c_void_p),))


def forward_noalloc(x, Wg, W1, W3, W2, K, y, stream=None):
    """moe_forward_noalloc: as forward(), with the intermediates in the library's
    fixed scratch (no device allocation by the library).  The caller passes y."""
    import torch
    if y is None:
        raise ValueError("forward_noalloc needs a caller-allocated y")
    return _forward(lib().moe_forward_noalloc, torch.bfloat16, x, Wg, W1, W3, W2, K, y, stream)


def check_dispatch(routing, T, n, K, capacity=0, stream=None):
    """moe_check_dispatch on a dict with the moe_route arrays (topk_idx, counts,
    offsets, perm_token, slot_pos; device int32).  Raises MoEError on a violation."""
    r = routing
    _check(lib().moe_check_dispatch(_ptr(r["topk_idx"]), _ptr(r["counts"]), _ptr(r["offsets"]),
                                    _ptr(r["perm_token"]), _ptr(r["slot_pos"]), T, n, K, int(capacity),
                                    _stream(stream)))


def pack_up(W1, W3, stream=None):
    """moe_pack_up: W1, W3 bf16 [n][d][f] -> the packed up pair, bf16 [n][2*d*f]."""
    import torch
    _expect(W1, torch.bfloat16, "W1", 3)
    _expect(W3, torch.bfloat16, "W3", 3)
    if W1.shape != W3.shape:
        raise ValueError("W1 and W3 must have the same shape")
    n, d, f = W1.shape
    out = torch.empty((n, 2 * d * f), dtype=torch.bfloat16, device=W1.device)
    _check(lib().moe_pack_up(_ptr(W1), _ptr(W3), n, d, f, _ptr(out), _stream(stream)))
    return out


def pack_down(W2, stream=None):
    """moe_pack_down: W2 bf16 [n][f][d] -> the packed down stack, bf16 [n][f*d]."""
    import torch
    _expect(W2, torch.bfloat16, "W2", 3)
    n, f, d = W2.shape
    out = torch.empty((n, f * d), dtype=torch.bfloat16, device=W2.device)
    _check(lib().moe_pack_down(_ptr(W2), n, f, d, _ptr(out), _stream(stream)))
    return out


def _forward_packed(fn, x, Wg, W13p, W2p, f, K, y, stream, extra=()):
    import torch
    for t, name, nd in ((x, "x", 2), (Wg, "Wg", 2), (W13p, "W13p", 2), (W2p, "W2p", 2)):
        _expect(t, torch.bfloat16, name, nd)
    T, d = x.shape
    n = Wg.shape[1]
    if Wg.shape != (d, n) or W13p.shape != (n, 2 * d * f) or W2p.shape != (n, f * d):
        raise ValueError("shapes must be x[T][d], Wg[d][n], W13p[n][2*d*f], W2p[n][f*d]")
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=x.device)
    else:
        _expect(y, torch.float32, "y", 2)
        if tuple(y.shape) != (T, d):
            raise ValueError("y must be [T][d]")
    _check(fn(_ptr(x), _ptr(Wg), _ptr(W13p), _ptr(W2p), T, d, int(f), n, int(K), _ptr(y), _stream(stream), *extra))
    return y


def forward_packed(x, Wg, W13p, W2p, f, K, y=None, stream=None):
    """moe_forward_packed: the layer on weights from pack_up / pack_down (f = FFN size)."""
    return _forward_packed(lib().moe_forward_packed, x, Wg, W13p, W2p, f, K, y, stream)


def forward_packed_traced(x, Wg, W13p, W2p, f, K, stage_events, y=None, stream=None):
    """moe_forward_packed_traced: forward_packed() recording six hipEvent_t handles between stages."""
    if len(stage_events) != 6:
        raise ValueError("need 6 events")
    arr = (ctypes.c_void_p * 6)(*stage_events)
    return _forward_packed(lib().moe_forward_packed_traced, x, Wg, W13p, W2p, f, K, y, stream,
                           extra=(ctypes.cast(arr, ctypes.c_void_p),))


def noalloc_scratch_bytes(T, d, f, n, K) -> int:
    """moe_noalloc_scratch_bytes: scratch a moe_forward_noalloc call of this shape needs."""
    return int(lib().moe_noalloc_scratch_bytes(T, d, f, n, K))


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def forward_f32(x, Wg, W1, W3, W2, K, y=None, stream=None):
    """moe_forward_f32: the same layer with fp32 inputs."""
    import torch
    return _forward(lib().moe_forward_f32, torch.float32, x, Wg, W1, W3, W2, K, y, stream)


def _route(fn, dtype, x, Wg, K, outputs, stream, mid=()):
    import torch
    _expect(x, dtype, "x", 2)
    _expect(Wg, dtype, "Wg", 2)
    T, d = x.shape
    n = Wg.shape[1]
    if Wg.shape[0] != d:
        raise ValueError("Wg must be [d][n]")
    dev = x.device
    shapes = {"topk_idx": ((T, K), torch.int32), "topk_w": ((T, K), torch.float32),
              "counts": ((n,), torch.int32), "offsets": ((n + 1,), torch.int32),
              "perm_token": ((T * K,), torch.int32), "slot_pos": ((T, K), torch.int32)}
    out = {}
    for name in outputs:
        shp, dt = shapes[name]
        out[name] = torch.empty(shp, dtype=dt, device=dev)
    _check(fn(_ptr(x), _ptr(Wg), T, d, n, int(K), *mid, _ptr(out.get("topk_idx")),
              _ptr(out.get("topk_w")), _ptr(out.get("counts")), _ptr(out.get("offsets")),
              _ptr(out.get("perm_token")), _ptr(out.get("slot_pos")), _stream(stream)))
    return out


ROUTE_OUTPUTS = ("topk_idx", "topk_w", "counts", "offsets", "perm_token", "slot_pos")


def route(x, Wg, K, outputs=ROUTE_OUTPUTS, stream=None):
    """moe_route on bf16 x, Wg; returns a dict of the requested int32/fp32 tensors."""
    import torch
    return _route(lib().moe_route, torch.bfloat16, x, Wg, K, outputs, stream)


def route_f32(x, Wg, K, outputs=ROUTE_OUTPUTS, stream=None):
    """moe_route_f32 on fp32 x, Wg."""
    import torch
    return _route(lib().moe_route_f32, torch.float32, x, Wg, K, outputs, stream)


def _route_stats(fn, dtype, x, Wg, K, alpha, outputs, stream):
    import torch
    _expect(x, dtype, "x", 2)
    _expect(Wg, dtype, "Wg", 2)
    T, d = x.shape
    n = Wg.shape[1]
    if Wg.shape[0] != d:
        raise ValueError("Wg must be [d][n]")
    shapes = {"frac": (n,), "prob": (n,), "aux_loss": (1,)}
    out = {name: torch.empty(shapes[name], dtype=torch.float32, device=x.device) for name in outputs}
    _check(fn(_ptr(x), _ptr(Wg), T, d, n, int(K), float(alpha), _ptr(out.get("frac")),
              _ptr(out.get("prob")), _ptr(out.get("aux_loss")), _stream(stream)))
    return out


STATS_OUTPUTS = ("frac", "prob", "aux_loss")


def route_stats(x, Wg, K, alpha=0.01, outputs=STATS_OUTPUTS, stream=None):
    """moe_route_stats on bf16 x, Wg: dict of frac[n], prob[n], aux_loss[1] (fp32)."""
    import torch
    return _route_stats(lib().moe_route_stats, torch.bfloat16, x, Wg, K, alpha, outputs, stream)


def route_stats_f32(x, Wg, K, alpha=0.01, outputs=STATS_OUTPUTS, stream=None):
    """moe_route_stats_f32 on fp32 x, Wg."""
    import torch
    return _route_stats(lib().moe_route_stats_f32, torch.float32, x, Wg, K, alpha, outputs, stream)


def expert_capacity(T, n, K, capacity_factor) -> int:
    """moe_expert_capacity: ceil(capacity_factor * T * K / n) (0 if invalid)."""
    return int(lib().moe_expert_capacity(int(T), int(n), int(K), float(capacity_factor)))


def route_capacity(x, Wg, K, capacity_factor, outputs=None, stream=None):
    """moe_route_capacity on bf16 x, Wg: routing with each expert keeping at most
    expert_capacity(...) assignments (slot_pos -1 marks a dropped one)."""
    import torch
    return _route(lib().moe_route_capacity, torch.bfloat16, x, Wg, K,
                  ROUTE_OUTPUTS if outputs is None else outputs, stream, mid=(float(capacity_factor),))


def forward_capacity(x, Wg, W1, W3, W2, K, capacity_factor, y=None, stream=None):
    """moe_forward_capacity: moe_forward with dropped assignments past each expert's capacity."""
    import torch
    return _forward(lib().moe_forward_capacity, torch.bfloat16, x, Wg, W1, W3, W2, K, y, stream,
                    mid=(float(capacity_factor),))


def expert_choice_capacity(T, n, capacity_factor) -> int:
    """moe_expert_choice_capacity: min(T, ceil(capacity_factor * T / n)) (0 if invalid)."""
    return int(lib().moe_expert_choice_capacity(int(T), int(n), float(capacity_factor)))


def route_expert_choice(x, Wg, capacity_factor, outputs=("scores", "perm_token", "slot_pos"), stream=None):
    """moe_route_expert_choice on bf16 x, Wg: dict of scores [T][n], perm_token [n*C], slot_pos [T][n]."""
    import torch
    _expect(x, torch.bfloat16, "x", 2)
    _expect(Wg, torch.bfloat16, "Wg", 2)
    T, d = x.shape
    n = Wg.shape[1]
    if Wg.shape[0] != d:
        raise ValueError("Wg must be [d][n]")
    C = max(expert_choice_capacity(T, n, capacity_factor), 0)
    shapes = {"scores": ((T, n), torch.float32), "perm_token": ((n * C,), torch.int32),
              "slot_pos": ((T, n), torch.int32)}
    out = {k: torch.empty(shapes[k][0], dtype=shapes[k][1], device=x.device) for k in outputs}
    _check(lib().moe_route_expert_choice(_ptr(x), _ptr(Wg), T, d, n, float(capacity_factor),
                                         _ptr(out.get("scores")), _ptr(out.get("perm_token")),
                                         _ptr(out.get("slot_pos")), _stream(stream)))
    return out


def forward_expert_choice(x, Wg, W1, W3, W2, capacity_factor, y=None, stream=None):
    """moe_forward_expert_choice: the layer with expert-choice routing."""
    import torch
    return _forward(lambda *a: lib().moe_forward_expert_choice(*a[:9], float(capacity_factor), *a[10:]),
                    torch.bfloat16, x, Wg, W1, W3, W2, 0, y, stream)


def quantize_q4(W, stream=None):
    """moe_quantize_q4: bf16 W[n][R][C] -> (codes uint8 [n*R*C/2], scales bf16 [n][R/128][C])."""
    import torch
    _expect(W, torch.bfloat16, "W", 3)
    n, R, C = W.shape
    codes = torch.empty((n * R * C // 2,), dtype=torch.uint8, device=W.device)
    scales = torch.empty((n, R // 128, C), dtype=torch.bfloat16, device=W.device)
    _check(lib().moe_quantize_q4(_ptr(W), n, R, C, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def forward_q4(x, Wg, w1, w3, w2, d, f, K, y=None, stream=None):
    """moe_forward_q4: w1, w3, w2 are (codes, scales) pairs from quantize_q4 of
    W1/W3 [n][d][f] and W2 [n][f][d]; returns fp32 y[T][d]."""
    import torch
    _expect(x, torch.bfloat16, "x", 2)
    _expect(Wg, torch.bfloat16, "Wg", 2)
    T = x.shape[0]
    n = Wg.shape[1]
    if x.shape[1] != d or Wg.shape[0] != d:
        raise ValueError("x must be [T][d] and Wg [d][n]")
    for (q, s), (R, C) in zip((w1, w3, w2), ((d, f), (d, f), (f, d))):
        if q.dtype != torch.uint8 or q.numel() != n * R * C // 2 or not q.is_contiguous():
            raise ValueError("codes must be contiguous uint8 of n*R*C/2 bytes")
        if s.dtype != torch.bfloat16 or tuple(s.shape) != (n, R // 128, C) or not s.is_contiguous():
            raise ValueError("scales must be contiguous bf16 [n][R/128][C]")
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _check(lib().moe_forward_q4(_ptr(x), _ptr(Wg), _ptr(w1[0]), _ptr(w1[1]), _ptr(w3[0]), _ptr(w3[1]),
                                _ptr(w2[0]), _ptr(w2[1]), T, d, f, n, int(K), _ptr(y), _stream(stream)))
    return y


def workspace_bytes(T, d, f, n, K) -> int:
    return int(lib().moe_workspace_bytes(T, d, f, n, K))


def release() -> None:
    _check(lib().moe_release())
