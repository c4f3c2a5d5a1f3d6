"""moe_route / moe_route_f32 on the GPU against the fp64 oracle: bit-exact
indices and dispatch arrays (margin rule), gate weights within 1e-4."""
import numpy as np
import pytest

import oracle
from gpu_util import config_inputs, log, upload
from parity import check_routing
from synth import make_inputs

pytestmark = pytest.mark.gpu


def _moe():
    import sparse_mixture_experts_22_amd as moe
    return moe


def _gpu_route(inp, K, outputs=None):
    import torch
    moe = _moe()
    dev = upload(inp)
    fn = moe.route if inp.dtype == "bf16" else moe.route_f32
    kw = {} if outputs is None else {"outputs": outputs}
    out = fn(dev["x"], dev["Wg"], K, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check(inp, K, outputs=None):
    log(f"route: T={inp.T} d={inp.d} n={inp.n} K={K} dtype={inp.dtype}")
    gpu = _gpu_route(inp, K, outputs)
    r = oracle.route(inp.f64("x"), inp.f64("Wg"), K)
    sub = check_routing(r, gpu, K)
    return r, gpu, sub


def test_route_tiny_fp32():
    _check(config_inputs("tiny_fp32"), 2)


@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_prefill", "mixtral_skewed", "many_experts"])
def test_route_full_configs(name):
    inp = config_inputs(name, router_only=True)
    r, gpu, _ = _check(inp, inp.K)
    counts = gpu["counts"]
    log(f"  {name}: counts={counts.tolist()[:16]} near-ties={(r['margin'] <= 1e-3).sum()}")
    if name == "mixtral_skewed":
        top1 = np.bincount(gpu["topk_idx"][:, 0], minlength=8) / inp.T
        assert 0.45 <= top1[0] <= 0.50 and top1[7] < 0.02


@pytest.mark.parametrize("T,d,n,K,dtype", [
    (1, 64, 8, 2, "bf16"),
    (32, 192, 8, 2, "bf16"),       # one routing block: W_g read in place, fused dispatch
    (20, 128, 5, 3, "bf16"),       # one block, n not a multiple of 8
    (32, 64, 16, 4, "bf16"),       # one block, 16 experts
    (17, 64, 1, 1, "bf16"),        # one block, one expert
    (32, 2048, 16, 2, "bf16"),     # one block, wide d
    (32, 64, 17, 2, "bf16"),       # one block, n > 16: transposed W_g copy, fused dispatch
    (32, 256, 8, 2, "bf16"),       # one block, d % 256 == 0: the reduction split over workgroups
    (7, 512, 5, 3, "bf16"),        # the same, n not a multiple of 8, a partial block
    (32, 1024, 16, 4, "bf16"),     # the same, 16 experts
    (1, 256, 1, 1, "bf16"),        # the same, one token, one expert
    (129, 128, 8, 2, "bf16"),      # ragged tail of a 128-token block
    (1000, 192, 8, 2, "bf16"),
    (300, 64, 1, 1, "bf16"),       # one expert
    (300, 64, 5, 3, "bf16"),       # n not a multiple of 8 (scalar W_g staging)
    (257, 64, 130, 4, "bf16"),     # 64-token routing blocks, 9 expert tiles
    (200, 64, 256, 8, "bf16"),     # maximum n and K
    (300, 64, 8, 8, "bf16"),       # K = n
    (300, 64, 8, 1, "bf16"),       # K = 1
    (1000, 256, 32, 2, "bf16"),    # many tokens, n % 16 == 0: a routing block per wave, W_g read in place
    (777, 512, 64, 2, "bf16"),     # 64 experts, ragged last routing block
    (300, 256, 128, 4, "bf16"),    # 128 experts: 16-token routing blocks
    (129, 256, 256, 8, "bf16"),    # 256 experts, K = 8
    (40, 256, 64, 1, "bf16"),      # two routing blocks, K = 1
    (333, 48, 6, 2, "f32"),
    (129, 64, 256, 8, "f32"),
])
def test_route_shapes(T, d, n, K, dtype):
    inp = make_inputs(T, d, 64, n, K, dtype=dtype, seed=T * 7 + n, router_only=True)
    _, gpu, _ = _check(inp, K)
    if K == 1:
        assert (gpu["topk_w"] == 1.0).all()
    assert np.abs(gpu["topk_w"].sum(axis=1) - 1.0).max() <= 1e-6


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_all_ties_pick_lowest_indices(dtype):
    inp = make_inputs(200, 64, 64, 8, 3, dtype=dtype, seed=3, wg_zero=True, router_only=True)
    gpu = _gpu_route(inp, 3)
    assert (gpu["topk_idx"] == np.array([0, 1, 2])).all()
    np.testing.assert_allclose(gpu["topk_w"], 1.0 / 3.0, rtol=0, atol=1e-7)
    assert gpu["counts"].tolist() == [200, 200, 200, 0, 0, 0, 0, 0]


# Logit rows with exact ties below a strictly larger later logit: the tied
# experts must still be kept in ascending index order (the displaced earlier
# expert outranks an equal later one).
_TIE_PATTERNS = np.array([
    [1, 1, 2, -4, -4, -4, -4, -4],
    [1, 1, 1, 2, -4, -4, -4, -4],
    [-4, 0.5, 0.5, 0.5, 3, 0.5, -4, -4],
    [2, 1, 1, 3, -4, -4, -4, -4],
    [0.25, 0.25, 0.25, 0.25, 0.25, 0.25, 0.25, 1],
], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [20, 200])    # one routing block (fused dispatch) and several
@pytest.mark.parametrize("K", [2, 3])
def test_route_ties_below_a_larger_later_logit(dtype, T, K):
    from synth import bf16_bits_from_f32
    inp = make_inputs(T, 64, 64, 8, K, dtype=dtype, seed=17, router_only=True)
    P = len(_TIE_PATTERNS)
    x = np.zeros((T, 64), dtype=np.float32)
    x[np.arange(T), np.arange(T) % P] = 1.0       # token t's logits are pattern t % P, exactly
    wg = np.zeros((64, 8), dtype=np.float32)
    wg[:P] = _TIE_PATTERNS
    if dtype == "bf16":
        inp.x, inp.Wg = bf16_bits_from_f32(x), bf16_bits_from_f32(wg)
    else:
        inp.x, inp.Wg = x, wg
    gpu = _gpu_route(inp, K)
    r = oracle.route(inp.f64("x"), inp.f64("Wg"), K)
    np.testing.assert_array_equal(gpu["topk_idx"], r["sel"])
    np.testing.assert_allclose(gpu["topk_w"], r["w"], rtol=0, atol=1e-6)
    for name in ("counts", "offsets", "perm_token", "slot_pos"):
        np.testing.assert_array_equal(gpu[name].reshape(np.shape(r[name])), r[name])


# Exact ties spread over the lanes and expert tiles of the wave-level top-K (64
# experts, several routing blocks): larger score first, then the lower index.
_TIE_PATTERNS_64 = [
    {7: 1.0, 40: 1.0},                      # a tie across expert tiles, then the zeros from 0 up
    {63: 3.0, 16: 2.0, 32: 2.0, 48: 2.0},   # one winner, then a three-way tie at the tiles' first lanes
    {},                                     # all equal: the lowest indices
    {0: 1.0, 15: 1.0, 31: 1.0, 47: 1.0},    # ties at the ends of the 16-lane groups
    {e: -e / 64.0 for e in range(64)},      # strictly decreasing with the index
    {e: -2.0 for e in range(8)},            # the first experts below all the others
]


@pytest.mark.parametrize("K", [1, 2, 3, 8])
def test_route_ties_many_experts(K):
    from synth import bf16_bits_from_f32
    T, d, n = 200, 256, 64
    inp = make_inputs(T, d, 64, n, K, dtype="bf16", seed=29, router_only=True)
    P = len(_TIE_PATTERNS_64)
    x = np.zeros((T, d), dtype=np.float32)
    x[np.arange(T), np.arange(T) % P] = 1.0       # token t's logits are pattern t % P, exactly
    wg = np.zeros((d, n), dtype=np.float32)
    for i, pat in enumerate(_TIE_PATTERNS_64):
        for e, v in pat.items():
            wg[i, e] = v
    inp.x, inp.Wg = bf16_bits_from_f32(x), bf16_bits_from_f32(wg)
    gpu = _gpu_route(inp, K)
    r = oracle.route(inp.f64("x"), inp.f64("Wg"), K)
    np.testing.assert_array_equal(gpu["topk_idx"], r["sel"])
    np.testing.assert_allclose(gpu["topk_w"], r["w"], rtol=0, atol=1e-6)
    for name in ("counts", "offsets", "perm_token", "slot_pos"):
        np.testing.assert_array_equal(gpu[name].reshape(np.shape(r[name])), r[name])


def test_route_partial_outputs():
    inp = make_inputs(500, 128, 64, 8, 2, dtype="bf16", seed=8, router_only=True)
    full = _gpu_route(inp, 2)
    for outs in (("perm_token",), ("counts", "offsets"), ("topk_w", "slot_pos")):
        part = _gpu_route(inp, 2, outputs=outs)
        for k in outs:
            np.testing.assert_array_equal(part[k], full[k])


def test_route_is_deterministic():
    inp = config_inputs("many_experts", router_only=True)
    a = _gpu_route(inp, 2)
    b = _gpu_route(inp, 2)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
