"""Expert-choice routing on the GPU against the fp64 oracle.  Each expert's
chosen set must equal the oracle's where the oracle's C-th and (C+1)-th scores
differ by more than 1e-5; elsewhere the GPU's set must be a valid top-C within
that tolerance and is substituted into the oracle.  Rows and slots are then
bit-exact, y within the bf16 bounds, unchosen tokens exactly 0."""
import numpy as np
import pytest

import oracle
from gpu_util import config_inputs, log, sample_rows, upload
from parity import BF16_MAX_REL, BF16_MEAN_REL, assert_rows_close
from synth import make_inputs

pytestmark = pytest.mark.gpu
SCORE_TOL = 1e-5


def _moe():
    import sparse_mixture_experts_22_amd as moe
    return moe


def _gpu_ec(dev, cf):
    import torch
    out = _moe().route_expert_choice(dev["x"], dev["Wg"], cf)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check_ec(inp, g, cf):
    T, n = inp.T, inp.n
    C = oracle.expert_choice_capacity(T, n, cf)
    assert _moe().expert_choice_capacity(T, n, cf) == C
    logits = oracle.router_logits(inp.f64("x"), inp.f64("Wg"))
    chosen, S, margin = oracle.expert_choice_select(logits, C)
    np.testing.assert_allclose(g["scores"], S, rtol=0, atol=1e-6)
    gch = g["slot_pos"] >= 0
    assert (gch.sum(axis=0) == C).all(), "every expert takes exactly C tokens"
    sub = chosen.copy()
    for e in range(n):
        if margin[e] > SCORE_TOL:
            np.testing.assert_array_equal(gch[:, e], chosen[:, e], err_msg=f"expert {e}")
        else:
            s = np.sort(S[:, e])[::-1]
            kth, nxt = s[C - 1], (s[C] if C < T else -np.inf)
            assert (S[gch[:, e], e] >= kth - SCORE_TOL).all() and (S[~gch[:, e], e] <= nxt + SCORE_TOL).all()
            sub[:, e] = gch[:, e]
    perm, slot = oracle.expert_choice_dispatch(sub, C)
    np.testing.assert_array_equal(g["perm_token"], perm)
    np.testing.assert_array_equal(g["slot_pos"], slot)
    log(f"  C={C} near-tie experts={int((margin <= SCORE_TOL).sum())} unchosen tokens={int((~sub.any(axis=1)).sum())}")
    return sub


@pytest.mark.parametrize("T,d,n,cf,zero", [
    (1, 64, 8, 2.0, False),
    (30, 64, 8, 2.0, False),
    (1000, 192, 8, 2.0, False),
    (257, 64, 130, 4.0, False),
    (200, 128, 8, 2.0, True),      # all scores tie: every expert takes tokens 0..C-1
    (5000, 64, 8, 2.0, True),      # all tie, the C earliest tokens spread over many waves' ranges
    (100, 64, 4, 100.0, False),    # C = T
    (40000, 64, 16, 1.0, False),   # T above the 32768 scores a workgroup stages in LDS
])
def test_route_expert_choice_shapes(T, d, n, cf, zero):
    inp = make_inputs(T, d, 64, n, 2, dtype="bf16", seed=60 + T + n, wg_zero=zero, router_only=True)
    log(f"route_expert_choice: T={T} d={d} n={n} cf={cf} zero={zero}")
    sub = _check_ec(inp, _gpu_ec(upload(inp), cf), cf)
    if zero:
        C = oracle.expert_choice_capacity(T, n, cf)
        assert sub[:C].all() and not sub[C:].any()


@pytest.mark.parametrize("name", ["mixtral_prefill", "many_experts"])
def test_route_expert_choice_full_size(name):
    inp = config_inputs(name, router_only=True)
    log(f"route_expert_choice {name}")
    _check_ec(inp, _gpu_ec(upload(inp), 2.0), 2.0)


def _forward_check(inp, cf, rows=None):
    import torch
    moe = _moe()
    dev = upload(inp)
    y = moe.forward_expert_choice(dev["x"], dev["Wg"], dev["W1"], dev["W3"], dev["W2"], cf)
    g = _gpu_ec(dev, cf)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    del dev
    sub = _check_ec(inp, g, cf)
    rs = np.arange(inp.T) if rows is None else sample_rows(inp.T, rows)
    if rows is None:
        ref = oracle.forward_expert_choice(inp.f64("x"), inp.f64("Wg"), inp.f64("W1"), inp.f64("W3"),
                                           inp.f64("W2"), sub)
    else:
        ref = oracle.forward_expert_choice(inp.f64("x")[rs], inp.f64("Wg"), lambda e: inp.expert_f64("W1", e),
                                           lambda e: inp.expert_f64("W3", e), lambda e: inp.expert_f64("W2", e),
                                           sub[rs])
    gone = ~sub[rs].any(axis=1)
    assert (y[rs][gone] == 0).all(), "a token no expert chose must get y = 0"
    rel = assert_rows_close(y[rs][~gone], ref[~gone], BF16_MAX_REL, BF16_MEAN_REL)
    log(f"  max_rel={rel.max():.3e} mean_rel={rel.mean():.3e} rows={len(rs)}")
    return y


@pytest.mark.parametrize("T,d,f,n,cf", [
    (32, 128, 192, 8, 2.0),       # weight-streaming kernels
    (300, 128, 192, 8, 1.0),
    (2000, 192, 320, 4, 2.0),     # tiled kernels
    (700, 256, 384, 8, 3.0),
])
def test_forward_expert_choice_shapes(T, d, f, n, cf):
    log(f"forward_expert_choice: T={T} d={d} f={f} n={n} cf={cf}")
    _forward_check(make_inputs(T, d, f, n, 2, dtype="bf16", seed=900 + T), cf)


def test_forward_expert_choice_full_capacity_matches_dense_top_n():
    import torch
    moe = _moe()
    inp = make_inputs(256, 128, 192, 4, 4, dtype="bf16", seed=31)
    dev = upload(inp)
    y_ec = moe.forward_expert_choice(dev["x"], dev["Wg"], dev["W1"], dev["W3"], dev["W2"], 4.0)
    y_tc = moe.forward(dev["x"], dev["Wg"], dev["W1"], dev["W3"], dev["W2"], 4)
    torch.cuda.synchronize()
    a, b = y_ec.cpu().numpy(), y_tc.cpu().numpy()
    rel = np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)
    assert rel.max() < 1e-5, rel.max()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_forward_expert_choice_mixtral_prefill():
    log("forward_expert_choice mixtral_prefill cf=2")
    _forward_check(config_inputs("mixtral_prefill"), 2.0, rows=128)


def test_expert_choice_invalid_factor():
    import torch
    moe = _moe()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    for cf in (0.0, -2.0, float("nan")):
        with pytest.raises(moe.MoEError):
            moe.route_expert_choice(x, wg, cf)
