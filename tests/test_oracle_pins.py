"""Pins of the fp64 oracle against what the pages and mathematics fix (CPU only).

Each test ties an oracle function to something other than itself: a value the
pages print, brute force over every expert subset, a special case with a known
answer, a closed form, or a metamorphic invariant.  A plausible slip in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a softmax
over all n experts, a top-K tie to the higher index) fails at least one test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import bf16_bits_from_f32, bf16_bits_to_f32, make_config_inputs, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _small(T=24, d=16, f=24, n=6, K=2, seed=7):
    inp = make_inputs(T, d, f, n, K, dtype="f32", seed=seed)
    return inp.f64("x"), inp.f64("Wg"), inp.f64("W1"), inp.f64("W3"), inp.f64("W2")


# ------------------------------------------------------------ worked example

def test_worked_example_selection_and_weights():
    g = _load("worked_example.json")
    logits = np.array(g["logits"])
    n = logits.size
    # x = e_0 makes the router's logits equal row 0 of W_g exactly
    x = np.zeros((1, n))
    x[0, 0] = 1.0
    Wg = np.zeros((n, n))
    Wg[0] = logits
    r = oracle.route(x, Wg, g["K"])
    assert list(r["sel"][0]) == g["selected_zero_based"]
    assert [i + 1 for i in r["sel"][0]] == g["selected_page_numbering"]
    w = r["w"][0]
    assert list(np.round(w, g["weights_printed_decimals"])) == g["weights_printed"]
    # two-way softmax closed form: the larger weight is sigmoid of the gap 2.3 - 1.5
    assert abs(w[0] - 1.0 / (1.0 + math.exp(-0.8))) < 1e-15
    assert abs(w[1] - 1.0 / (1.0 + math.exp(0.8))) < 1e-15


# ------------------------------------------------------------------- router

def test_router_logits_match_triple_loop():
    x, Wg, *_ = _small(T=5, d=7, n=3)
    L = oracle.router_logits(x, Wg)
    for t in range(5):
        for e in range(3):
            s = 0.0
            for j in range(7):
                s += x[t, j] * Wg[j, e]
            assert abs(L[t, e] - s) < 1e-13


def test_router_one_hot_reads_wg_row():
    rng = np.random.default_rng(3)
    Wg = rng.standard_normal((8, 8))
    for j in range(8):
        x = np.zeros((1, 8))
        x[0, j] = 1.0
        np.testing.assert_array_equal(oracle.router_logits(x, Wg)[0], Wg[j])


# -------------------------------------------------------------------- top-K

@pytest.mark.parametrize("K", [1, 2, 3, 8])
def test_topk_equals_brute_force_distinct(K):
    rng = np.random.default_rng(11 + K)
    L = rng.standard_normal((200, 8))
    sel, margin, _ = oracle.topk_select(L, K)
    for t in range(L.shape[0]):
        assert tuple(sorted(sel[t])) == oracle.brute_force_topk(L[t], K)
        # slot order: descending logit
        assert all(L[t, sel[t][k]] >= L[t, sel[t][k + 1]] for k in range(K - 1))
        if K < 8:
            assert margin[t] >= 0


@pytest.mark.parametrize("K", [1, 2, 4])
def test_topk_ties_go_to_lower_index(K):
    rng = np.random.default_rng(5)
    L = rng.integers(-2, 3, size=(300, 8)).astype(np.float64)  # many ties
    sel, _, _ = oracle.topk_select(L, K)
    for t in range(L.shape[0]):
        assert tuple(sorted(sel[t])) == oracle.brute_force_topk(L[t], K)
        # slot order: descending value, equal values by ascending index
        keys = [(-L[t, e], e) for e in sel[t]]
        assert keys == sorted(keys)


def test_brute_force_is_exhaustive():
    # every subset considered: a lone large logit at the last index must be found
    row = np.zeros(9)
    row[8] = 1.0
    assert oracle.brute_force_topk(row, 1) == (8,)
    assert oracle.brute_force_topk(row, 2) == (0, 8)
    assert len(list(itertools.combinations(range(8), 2))) == 28


def test_wg_zero_picks_first_k_with_equal_weights():
    inp = make_inputs(64, 32, 16, 8, 3, dtype="f32", seed=2, wg_zero=True)
    r = oracle.route(inp.f64("x"), inp.f64("Wg"), 3)
    assert (r["sel"] == np.array([0, 1, 2])).all()
    assert (r["w"] == 1.0 / 3.0).all()
    assert (r["margin"] == 0).all()


# ------------------------------------------------------------ gate weights

def test_gate_weights_sum_to_one_positive_descending():
    x, Wg, *_ = _small(T=200, n=8)
    r = oracle.route(x, Wg, 2)
    w = r["w"]
    assert (w > 0).all()
    assert np.abs(w.sum(axis=1) - 1.0).max() <= 1e-15
    assert (w[:, 0] >= w[:, 1]).all()


def test_k1_weight_exactly_one_and_argmax_expert():
    x, Wg, W1, W3, W2 = _small(T=40, n=5, K=1)
    r = oracle.route(x, Wg, 1)
    assert (r["w"] == 1.0).all()
    assert (r["sel"][:, 0] == np.argmax(r["logits"], axis=1)).all()
    y = oracle.forward(x, Wg, W1, W3, W2, 1)
    for t in range(x.shape[0]):
        e = int(np.argmax(r["logits"][t]))
        ref = oracle.expert_swiglu(x[t:t + 1], W1[e], W3[e], W2[e])[0]
        np.testing.assert_allclose(y[t], ref, rtol=0, atol=1e-13)


def test_softmax_over_kept_not_over_all():
    # renormalising a full n-way softmax restricted to the top K gives the same
    # weights; a full softmax without renormalisation does not (n > K)
    x, Wg, *_ = _small(T=50, n=8)
    r = oracle.route(x, Wg, 2)
    L = r["logits"]
    full = np.exp(L - L.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    kept = np.take_along_axis(full, r["sel"], axis=1)
    np.testing.assert_allclose(r["w"], kept / kept.sum(axis=1, keepdims=True), atol=1e-15)
    assert np.abs(r["w"] - kept).max() > 1e-3


# ---------------------------------------------------------- special cases

def test_k_equals_n_is_dense_softmax_mixture():
    x, Wg, W1, W3, W2 = _small(T=12, n=4, K=4)
    y = oracle.forward(x, Wg, W1, W3, W2, 4)
    L = x @ Wg
    for t in range(x.shape[0]):
        p = np.exp(L[t] - L[t].max())
        p /= p.sum()
        ref = sum(p[e] * oracle.expert_swiglu(x[t:t + 1], W1[e], W3[e], W2[e])[0] for e in range(4))
        np.testing.assert_allclose(y[t], ref, rtol=0, atol=1e-13)


def test_n_k_one_is_dense_swiglu_ffn():
    # the dense 4x FFN of "A visual guide to MoE models" (Dense Layers): 512 -> 2048 -> 512
    rng = np.random.default_rng(9)
    d, f, T = 512, 2048, 3
    x = rng.standard_normal((T, d))
    Wg = rng.standard_normal((d, 1))
    W1 = rng.standard_normal((1, d, f)) / math.sqrt(d)
    W3 = rng.standard_normal((1, d, f)) / math.sqrt(d)
    W2 = rng.standard_normal((1, f, d)) / math.sqrt(f)
    y = oracle.forward(x, Wg, W1, W3, W2, 1)
    for t in range(T):
        hid = np.empty(f)
        for j in range(f):
            a = float(np.dot(x[t], W1[0][:, j]))
            b = float(np.dot(x[t], W3[0][:, j]))
            hid[j] = a / (1.0 + math.exp(-a)) * b
        ref = np.array([np.dot(hid, W2[0][:, c]) for c in range(d)])
        np.testing.assert_allclose(y[t], ref, rtol=0, atol=1e-11)


def test_unselected_experts_contribute_nothing():
    # a constant input feature with a -1e3 router weight makes experts 4 and 5
    # lose every token; their weights are then poisoned with NaN
    x, Wg, W1, W3, W2 = _small(T=30, n=6)
    x2 = np.concatenate([x, np.ones((x.shape[0], 1))], axis=1)
    Wg2 = np.concatenate([Wg, np.zeros((1, 6))], axis=0)
    Wg2[-1, 4:] = -1e3
    W1p = np.concatenate([W1, np.zeros((6, 1, W1.shape[2]))], axis=1)
    W3p = np.concatenate([W3, np.zeros((6, 1, W3.shape[2]))], axis=1)
    W2p = np.concatenate([W2, np.zeros((6, W2.shape[1], 1))], axis=2)
    sel, _, _ = oracle.topk_select(x2 @ Wg2, 2)
    assert not np.isin(sel, [4, 5]).any()
    y_ref = oracle.forward(x2, Wg2, W1p, W3p, W2p, 2)
    for W in (W1p, W3p, W2p):
        W[4:] = np.nan
    y_nan = oracle.forward(x2, Wg2, W1p, W3p, W2p, 2)
    assert np.isfinite(y_nan).all()
    np.testing.assert_array_equal(y_nan, y_ref)


def test_mask_form_matches_gather_form():
    for (n, K) in [(8, 2), (6, 1), (5, 5), (7, 3)]:
        x, Wg, W1, W3, W2 = _small(T=40, n=n, K=K, seed=n * 10 + K)
        a = oracle.forward(x, Wg, W1, W3, W2, K)
        b = oracle.forward_mask_form(x, Wg, W1, W3, W2, K)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_mask_form_matches_gather_form_with_ties():
    inp = make_inputs(16, 8, 12, 6, 2, dtype="f32", seed=4, wg_zero=True)
    args = (inp.f64("x"), inp.f64("Wg"), inp.f64("W1"), inp.f64("W3"), inp.f64("W2"))
    np.testing.assert_allclose(oracle.forward(*args, 2), oracle.forward_mask_form(*args, 2),
                               rtol=0, atol=1e-12)


def test_forward_equals_brute_force_per_token():
    inp = make_config_inputs("tiny_fp32")
    x, Wg, W1, W3, W2 = (inp.f64(k) for k in ("x", "Wg", "W1", "W3", "W2"))
    x = x[:16]
    y = oracle.forward(x, Wg, W1, W3, W2, 2)
    L = x @ Wg
    for t in range(x.shape[0]):
        sub = oracle.brute_force_topk(L[t], 2)
        order = sorted(sub, key=lambda e: (-L[t, e], e))
        z = np.array([math.exp(L[t, e] - L[t, order[0]]) for e in order])
        w = z / z.sum()
        ref = np.zeros(x.shape[1])
        for k, e in enumerate(order):
            a = x[t] @ W1[e]
            b = x[t] @ W3[e]
            h = np.array([ai / (1.0 + math.exp(-ai)) * bi for ai, bi in zip(a, b)])
            ref += w[k] * (h @ W2[e])
        np.testing.assert_allclose(y[t], ref, rtol=0, atol=1e-12)


# -------------------------------------------------------------- metamorphic

def test_relabelling_experts_leaves_y_unchanged():
    x, Wg, W1, W3, W2 = _small(T=50, n=8)
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    y = oracle.forward(x, Wg, W1, W3, W2, 2)
    yp = oracle.forward(x, Wg[:, perm], W1[perm], W3[perm], W2[perm], 2)
    _, margin, slot_margin = oracle.topk_select(x @ Wg, 2)
    ok = (margin > 1e-9) & (slot_margin > 1e-9)
    assert ok.mean() > 0.9
    np.testing.assert_allclose(yp[ok], y[ok], rtol=0, atol=1e-12)


def test_token_permutation_permutes_rows():
    x, Wg, W1, W3, W2 = _small(T=50, n=8)
    perm = np.random.default_rng(1).permutation(50)
    y = oracle.forward(x, Wg, W1, W3, W2, 2)
    yp = oracle.forward(x[perm], Wg, W1, W3, W2, 2)
    np.testing.assert_allclose(yp, y[perm], rtol=0, atol=1e-12)


def test_scaling_down_projection_scales_y_exactly():
    x, Wg, W1, W3, W2 = _small(T=50, n=8)
    y = oracle.forward(x, Wg, W1, W3, W2, 2)
    y2 = oracle.forward(x, Wg, W1, W3, 2.0 * W2, 2)
    np.testing.assert_array_equal(y2, 2.0 * y)


def test_swapping_gate_and_up_changes_y():
    # SiLU acts on the W1 side only; a transposed reading would swap W1/W3
    x, Wg, W1, W3, W2 = _small(T=20, n=4)
    a = oracle.forward(x, Wg, W1, W3, W2, 2)
    b = oracle.forward(x, Wg, W3, W1, W2, 2)
    assert np.abs(a - b).max() > 1e-3


# ----------------------------------------------------------- SiLU / sigmoid

def test_sigmoid_and_silu_closed_forms():
    z = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(oracle.sigmoid(z), 0.5 * (1.0 + np.tanh(z / 2.0)), rtol=0, atol=1e-15)
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    # z*s(z) - (-z)*s(-z) = z (s(z) + s(-z)) = z
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
    assert abs(float(oracle.silu(1.0)) - 0.7310585786300049) < 1e-16
    assert float(oracle.silu(-800.0)) == 0.0  # no overflow to NaN


# ---------------------------------------------------------------- dispatch

def test_dispatch_matches_sorting_by_expert_then_token():
    rng = np.random.default_rng(21)
    T, n, K = 300, 8, 2
    sel = np.stack([rng.choice(n, size=K, replace=False) for _ in range(T)])
    counts, offsets, perm_token, slot_pos = oracle.dispatch(sel, n)
    pairs = sorted((int(sel[t, k]), t, k) for t in range(T) for k in range(K))
    assert [t for (_, t, _) in pairs] == list(perm_token)
    for p, (e, t, k) in enumerate(pairs):
        assert slot_pos[t, k] == p
    assert list(counts) == [sum(1 for q in pairs if q[0] == e) for e in range(n)]
    assert offsets[0] == 0 and offsets[-1] == T * K


def test_dispatch_invariants_with_empty_experts():
    sel = np.array([[3, 1], [1, 3], [0, 3], [3, 0]])
    counts, offsets, perm_token, slot_pos = oracle.dispatch(sel, 6)
    assert list(counts) == [2, 2, 0, 4, 0, 0]
    assert list(offsets) == [0, 2, 4, 4, 8, 8, 8]
    assert list(perm_token) == [2, 3, 0, 1, 0, 1, 2, 3]
    for t in range(4):
        for k in range(2):
            p = slot_pos[t, k]
            assert perm_token[p] == t
            e = sel[t, k]
            assert offsets[e] <= p < offsets[e + 1]


# ----------------------------------------------------- parameter arithmetic

def test_mixtral_parameter_arithmetic():
    g = _load("mixtral_params.json")
    c = oracle.mixtral_param_counts(**g["config"])
    p = g["printed"]
    assert round(c["per_expert"] / 1e6) == p["per_expert_millions"]
    assert round(c["experts"] / 1e9, 1) == p["experts_billions_1dp"]
    assert round(c["attention"] / 1e9, 1) == p["attention_billions_1dp"]
    assert round(c["embeddings"] / 1e9, 2) == p["embeddings_billions_2dp"]
    assert round(c["routers"] / 1e6) == p["routers_millions"]
    assert round(c["total"] / 1e9, 1) == p["total_billions_1dp"]
    assert round(c["shared"] / 1e9, 1) == p["shared_billions_1dp"]
    assert round(c["two_experts_all_layers"] / 1e9, 1) == p["two_experts_all_layers_billions_1dp"]
    assert round(c["active"] / 1e9, 1) == p["active_billions_1dp"]
    assert c["naive"] / 1e9 == p["naive_billions"]
    assert round(c["total"] / 1e9) == p["total_rounded_billions"]
    assert round(c["active"] / 1e9) == p["active_rounded_billions"]
    assert round(c["total"] * 2 / 1e9) == p["memory_16bit_gb"]
    assert round(c["total"] * 0.5 / 1e9) == p["memory_4bit_gb"]
    # exact integers of the closed form
    assert c["total"] == 46_704_349_184
    assert c["active"] == 12_881_481_728


# ---------------------------------------------------------------- generator

def test_generator_is_seeded_and_rounds_to_nearest_even():
    a = make_inputs(8, 64, 64, 4, 2, dtype="bf16", seed=5)
    b = make_inputs(8, 64, 64, 4, 2, dtype="bf16", seed=5)
    for k in ("x", "Wg", "W1", "W3", "W2"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    r = make_inputs(8, 64, 64, 4, 2, dtype="bf16", seed=5, router_only=True)
    np.testing.assert_array_equal(r.x, a.x)
    np.testing.assert_array_equal(r.Wg, a.Wg)
    v = np.array([1.0, 1.00390625, 1.005859375, 1.01171875, -2.5], dtype=np.float32)
    np.testing.assert_array_equal(bf16_bits_to_f32(bf16_bits_from_f32(v)),
                                  np.array([1.0, 1.0, 1.0078125, 1.015625, -2.5], dtype=np.float32))


def test_skewed_router_recipe_shares():
    inp = make_config_inputs("mixtral_skewed", router_only=True)
    sel, _, _ = oracle.topk_select(oracle.router_logits(inp.f64("x"), inp.f64("Wg")), 2)
    top1 = np.bincount(sel[:, 0], minlength=8) / sel.shape[0]
    assert 0.45 <= top1[0] <= 0.50
    assert top1[7] < 0.02


# ------------------------------------------------------ router statistics
# Part 5 of the explainer ("The favourite expert problem", tool 2): the loss
# alpha * N * sum_i f_i P_i is smallest when both shares are even (1/N each).

@pytest.mark.parametrize("K", [1, 2, 3])
def test_stats_uniform_probabilities_give_alpha(K):
    # W_g = 0: every logit ties, P_i = 1/N exactly; any f then gives alpha
    n, T, alpha = 8, 40, 0.02
    logits = np.zeros((T, n))
    sel, _, _ = oracle.topk_select(logits, K)
    st = oracle.router_stats(logits, sel, alpha)
    np.testing.assert_array_equal(st["prob"], np.full(n, 1.0 / n))
    assert abs(st["aux_loss"] - alpha) <= 1e-15


def test_stats_balanced_assignment_gives_alpha():
    # round-robin top-1 routing (token t prefers expert t mod N): f_i = 1/N
    # exactly, so the loss is alpha * sum_i P_i = alpha whatever P is
    n, T, alpha = 8, 64, 0.01
    logits = np.zeros((T, n))
    # token t's own expert wins by a margin that grows with the expert index,
    # so the average probabilities are far from uniform
    logits[np.arange(T), np.arange(T) % n] = 0.5 + (np.arange(T) % n)
    sel, _, _ = oracle.topk_select(logits, 1)
    st = oracle.router_stats(logits, sel, alpha)
    np.testing.assert_array_equal(st["frac"], np.full(n, 1.0 / n))
    assert not np.allclose(st["prob"], 1.0 / n)
    assert abs(st["aux_loss"] - alpha) <= 1e-15


def test_stats_collapse_to_one_expert_gives_alpha_n():
    # the favourite-expert failure: every token sends everything to expert 0
    n, T, alpha = 8, 16, 0.01
    logits = np.zeros((T, n))
    logits[:, 0] = 60.0  # exp(-60) ~ 1e-26: P_0 = 1 to double precision
    sel, _, _ = oracle.topk_select(logits, 1)
    st = oracle.router_stats(logits, sel, alpha)
    assert st["frac"][0] == 1.0 and st["frac"][1:].sum() == 0.0
    assert abs(st["aux_loss"] - alpha * n) <= 1e-15 * n


def test_stats_shares_sum_to_one_and_two_expert_softmax_is_logistic():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((50, 2)) * 3
    sel, _, _ = oracle.topk_select(logits, 1)
    st = oracle.router_stats(logits, sel, 0.01)
    assert abs(st["frac"].sum() - 1.0) <= 1e-15 and abs(st["prob"].sum() - 1.0) <= 1e-15
    # P_0 for two experts is the mean of the logistic function of the logit gap
    gap = logits[:, 0] - logits[:, 1]
    np.testing.assert_allclose(st["prob"][0], np.mean(1.0 / (1.0 + np.exp(-gap))), rtol=0, atol=1e-15)


def test_stats_cauchy_schwarz_bound_when_shares_match():
    # with f = P the loss is alpha * N * sum f^2 >= alpha (equality iff uniform):
    # K = N makes f uniform, and with W_g = 0 P is uniform too
    n = 6
    logits = np.zeros((10, n))
    sel, _, _ = oracle.topk_select(logits, n)
    st = oracle.router_stats(logits, sel, 0.5)
    assert abs(st["aux_loss"] - 0.5) <= 1e-15


# -------------------------------------------------------- capacity dispatch
# Part 5 of the explainer ("What happens when an expert is full"): capacity =
# tokens / experts * capacity factor; overflowing work is dropped and the
# token passes on through the residual connection.

def test_capacity_formula():
    assert oracle.expert_capacity(8192, 8, 2, 1.0) == 8192 * 2 // 8
    assert oracle.expert_capacity(8192, 8, 2, 1.25) == 2560
    assert oracle.expert_capacity(8192, 64, 2, 1.0) == 256
    assert oracle.expert_capacity(100, 8, 1, 1.0) == 13      # ceil(12.5)
    assert oracle.expert_capacity(10, 8, 2, 1e-9) == 1


def test_capacity_hand_example():
    # expert loads in token order: e0 <- t0, t1, (t2, t3, t4 overflow at C = 2);
    # e1 <- t0, t2, (t3 overflows); e2 <- t1, t4
    sel = np.array([[0, 1], [0, 2], [0, 1], [1, 0], [2, 0]])
    d = oracle.capacity_dispatch(sel, 3, 2)
    np.testing.assert_array_equal(d["kept"], [[1, 1], [1, 1], [0, 1], [0, 0], [1, 0]])
    np.testing.assert_array_equal(d["counts"], [2, 2, 2])
    np.testing.assert_array_equal(d["offsets"], [0, 2, 4, 6])
    np.testing.assert_array_equal(d["perm_token"], [0, 1, 0, 2, 1, 4])
    np.testing.assert_array_equal(d["slot_pos"], [[0, 2], [1, 4], [-1, 3], [-1, -1], [5, -1]])


def test_capacity_drops_latest_tokens_of_overfull_experts_only():
    rng = np.random.default_rng(11)
    T, n, K = 400, 6, 2
    sel = np.stack([rng.choice(n, size=K, replace=False, p=[0.4, 0.2, 0.1, 0.1, 0.1, 0.1]) for _ in range(T)])
    cap = 90
    d = oracle.capacity_dispatch(sel, n, cap)
    full = oracle.dispatch(sel, n)
    np.testing.assert_array_equal(d["counts"], np.minimum(full[0], cap))
    for e in range(n):
        toks = np.nonzero((sel == e).any(axis=1))[0]          # token order
        kept_toks = np.nonzero(((sel == e) & d["kept"]).any(axis=1))[0]
        np.testing.assert_array_equal(kept_toks, toks[:cap])
    # kept rows point back to their tokens
    for t in range(T):
        for k in range(K):
            if d["kept"][t, k]:
                assert d["perm_token"][d["slot_pos"][t, k]] == t


def test_capacity_without_overflow_is_dropless():
    x, Wg, W1, W3, W2 = _small(T=60, n=6)
    r = oracle.route(x, Wg, 2)
    d = oracle.capacity_dispatch(r["sel"], 6, 60 * 2)
    full = oracle.dispatch(r["sel"], 6)
    for a, b in zip((d["counts"], d["offsets"], d["perm_token"], d["slot_pos"]), full):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(oracle.forward_capacity(x, Wg, W1, W3, W2, r["sel"], 120),
                                  oracle.forward(x, Wg, W1, W3, W2, 2))


def test_capacity_forward_keeps_only_kept_terms():
    x, Wg, W1, W3, W2 = _small(T=40, n=4)
    r = oracle.route(x, Wg, 2)
    cap = 12
    y = oracle.forward_capacity(x, Wg, W1, W3, W2, r["sel"], cap)
    kept = oracle.capacity_dispatch(r["sel"], 4, cap)["kept"]
    assert (~kept).any(axis=1).any() and (~kept).all(axis=1).any()  # partial and total drops occur
    for t in range(40):
        ref = np.zeros(x.shape[1])
        for k in range(2):
            if kept[t, k]:
                e = r["sel"][t, k]
                ref += r["w"][t, k] * oracle.expert_swiglu(x[t:t + 1], W1[e], W3[e], W2[e])[0]
        np.testing.assert_allclose(y[t], ref, rtol=0, atol=1e-13)
        if not kept[t].any():
            assert (y[t] == 0).all()


# ------------------------------------------------------------ 4-bit weights

def test_q4_word_layout_hand_example():
    # one expert, R = 256 (two groups of 128), C = 32 (two tiles of 16 columns)
    n, R, C = 1, 256, 32
    base = np.full(n * R * C // 2, 0x88, dtype=np.uint8)  # every code 0
    # codes -7..0 for r = 0..7 of column 0: nibbles u = 1..8; even elements in
    # the low half-word (1, 3, 5, 7 -> 0x7531), odd ones in the high half-word (0x8642)
    packed = base.copy()
    packed[0:4] = [0x31, 0x75, 0x42, 0x86]
    codes = oracle.unpack_q4(packed, n, R, C)
    np.testing.assert_array_equal(codes[0, 0:8, 0], np.arange(-7, 1))
    codes[0, 0:8, 0] = 0
    assert (codes == 0).all()
    # the first byte of a word: low nibble element 0 (+2 from 0xA), high
    # nibble element 2 (+1 from 0x9).  Strides from the stated order: 4 bytes
    # per word (8 reduction indices), 16 per column, 256 per 32-index chunk,
    # 1024 per 16-column tile, C*64 = 2048 per 128-index group.
    for off, (r, c) in [(16, (0, 1)), (4, (8, 0)), (256, (32, 0)), (1024, (0, 16)),
                        (2048, (128, 0)), (2048 + 1024 + 256 + 16 + 4, (168, 17))]:
        p = base.copy()
        p[off] = 0x9A
        cd = oracle.unpack_q4(p, n, R, C)
        assert cd[0, r, c] == 2 and cd[0, r + 2, c] == 1, off
        cd[0, r, c] = 0
        cd[0, r + 2, c] = 0
        assert (cd == 0).all(), off


def test_q4_exactly_representable_weights_round_trip():
    rng = np.random.default_rng(21)
    n, R, C = 2, 256, 6
    q = rng.integers(-7, 8, size=(n, R, C)).astype(np.float32)
    q[:, ::128, :] = 7.0                       # every group-column reaches |q| = 7
    s = np.float32(2.0) ** rng.integers(-9, -2, size=(n, R // 128, C)).astype(np.float32)
    W = (q.reshape(n, R // 128, 128, C) * s[:, :, None, :]).reshape(n, R, C)
    codes, scales = oracle.quantize_q4(W)
    np.testing.assert_array_equal(scales, s)
    np.testing.assert_array_equal(codes, q.astype(np.int8))
    np.testing.assert_array_equal(oracle.dequantize_q4(codes, scales), W.astype(np.float64))


def test_q4_error_bound_and_extremes():
    rng = np.random.default_rng(22)
    n, R, C = 3, 384, 10
    W = (rng.standard_normal((n, R, C)) * 0.02).astype(np.float32)
    W[1, 128:256, 4] = 0.0                     # an all-zero group
    codes, scales = oracle.quantize_q4(W)
    assert codes.min() >= -7 and codes.max() <= 7
    assert scales[1, 1, 4] == 0 and (codes[1, 128:256, 4] == 0).all()
    # the bf16 scale is within 2^-9 of max/7, so |W/s| <= 7.02 and no code clips:
    # every element is within half a step of its code
    step = np.repeat(scales, 128, axis=1).astype(np.float64)
    err = np.abs(W.astype(np.float64) - oracle.dequantize_q4(codes, scales))
    assert (err <= 0.5 * step * (1 + 1e-6)).all()
    # the largest magnitude of each group-column maps to +-7
    Wg = np.abs(W.reshape(n, R // 128, 128, C))
    at = Wg.argmax(axis=2)
    cg = codes.reshape(n, R // 128, 128, C)
    top = np.take_along_axis(cg, at[:, :, None, :], axis=2)[:, :, 0, :]
    assert (np.abs(top)[scales > 0] == 7).all()


def test_q4_bf16_round_ties_to_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8)], dtype=np.float32)
    np.testing.assert_array_equal(oracle.bf16_round(v),
                                  np.array([1.0, 1.0 + 2 ** -6, 1.0, -1.0], dtype=np.float32))


# ----------------------------------------------------- expert-choice routing
# First page, "How Experts Are Chosen (Routing Methods)": experts choose the
# tokens they process, each with a fixed capacity.

def test_expert_choice_equals_brute_force_subsets():
    rng = np.random.default_rng(41)
    T, n, C = 7, 3, 3
    logits = rng.standard_normal((T, n))
    logits[4] = logits[2]                       # tokens 2 and 4 tie for every expert
    chosen, S, _ = oracle.expert_choice_select(logits, C)
    for e in range(n):
        best, best_key = None, None
        for sub in itertools.combinations(range(T), C):   # lexicographic order
            key = sum(S[list(sub), e])
            if best is None or key > best_key + 1e-15:
                best, best_key = sub, key
        np.testing.assert_array_equal(np.nonzero(chosen[:, e])[0], best)


def test_expert_choice_full_capacity_is_dense_mixture():
    # C = T: every expert takes every token, y = sum_e softmax_e * E_e(x), the
    # token-choice layer with K = n
    x, Wg, W1, W3, W2 = _small(T=20, n=4)
    C = oracle.expert_choice_capacity(20, 4, 4.0)
    assert C == 20
    chosen, _, _ = oracle.expert_choice_select(oracle.router_logits(x, Wg), C)
    assert chosen.all()
    np.testing.assert_allclose(oracle.forward_expert_choice(x, Wg, W1, W3, W2, chosen),
                               oracle.forward(x, Wg, W1, W3, W2, 4), rtol=0, atol=1e-12)


def test_expert_choice_ties_take_earliest_tokens_and_unchosen_get_zero():
    # W_g = 0: all scores tie at 1/n, every expert takes tokens 0..C-1
    x, Wg, W1, W3, W2 = _small(T=24, n=6)
    C = oracle.expert_choice_capacity(24, 6, 2.0)
    assert C == 8
    chosen, S, margin = oracle.expert_choice_select(np.zeros((24, 6)), C)
    assert (chosen[:C].all()) and not chosen[C:].any() and (margin == 0).all()
    y = oracle.forward_expert_choice(x, 0 * Wg, W1, W3, W2, chosen)
    assert (y[C:] == 0).all()
    ref = sum(oracle.expert_swiglu(x[:C], W1[e], W3[e], W2[e]) for e in range(6)) / 6.0
    np.testing.assert_allclose(y[:C], ref, rtol=0, atol=1e-13)


def test_expert_choice_dispatch_layout():
    rng = np.random.default_rng(43)
    T, n = 50, 5
    C = oracle.expert_choice_capacity(T, n, 1.5)
    assert C == 15
    chosen, _, _ = oracle.expert_choice_select(rng.standard_normal((T, n)), C)
    assert (chosen.sum(axis=0) == C).all()
    perm, slot = oracle.expert_choice_dispatch(chosen, C)
    for e in range(n):
        toks = perm[e * C:(e + 1) * C]
        assert (np.diff(toks) > 0).all()
        np.testing.assert_array_equal(slot[toks, e], e * C + np.arange(C))
    assert ((slot >= 0) == chosen).all()


# --------------------------------------- near-tie margins (acceptance rule)
# The acceptance rule compares the top-K set exactly where the gap between the
# K-th and (K+1)-th scores exceeds 1e-3, and the slot order exactly where every
# gap between consecutive kept scores does (Part 3 of the explainer, step 2:
# keep the highest scores, the larger listed first).  Hand-worked rows with
# known gaps fix both margins.

# scores 5, 1.0005, 1.0, 0.2 placed out of order: sorted order is e2, e3, e0, e1
_MARGIN_ROW = np.array([[1.0, 0.2, 5.0, 1.0005]])


@pytest.mark.parametrize("K,sel,margin,slot_margin", [
    (1, [2], 5.0 - 1.0005, math.inf),
    (2, [2, 3], 1.0005 - 1.0, 5.0 - 1.0005),
    (3, [2, 3, 0], 1.0 - 0.2, 1.0005 - 1.0),
    (4, [2, 3, 0, 1], math.inf, 1.0005 - 1.0),
])
def test_topk_margins_hand_worked(K, sel, margin, slot_margin):
    s, m, sm = oracle.topk_select(_MARGIN_ROW, K)
    assert list(s[0]) == sel
    assert m[0] == margin            # exact: the same two fp64 subtractions
    assert sm[0] == slot_margin


def test_topk_margins_ties_and_rows():
    # an exact tie at the K-th place gives margin 0; a tie inside the kept slots
    # gives slot margin 0; rows are independent
    L = np.array([[3.0, 1.0, 1.0, 0.0],      # K=2: 1.0 vs 1.0 tie at 2nd/3rd -> margin 0
                  [2.0, 2.0, -1.0, -4.0],    # K=2: kept slots tie -> slot margin 0, margin 3
                  [-1.0, -2.5, -0.5, -3.0]])
    s, m, sm = oracle.topk_select(L, 2)
    np.testing.assert_array_equal(s, [[0, 1], [0, 1], [2, 0]])
    np.testing.assert_array_equal(m, [0.0, 3.0, 1.5])
    np.testing.assert_array_equal(sm, [2.0, 0.0, 0.5])


# ------------------------------- expert-choice readings, pinned by hand
# "How Experts Are Chosen (Routing Methods)" names expert-based routing without
# details; the readings (probability score, unnormalised weights, ceil in the
# capacity) are pinned here against hand-computed values.

def _two_token_router():
    # x = the logits themselves (W_g = I): token 0 scores (3, 5), token 1 (1, -1)
    x = np.array([[3.0, 5.0], [1.0, -1.0]])
    return x, np.eye(2)


def test_expert_choice_ranks_by_probability_not_logit():
    # expert 0: token 0 has the larger logit (3 > 1) but the smaller probability
    # (sigmoid(-2) = 0.119 < sigmoid(2) = 0.881), so with C = 1 expert 0 takes
    # token 1; expert 1 takes token 0 either way
    x, Wg = _two_token_router()
    C = oracle.expert_choice_capacity(2, 2, 1.0)
    assert C == 1
    chosen, S, margin = oracle.expert_choice_select(oracle.router_logits(x, Wg), C)
    np.testing.assert_array_equal(chosen, [[False, True], [True, False]])
    sig2 = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(S, [[1 - sig2, sig2], [sig2, 1 - sig2]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(margin, [2 * sig2 - 1, 2 * sig2 - 1], rtol=0, atol=1e-15)


def test_expert_choice_weights_are_not_renormalised():
    # each token is chosen by one expert only; its output is that expert's output
    # times the router probability sigmoid(2) = 0.8808, not times 1
    x, Wg = _two_token_router()
    rng = np.random.default_rng(5)
    W1, W3 = rng.standard_normal((2, 2, 3)), rng.standard_normal((2, 2, 3))
    W2 = rng.standard_normal((2, 3, 2))
    chosen = np.array([[False, True], [True, False]])
    y = oracle.forward_expert_choice(x, Wg, W1, W3, W2, chosen)
    sig2 = 1.0 / (1.0 + math.exp(-2.0))
    e1_t0 = oracle.expert_swiglu(x[0:1], W1[1], W3[1], W2[1])[0]
    e0_t1 = oracle.expert_swiglu(x[1:2], W1[0], W3[0], W2[0])[0]
    np.testing.assert_allclose(y[0], sig2 * e1_t0, rtol=1e-14, atol=0)
    np.testing.assert_allclose(y[1], sig2 * e0_t1, rtol=1e-14, atol=0)
    assert np.abs(y[0] - e1_t0).max() > 0.05 * np.abs(e1_t0).max()


@pytest.mark.parametrize("T,n,cf,C", [
    (10, 4, 1.0, 3),      # 2.5 -> 3 (floor would give 2)
    (7, 3, 1.0, 3),       # 2.33 -> 3
    (9, 4, 2.0, 5),       # 4.5 -> 5
    (100, 8, 0.01, 1),    # 0.125 -> 1
    (3, 2, 5.0, 3),       # 7.5 -> 8, at most T
    (8192, 8, 2.0, 2048),
])
def test_expert_choice_capacity_rounds_up(T, n, cf, C):
    assert oracle.expert_choice_capacity(T, n, cf) == C


def test_expert_choice_capacity_ceil_changes_selection():
    # T = 10, n = 4, cf = 1: each expert takes 3 tokens (not 2)
    rng = np.random.default_rng(17)
    logits = rng.standard_normal((10, 4))
    C = oracle.expert_choice_capacity(10, 4, 1.0)
    chosen, _, _ = oracle.expert_choice_select(logits, C)
    np.testing.assert_array_equal(chosen.sum(axis=0), [3, 3, 3, 3])
