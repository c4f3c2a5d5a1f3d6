"""Parity helpers: compare the HIP path's outputs with the fp64 oracle.

Acceptance (the layer's stated bar):
  * routing indices, counts, offsets and the permutation are bit-exact on tokens
    whose oracle margin between the K-th and (K+1)-th logit exceeds 1e-3;
  * a token at or below that margin must have a valid near-top-K set, checked
    from both sides: every chosen expert lies within 1e-3 of the K-th oracle
    logit, and every expert more than 1e-3 above it is chosen; the slots are in
    descending oracle logit up to 1e-3.  Its GPU choice is then substituted into
    the oracle's selection, and the integer dispatch arrays must equal the
    oracle's dispatch of that selection bit for bit;
  * fp outputs: row-wise normwise relative error |y_gpu - y|_2 / |y|_2 has
    max <= 2e-2 and mean <= 2e-3 (bf16 inputs, fp32 accumulation), and every
    element lies within ELEM_REL * rms(y_t) of the oracle, so that one wrong
    element in an otherwise accurate row is caught.

The element bound.  The bf16 path rounds the hidden activation h once (relative
error at most 2^-9, uniform in sign); each y element is a sum over f such
rounding errors weighted by W2, so its error is close to Gaussian with a
standard deviation of about 1.7e-3 * rms(y_t) (host simulation with bf16 h:
1.66e-3 at d = 64 ... 1024, f = 64 ... 3584, maximum 8.4e-3 over 10^5 .. 10^6
elements).  Over the 3.4e7 elements of the largest configuration the expected
maximum is about 6 standard deviations (1e-2); 2.5e-2 is 15 standard
deviations, while a misplaced or dropped element of typical size is off by
about 1 * rms(y_t).  The fp32 path's errors are below 1e-6 * rms; its bound is
1.25e-4 (the same 1.25 x the normwise maximum).
"""
from __future__ import annotations

import numpy as np

import oracle

MARGIN = 1e-3
BF16_MAX_REL = 2e-2
BF16_MEAN_REL = 2e-3
# fp32 path: inputs are exact in fp32, sums of a few hundred terms in fp32
# carry a relative error of order 1e-6; 1e-4 / 1e-5 leave two orders of margin.
F32_MAX_REL = 1e-4
F32_MEAN_REL = 1e-5
BF16_ELEM_REL = 2.5e-2
F32_ELEM_REL = 1.25e-4
_ELEM_FOR = {BF16_MAX_REL: BF16_ELEM_REL, F32_MAX_REL: F32_ELEM_REL}


# Smallest normal fp32 number.  The GPU keeps gate weights and y in fp32, so an
# oracle row whose size lies below this (a kept expert whose logit trails the
# top one by more than about 87, as the skewed router produces, has a weight
# that fp32 flushes towards 0) cannot be resolved; such rows are compared with
# this absolute scale instead of their own norm.
FP32_TINY = 2.0 ** -126


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref, axis=1)
    num = np.linalg.norm(got - ref, axis=1)
    return num / np.maximum(den, FP32_TINY)


def elem_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """|y_gpu - y| / rms(y_t), element by element (rms over the row's d values,
    at least FP32_TINY)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    return np.abs(got - ref) / np.maximum(rms, FP32_TINY)


def assert_rows_close(got, ref, max_rel, mean_rel, what="y", elem_rel=None):
    """Normwise row bounds plus the element bound (derived in the module header;
    by default the one that goes with the bf16 or fp32 row bounds)."""
    if elem_rel is None:
        elem_rel = _ELEM_FOR[max_rel]
    r = row_rel_err(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert r.max() <= max_rel and r.mean() <= mean_rel, (
        f"{what}: max_rel={r.max():.3e} (<= {max_rel}) mean_rel={r.mean():.3e} (<= {mean_rel}); "
        f"worst row {int(r.argmax())}")
    if np.asarray(ref).size:
        e = elem_rel_err(got, ref)
        worst = np.unravel_index(int(e.argmax()), e.shape)
        assert e.max() <= elem_rel, (
            f"{what}: element {tuple(int(i) for i in worst)} off by {e.max():.3e} x rms(row) "
            f"(<= {elem_rel}); {int((e > elem_rel).sum())} elements over")
        print(f"  {what}: rows {r.size}, normwise max {r.max():.3e} mean {r.mean():.3e} "
              f"(bounds {max_rel:g}, {mean_rel:g}); elementwise max {e.max():.3e} x rms(row) "
              f"(bound {elem_rel:g})", flush=True)
    return r


def check_routing(r: dict, gpu: dict, K: int, w_atol: float = 1e-4) -> np.ndarray:
    """Check GPU routing outputs against the oracle route record ``r``.
    Returns the substituted selection (the GPU's, validated) for later fp checks."""
    logits, sel, margin, slot_margin = r["logits"], r["sel"], r["margin"], r["slot_margin"]
    T, n = logits.shape
    g_idx = np.asarray(gpu["topk_idx"], dtype=np.int64).reshape(T, K)
    assert ((g_idx >= 0) & (g_idx < n)).all(), "expert index out of range"
    # distinct experts per token
    srt = np.sort(g_idx, axis=1)
    assert (srt[:, 1:] != srt[:, :-1]).all() if K > 1 else True, "repeated expert in a token"
    decided = margin > MARGIN
    # set equality on decided tokens
    assert (np.sort(sel[decided], axis=1) == srt[decided]).all(), (
        f"top-K set differs on {int((np.sort(sel[decided], axis=1) != srt[decided]).any(axis=1).sum())} "
        "decided tokens")
    # slot order where the kept logits are separated
    ordered = decided & (slot_margin > MARGIN)
    assert (sel[ordered] == g_idx[ordered]).all(), "slot order differs on separated tokens"
    # near-tie tokens, checked from both sides: every GPU choice within the
    # margin of the K-th oracle logit, and every expert clearly above it chosen
    und = ~decided
    if und.any():
        kth = np.take_along_axis(logits, sel[:, K - 1:K], axis=1)[:, 0][und]
        lu = logits[und]
        chosen = np.take_along_axis(lu, g_idx[und], axis=1)
        assert (chosen >= kth[:, None] - MARGIN).all(), "invalid near-tie selection (a chosen expert is too low)"
        mask = np.zeros(lu.shape, dtype=bool)
        np.put_along_axis(mask, g_idx[und], True, axis=1)
        clear = lu > kth[:, None] + MARGIN
        assert not (clear & ~mask).any(), "invalid near-tie selection (a clearly higher expert is missing)"
    # slot order of every token: descending oracle logit up to the margin
    if K > 1:
        lg = np.take_along_axis(logits, g_idx, axis=1)
        assert (lg[:, :-1] >= lg[:, 1:] - MARGIN).all(), "slots out of descending logit order"
    # substituted selection: the oracle's on decided tokens (verified equal as a
    # set, and in order where separated), the GPU's elsewhere
    sub = g_idx.copy()
    counts, offsets, perm_token, slot_pos = oracle.dispatch(sub, n)
    if "counts" in gpu:
        np.testing.assert_array_equal(np.asarray(gpu["counts"]), counts)
    if "offsets" in gpu:
        np.testing.assert_array_equal(np.asarray(gpu["offsets"]), offsets)
    if "perm_token" in gpu:
        np.testing.assert_array_equal(np.asarray(gpu["perm_token"]), perm_token)
    if "slot_pos" in gpu:
        np.testing.assert_array_equal(np.asarray(gpu["slot_pos"]).reshape(T, K), slot_pos)
    if "topk_w" in gpu:
        w_ref = oracle.gate_weights(logits, sub)
        gw = np.asarray(gpu["topk_w"], dtype=np.float64).reshape(T, K)
        err = np.abs(gw - w_ref).max()
        assert err <= w_atol, f"gate weights off by {err:.3e}"
    return sub
