"""Parity helpers: compare the HIP path's outputs with the fp64 oracle.

Acceptance (the layer's stated bar):
  * routing indices, counts, offsets and the permutation are bit-exact on tokens
    whose oracle margin between the K-th and (K+1)-th logit exceeds 1e-3;
  * a token at or below that margin must have a valid near-top-K set (every
    chosen expert within 1e-3 of the K-th oracle logit); its GPU choice is then
    substituted into the oracle's selection, and the integer dispatch arrays
    must equal the oracle's dispatch of that selection bit for bit;
  * fp outputs: row-wise normwise relative error |y_gpu - y|_2 / |y|_2 has
    max <= 2e-2 and mean <= 2e-3 (bf16 inputs, fp32 accumulation).
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


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref, axis=1)
    num = np.linalg.norm(got - ref, axis=1)
    return num / np.where(den == 0, 1.0, den)


def assert_rows_close(got, ref, max_rel, mean_rel, what="y"):
    r = row_rel_err(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert r.max() <= max_rel and r.mean() <= mean_rel, (
        f"{what}: max_rel={r.max():.3e} (<= {max_rel}) mean_rel={r.mean():.3e} (<= {mean_rel}); "
        f"worst row {int(r.argmax())}")
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
    # near-tie tokens: every GPU choice within the margin of the K-th oracle logit
    und = ~decided
    if und.any():
        kth = np.take_along_axis(logits, sel[:, K - 1:K], axis=1)[:, 0]
        chosen = np.take_along_axis(logits[und], g_idx[und], axis=1)
        assert (chosen >= kth[und][:, None] - MARGIN).all(), "invalid near-tie selection"
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
