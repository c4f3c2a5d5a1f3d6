"""The acceptance checks themselves (tests/parity.py), on the CPU: fake GPU
records that break the rule must be rejected, valid ones accepted.

Near-tie tokens are those whose K-th and (K+1)-th oracle logits are within 1e-3
(Part 3 of "Mixture of Experts: Why Mixtral Only Wakes Up Two Specialists",
step 2, keeps the highest scores; a tie is only decided by rounding)."""
import numpy as np
import pytest

import oracle
from parity import (BF16_MAX_REL, BF16_MEAN_REL, F32_MAX_REL, F32_MEAN_REL, assert_rows_close,
                    check_routing)


def _route_record(L, K):
    # oracle.route on x = I, W_g = L^T ... built directly from the logits
    sel, margin, slot_margin = oracle.topk_select(L, K)
    return dict(logits=L, sel=sel, margin=margin, slot_margin=slot_margin)


def _fake_gpu(idx, n):
    idx = np.asarray(idx, dtype=np.int64)
    counts, offsets, perm_token, slot_pos = oracle.dispatch(idx, n)
    return dict(topk_idx=idx, counts=counts, offsets=offsets, perm_token=perm_token, slot_pos=slot_pos)


# token 0: a clear winner (5) then a near-tie between 1.0005 and 1.0 for 2nd place;
# token 1: well separated
_L = np.array([[5.0, 1.0005, 1.0, -2.0],
               [0.1, 3.0, -1.0, 2.0]])


def test_exact_selection_passes():
    r = _route_record(_L, 2)
    assert r["margin"][0] <= 1e-3 < r["margin"][1]
    sub = check_routing(r, _fake_gpu([[0, 1], [1, 3]], 4), 2)
    np.testing.assert_array_equal(sub, [[0, 1], [1, 3]])


def test_near_tie_substitution_is_accepted():
    # picking expert 2 instead of 1 on the near-tie token is valid
    sub = check_routing(_route_record(_L, 2), _fake_gpu([[0, 2], [1, 3]], 4), 2)
    np.testing.assert_array_equal(sub, [[0, 2], [1, 3]])


def test_near_tie_that_drops_the_clear_winner_is_rejected():
    # {1, 2} are both within 1e-3 of the 2nd logit but expert 0 (5.0) is missing
    with pytest.raises(AssertionError, match="clearly higher expert is missing"):
        check_routing(_route_record(_L, 2), _fake_gpu([[1, 2], [1, 3]], 4), 2)


def test_near_tie_with_a_low_expert_is_rejected():
    with pytest.raises(AssertionError, match="too low"):
        check_routing(_route_record(_L, 2), _fake_gpu([[0, 3], [1, 3]], 4), 2)


def test_reversed_slots_are_rejected():
    # on the near-tie token the slot order must still put 5.0 first
    with pytest.raises(AssertionError, match="descending logit order"):
        check_routing(_route_record(_L, 2), _fake_gpu([[2, 0], [1, 3]], 4), 2)
    # and on the separated token exactly
    with pytest.raises(AssertionError):
        check_routing(_route_record(_L, 2), _fake_gpu([[0, 1], [3, 1]], 4), 2)


def test_wrong_set_on_decided_token_is_rejected():
    with pytest.raises(AssertionError, match="top-K set differs"):
        check_routing(_route_record(_L, 2), _fake_gpu([[0, 1], [1, 0]], 4), 2)


def test_wrong_dispatch_is_rejected():
    gpu = _fake_gpu([[0, 1], [1, 3]], 4)
    gpu["perm_token"] = gpu["perm_token"][::-1].copy()
    with pytest.raises(AssertionError):
        check_routing(_route_record(_L, 2), gpu, 2)


def _rows(T=64, d=4096, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, d))


def test_rounding_sized_noise_passes_bf16_bounds():
    ref = _rows()
    rng = np.random.default_rng(1)
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    got = ref + 1.7e-3 * rms * rng.standard_normal(ref.shape)
    assert_rows_close(got, ref, BF16_MAX_REL, BF16_MEAN_REL)


def test_one_wrong_element_fails_although_row_norms_pass():
    # one element of a 4096-wide row off by the row's rms (a typical-size error):
    # the row's normwise error, 1/64, stays under the 2e-2 maximum; the element bound catches it
    ref = _rows()
    rng = np.random.default_rng(2)
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    got = ref + 1e-4 * rms * rng.standard_normal(ref.shape)
    got[7, 100] = ref[7, 100] + rms[7, 0]
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() < BF16_MAX_REL and rel.mean() < BF16_MEAN_REL
    with pytest.raises(AssertionError, match=r"element \(7, 100\)"):
        assert_rows_close(got, ref, BF16_MAX_REL, BF16_MEAN_REL)


def test_fp32_bounds_are_tighter():
    ref = _rows(T=8, d=64)
    got = ref.copy()
    got[3, 5] += 2e-4 * np.sqrt((ref[3] ** 2).mean())
    assert_rows_close(got, ref, BF16_MAX_REL, BF16_MEAN_REL)
    with pytest.raises(AssertionError):
        assert_rows_close(got, ref, F32_MAX_REL, F32_MEAN_REL)


def test_rows_below_fp32_range_are_compared_absolutely():
    # a row whose only kept expert has a gate weight of e^-104 (about 7e-46, below
    # fp32's range) is 0 on the GPU; that is fp32's resolution, not an error
    ref = _rows(T=4, d=64)
    ref[2] *= np.exp(-104.0)
    got = ref.copy()
    got[2] = 0.0
    assert_rows_close(got, ref, BF16_MAX_REL, BF16_MEAN_REL)
    # a row of ordinary size that comes back as zeros still fails
    got[1] = 0.0
    with pytest.raises(AssertionError):
        assert_rows_close(got, ref, BF16_MAX_REL, BF16_MEAN_REL)
