"""The comparison rules of the GPU parity harness, on hand-made values (no GPU).

Appended K/V rows are bf16; a GPU row passes when every element is within one
bf16 step of the oracle's (one unit in the last place of the larger of the two
values), with an absolute floor of 2^-16 for values below 2^-9.
"""
import numpy as np

from parity_util import KV_ABS_FLOOR, bf16_values, kv_row_excess


def bits(x):
    """float -> bf16 bits by truncation (the values below are exact in bf16)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_values_decode_exactly():
    x = np.array([1.0, -2.5, 0.0, 2.0 ** -20, 3.0 * 2.0 ** 10], dtype=np.float32)
    assert np.array_equal(bf16_values(bits(x)), x.astype(np.float64))


def test_identical_rows_pass_with_no_difference():
    b = bits(np.linspace(-3, 3, 128))
    x, n = kv_row_excess(b, b)
    assert x == 0.0 and n == 0


def test_one_step_passes_two_steps_fail():
    base = np.array([1.0, -1.5, 3.0, 0.75], dtype=np.float32)
    b = bits(base)
    one = b.astype(np.int32).copy()
    one[0] += 1          # 1.0 -> 1 + 2^-7: one step of [1, 2)
    one[2] -= 1          # 3.0 -> 3 - 2^-6: one step of [2, 4)
    x, n = kv_row_excess(one.astype(np.uint16), b)
    assert n == 2 and abs(x - 1.0) < 1e-12
    two = b.astype(np.int32).copy()
    two[1] += 2          # -1.5 -> two steps
    x2, _ = kv_row_excess(two.astype(np.uint16), b)
    assert abs(x2 - 2.0) < 1e-12


def test_a_step_counts_at_the_larger_value():
    # 2 - 2^-7 (top of [1, 2), step 2^-7) against 2.0 (step 2^-6): one step of
    # the larger value is 2^-6, the difference 2^-7, half a step
    x, _ = kv_row_excess(bits([2.0 - 2.0 ** -7]), bits([2.0]))
    assert abs(x - 0.5) < 1e-12


def test_small_values_use_the_absolute_floor():
    # opposite signs near zero: many steps of such small values, but far
    # below the floor
    x, n = kv_row_excess(bits([1e-7]), bits([-1e-7]))
    assert n == 1 and x < 0.02
    # 2^-10 + 2^-16 against 2^-10 (both exact in bf16): the step of
    # [2^-10, 2^-9) is 2^-17, so the difference is 2 steps and exactly the floor
    x, _ = kv_row_excess(bits([2.0 ** -10 + 2.0 ** -16]), bits([2.0 ** -10]))
    assert abs(x - 1.0) < 1e-12
    assert KV_ABS_FLOOR == 2.0 ** -16
    # above 2^-9 the floor no longer widens the bound
    x, _ = kv_row_excess(bits([2.0 ** -8 + 2.0 * 2.0 ** -15]), bits([2.0 ** -8]))
    assert abs(x - 2.0) < 1e-12


def test_a_wrong_row_is_far_out():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(1024).astype(np.float32)
    b = a.copy()
    b[:512], b[512:] = a[512:], a[:512].copy()  # halves swapped (a wrong RoPE pairing, a transposed row)
    x, _ = kv_row_excess(bits(b), bits(a))
    assert x > 100


def _routing_case(slip=False):
    """One (layer, row): logits, the top-3 ids and their weights, and an
    oracle report whose logits differ from the GPU's by 1e-4."""
    z = np.array([0.3, -1.2, 2.0, 0.9, -0.4, 1.5, 0.0, -2.2])
    ids = np.array([2, 5, 3], dtype=np.int32)
    p = np.exp(z - z.max())
    p /= p.sum()
    w = p[ids] / (p.sum() if slip else p[ids].sum())  # slip: not renormalised over the chosen experts
    zo = z + 1e-4 * np.array([1, -1, 1, -1, 1, -1, 1, -1])
    po = np.exp(zo - zo.max())
    wo = po[ids] / po[ids].sum()
    rep = dict(oracle_ids=[ids[None]], oracle_w=[wo[None]], oracle_logits=[zo[None]])
    return ids[None, None], w[None, None].astype(np.float32), z[None, None].astype(np.float32), rep


def test_routing_weight_rule_accepts_a_correct_step(orc):
    from parity_util import assert_routing_weights
    ids, w, z, rep = _routing_case()
    assert_routing_weights(ids, w, z, rep, 1, 1)


def test_routing_weight_rule_catches_a_missing_renormalisation(orc):
    import pytest
    from parity_util import assert_routing_weights
    ids, w, z, rep = _routing_case(slip=True)
    with pytest.raises(AssertionError):
        assert_routing_weights(ids, w, z, rep, 1, 1)
