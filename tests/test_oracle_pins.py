"""Pins of the CPU oracle against closed forms, invariants, special cases and
brute force -- never against itself re-typed.

Each test names the mistake it would catch.  The decode step's structure
(deep MoE stack, router choosing a few experts per token per layer,
attention before the MoE block, a KV cache) is what the pages describe
[P3 "TPU Megakernel Achieves 709 tokens/s on Kimi K3, Outpacing GB200",
sections "The Key Innovation..." and "Cross-Layer Weight Prefetching"];
the operator definitions are the standard ones stated in oracle/oracle.h.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

pytestmark = []

# ---------------------------------------------------------------- helpers


def f32_to_bf16_bits(a):
    """Exact bf16 bit patterns for values that are exactly representable."""
    a = np.asarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def bf16_value(bits):
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def mk_layer(orc, d, E, F, n_shared, dtype, rng=None, std=0.02, gate_zero=False, identical=False,
             router_zero=False, bias=None, down_zero=False):
    """A random MoE layer as numpy arrays (fp32; dtype BF16 rounds to bf16 bits)."""
    rng = rng or np.random.default_rng(0)

    def mat(*shape, zero=False):
        if zero:
            a = np.zeros(shape, dtype=np.float32)
        else:
            a = (rng.standard_normal(shape) * std).astype(np.float32)
        if dtype == orc.BF16:
            a = (a.view(np.uint32) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16
            return a.astype(np.uint16)
        return a

    def gain():
        a = rng.uniform(0.9, 1.1, d).astype(np.float32)
        if dtype == orc.BF16:
            return ((a.view(np.uint32) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
        return a

    g2 = gain()
    wr = mat(E, d, zero=router_zero)
    if identical:
        wg0, wu0, wd0 = mat(F, d, zero=gate_zero), mat(F, d), mat(d, F, zero=down_zero)
        wg = [wg0] * E
        wu = [wu0] * E
        wd = [wd0] * E
    else:
        wg = [mat(F, d, zero=gate_zero) for _ in range(E)]
        wu = [mat(F, d) for _ in range(E)]
        wd = [mat(d, F, zero=down_zero) for _ in range(E)]
    sg = [mat(F, d, zero=gate_zero) for _ in range(n_shared)]
    su = [mat(F, d) for _ in range(n_shared)]
    sd = [mat(d, F) for _ in range(n_shared)]
    return orc.OracleLayer(g2, wr, bias, wg, wu, wd, sg, su, sd)


def widen(orc, a):
    return a.astype(np.float64) if a.dtype == np.float32 else (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- bf16


def test_bf16_widening_known_patterns(orc):
    # 1.0, -2.0, smallest subnormal 2^-133, largest finite (2 - 2^-7) * 2^127
    assert orc.bf16_to_double(0x3F80) == 1.0
    assert orc.bf16_to_double(0xC000) == -2.0
    assert orc.bf16_to_double(0x0001) == 2.0 ** -133
    assert orc.bf16_to_double(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127


def test_bf16_rounding_ties_to_even(orc):
    # 1 + 2^-8 is half way between 1.0 (even mantissa) and 1 + 2^-7 (odd): goes down
    assert orc.double_to_bf16(1 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is half way between 1 + 2^-7 (odd) and 1 + 2^-6 (even): goes up
    assert orc.double_to_bf16(1 + 3 * 2 ** -8) == 0x3F82
    # just above a tie rounds up
    assert orc.double_to_bf16(1 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert orc.double_to_bf16(-1.0) == 0xBF80
    assert orc.double_to_bf16(0.0) == 0x0000
    assert orc.double_to_bf16(1e40) == 0x7F80  # overflow to +inf


def test_bf16_rounding_brute_force_exact(orc):
    """Nearest bf16 by exact rational comparison with the two neighbours."""
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300),
                         rng.standard_normal(100)])
    for x in xs:
        x = float(x)
        b = orc.double_to_bf16(x)
        # candidates: truncation of the binary32 value and its neighbours
        f32bits = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
        base = f32bits >> 16
        cands = [c for c in (base - 1, base, base + 1, base + 2) if 0 <= c < 0x10000]
        cands = [c for c in cands if math.isfinite(bf16_value(c))]
        fx = Fraction(x)
        best = min(cands, key=lambda c: (abs(Fraction(bf16_value(c)) - fx), c & 1))
        assert b == best, (x, hex(b), hex(best))


# ---------------------------------------------------------------- RMSNorm


def test_rmsnorm_constant_vector_closed_form(orc):
    # x = c*1: mean(x^2) = c^2, out = c / sqrt(c^2 + eps) * g
    for c, eps in ((1.0, 3.0), (2.0, 1.0), (-0.5, 1e-6)):
        x = np.full(8, c)
        g = np.linspace(0.5, 1.5, 8).astype(np.float32)
        out = orc.rmsnorm(x, g, eps)
        np.testing.assert_allclose(out, c / math.sqrt(c * c + eps) * g.astype(np.float64), rtol=1e-15)
    # eps inside the root: c = 1, eps = 3 gives exactly 1/2 (not 1/(1+3))
    assert orc.rmsnorm(np.ones(4), np.ones(4, np.float32), 3.0)[0] == 0.5


def test_rmsnorm_known_vector_and_scale_invariance(orc):
    x = np.array([3.0, 4.0])
    out = orc.rmsnorm(x, np.ones(2, np.float32), 0.0)
    # mean square = 12.5
    np.testing.assert_allclose(out, x / math.sqrt(12.5), rtol=1e-15)
    rng = np.random.default_rng(2)
    v = rng.standard_normal(64)
    g = rng.uniform(0.9, 1.1, 64).astype(np.float32)
    np.testing.assert_allclose(orc.rmsnorm(7.5 * v, g, 0.0), orc.rmsnorm(v, g, 0.0), rtol=1e-13)


def test_rmsnorm_bf16_gain_widened(orc):
    g = f32_to_bf16_bits([2.0, 0.5])
    out = orc.rmsnorm(np.array([1.0, 1.0]), g, 0.0)
    np.testing.assert_array_equal(out, [2.0, 0.5])


# ---------------------------------------------------------------- matvec


def test_matvec_orientation_out_in(orc):
    # W is [out][in]: y_o = sum_i W[o][i] x_i
    W = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float32)
    x = np.array([1.0, 10.0, 100.0])
    np.testing.assert_array_equal(orc.matvec(W, x), [321.0, 654.0])
    np.testing.assert_array_equal(orc.matvec(f32_to_bf16_bits(W), x), [321.0, 654.0])


def test_matvec_integer_brute_force(orc):
    rng = np.random.default_rng(3)
    W = rng.integers(-8, 8, size=(5, 7)).astype(np.float32)
    x = rng.integers(-8, 8, size=7).astype(np.float64)
    exact = [sum(int(W[o, i]) * int(x[i]) for i in range(7)) for o in range(5)]
    np.testing.assert_array_equal(orc.matvec(W, x), exact)


# ---------------------------------------------------------------- silu / softmax / top-k


def test_silu_closed_forms(orc):
    ln3 = math.log(3.0)
    assert orc.silu(0.0) == 0.0
    assert math.isclose(orc.silu(ln3), 0.75 * ln3, rel_tol=1e-15)     # sigmoid(ln 3) = 3/4
    assert math.isclose(orc.silu(-ln3), -0.25 * ln3, rel_tol=1e-15)   # sigmoid(-ln 3) = 1/4
    assert math.isclose(orc.silu(40.0), 40.0, rel_tol=1e-15)
    assert abs(orc.silu(-40.0)) < 1e-15


def test_softmax_closed_form_and_shift(orc):
    z = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    np.testing.assert_allclose(orc.softmax(z), [0.1, 0.2, 0.3, 0.4], rtol=1e-14)
    np.testing.assert_allclose(orc.softmax(z + 700.0), [0.1, 0.2, 0.3, 0.4], rtol=1e-13)


def test_topk_closed_form(orc):
    p = np.array([0.1, 0.2, 0.3, 0.4])
    ids, w = orc.topk(p, 2)
    assert list(ids) == [3, 2]
    np.testing.assert_allclose(w, [4 / 7, 3 / 7], rtol=1e-15)


def test_topk_ties_lower_id_first(orc):
    ids, w = orc.topk(np.full(8, 0.125), 3)
    assert list(ids) == [0, 1, 2]
    np.testing.assert_allclose(w, [1 / 3] * 3, rtol=1e-15)
    ids, _ = orc.topk(np.array([0.2, 0.3, 0.2, 0.3]), 3)
    assert list(ids) == [1, 3, 0]


def test_topk_forced_weights_from_p(orc):
    ids, w = orc.topk(np.array([0.1, 0.2, 0.3, 0.4]), 2, forced=[0, 3])
    assert list(ids) == [0, 3]
    np.testing.assert_allclose(w, [0.2, 0.8], rtol=1e-15)


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8])
def test_topk_brute_force_subsets(orc, k):
    """The chosen set maximises the summed logit over all C(E, k) subsets."""
    rng = np.random.default_rng(10 + k)
    E = 8
    for _ in range(20):
        z = rng.standard_normal(E)
        ids, w = orc.topk(orc.softmax(z), k)
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(z[list(s)]))
        assert set(ids) == set(best)
        assert math.isclose(w.sum(), 1.0, rel_tol=1e-14)
        # weights ordered like the selection (non-increasing)
        assert all(w[i] >= w[i + 1] for i in range(k - 1))


def test_topk_all_experts(orc):
    z = np.random.default_rng(4).standard_normal(8)
    p = orc.softmax(z)
    ids, w = orc.topk(p, 8)
    assert sorted(ids) == list(range(8))
    np.testing.assert_allclose(w, p[ids], rtol=1e-14)


# ---------------------------------------------------------------- expert


def test_expert_one_hot_orientation(orc):
    """gate picks x1, up picks x0, down writes element 0: y0 = silu(x1) * x0."""
    Wg = np.array([[0, 1, 0], [0, 0, 0]], dtype=np.float32)  # [F=2][d=3]
    Wu = np.array([[1, 0, 0], [0, 0, 1]], dtype=np.float32)
    Wd = np.array([[1, 0], [0, 0], [0, 2]], dtype=np.float32)  # [d=3][F=2]
    x = np.array([2.0, math.log(3.0), 5.0])
    y = orc.expert(Wg, Wu, Wd, x)
    # a = [silu(ln3) * 2, silu(0) * 5 = 0]
    np.testing.assert_allclose(y, [2 * 0.75 * math.log(3.0), 0.0, 0.0], rtol=1e-15, atol=0)


def test_expert_zero_gate_gives_zero(orc):
    rng = np.random.default_rng(5)
    y = orc.expert(np.zeros((4, 6), np.float32), rng.standard_normal((4, 6)).astype(np.float32),
                   rng.standard_normal((6, 4)).astype(np.float32), rng.standard_normal(6))
    np.testing.assert_array_equal(y, np.zeros(6))


# ---------------------------------------------------------------- RoPE


def test_rope_half_split_pairs_closed_form(orc):
    hd, theta, p = 4, 10000.0, 3
    # pair (0, 2) rotates by p * theta^0 = p
    np.testing.assert_allclose(orc.rope([1, 0, 0, 0], p, theta), [math.cos(p), 0, math.sin(p), 0], atol=1e-16)
    # pair (1, 3) rotates by p * theta^(-2/4) = p / 100
    a = p / 100.0
    np.testing.assert_allclose(orc.rope([0, 1, 0, 0], p, theta), [0, math.cos(a), 0, math.sin(a)], atol=1e-16)
    # second element of a pair: (x_i, x_{i+hd/2}) = (0, 1) -> (-sin, cos)
    np.testing.assert_allclose(orc.rope([0, 0, 1, 0], p, theta), [-math.sin(p), 0, math.cos(p), 0], atol=1e-16)


def test_rope_position_zero_identity_and_norm(orc):
    rng = np.random.default_rng(6)
    x = rng.standard_normal(128)
    np.testing.assert_array_equal(orc.rope(x, 0, 1e6), x)
    for p in (1, 77, 4100):
        np.testing.assert_allclose(np.linalg.norm(orc.rope(x, p, 1e6)), np.linalg.norm(x), rtol=1e-14)


def test_rope_relative_position_invariance(orc):
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    base = orc.rope(q, 4100, 1e6) @ orc.rope(k, 4000, 1e6)
    for shift in (-3000, -17, 5, 1234):
        s = orc.rope(q, 4100 + shift, 1e6) @ orc.rope(k, 4000 + shift, 1e6)
        assert math.isclose(s, base, rel_tol=1e-9, abs_tol=1e-9)


# ---------------------------------------------------------------- attention block


def attn_layer(orc, d, H, G, hd, wq, wk, wv, wo, dtype=0):
    g1 = np.ones(d, np.float32)
    E = 2
    dummy = np.zeros((E, d), np.float32)
    ly = orc.OracleLayer(np.ones(d, np.float32), dummy, None, [None] * E, [None] * E, [None] * E,
                         g1=g1, wq=wq, wk=wk, wv=wv, wo=wo)
    dims = orc.make_dims(d, E, 1, 4, 0, dtype, rms_eps=0.0, n_heads=H, n_kv_heads=G, head_dim=hd,
                         rope_theta=10000.0)
    return dims, ly


def test_attention_uniform_scores_mean_of_values_and_group_map(orc):
    """Wq = 0 gives uniform attention: o_h = mean of V over positions 0..p of
    kv head h // (H/G).  Values per kv head differ, so a wrong head->group
    map (h % G instead of h // (H/G)) fails."""
    H, G, hd = 4, 2, 4
    d = H * hd
    p = 5
    wq = np.zeros((H * hd, d), np.float32)
    wk = np.zeros((G * hd, d), np.float32)
    wv = np.zeros((G * hd, d), np.float32)   # new v row = 0
    wo = np.eye(d, dtype=np.float32)          # Attn output lands on h unchanged
    dims, ly = attn_layer(orc, d, H, G, hd, wq, wk, wv, wo)
    cap = 8
    kc = np.zeros((1, G, cap, hd), np.uint16)
    vc = np.zeros((1, G, cap, hd), np.uint16)
    vals = {0: 1.5, 1: -4.0}
    for g in range(G):
        vc[0, g, :p, :] = f32_to_bf16_bits(np.full((p, hd), vals[g], np.float32))
    kv = orc.OracleKV(kc, vc)
    h = np.full((1, d), 2.0)
    out = orc.attn_block(dims, ly, h, [p], kv)
    expect = h.copy()
    for hh in range(H):
        g = hh // (H // G)
        expect[0, hh * hd:(hh + 1) * hd] += vals[g] * p / (p + 1)  # new row v = 0 included
    np.testing.assert_allclose(out, expect, rtol=1e-15)
    # the step wrote its (zero) k, v row at position p
    assert np.all(kv.v[0, :, p, :] == 0) and np.all(kv.k[0, :, p, :] == 0)


def test_attention_single_position_returns_new_value(orc):
    """Empty past (position 0): every head returns the new v row of its kv
    head, rounded to bf16; with x-hat = 1 (constant h, eps = 0, g = 1) the v
    row is the row sums of Wv."""
    H, G, hd = 2, 1, 4
    d = H * hd
    wv = np.zeros((G * hd, d), np.float32)
    for i in range(hd):
        wv[i, i] = 0.25 * (i + 1)   # v_i = 0.25 (i+1), exact in bf16
    dims, ly = attn_layer(orc, d, H, G, hd, np.zeros((H * hd, d), np.float32),
                          np.zeros((G * hd, d), np.float32), wv, np.eye(d, dtype=np.float32))
    kv = orc.OracleKV(np.zeros((1, G, 4, hd), np.uint16), np.zeros((1, G, 4, hd), np.uint16))
    h = np.full((1, d), 3.0)
    out = orc.attn_block(dims, ly, h, [0], kv)
    v = 0.25 * np.arange(1, hd + 1)
    np.testing.assert_allclose(out[0], 3.0 + np.concatenate([v, v]), rtol=1e-15)
    np.testing.assert_array_equal(kv.v[0, 0, 0], f32_to_bf16_bits(v.astype(np.float32)))


def test_attention_two_positions_softmax_closed_form(orc):
    """One cached key k0 and the new key k1 (position 1): weights are the
    2-way softmax of q.k/sqrt(hd).  q = e0 * a via Wq, keys set in the cache /
    via Wk so that scores are known; positions chosen so RoPE is the identity
    on the used pair at position 0 and a known rotation at position 1."""
    H, G, hd = 1, 1, 2
    d = 2
    theta = 10000.0
    # x-hat = [1, 1] (h constant, eps 0, g 1)
    wq = np.array([[1.0, 1.0], [0.0, 0.0]], np.float32)      # q = [2, 0] before RoPE
    wk = np.array([[0.5, 0.0], [0.0, 0.0]], np.float32)      # k_new = [0.5, 0] before RoPE
    wv = np.array([[1.0, 0.0], [0.0, 0.0]], np.float32)      # v_new = [1, 0]
    dims, ly = attn_layer(orc, d, H, G, hd, wq, wk, wv, np.eye(2, dtype=np.float32))
    kc = np.zeros((1, 1, 4, hd), np.uint16)
    vc = np.zeros((1, 1, 4, hd), np.uint16)
    kc[0, 0, 0] = f32_to_bf16_bits([1.0, 0.0])    # k0 (already rotated, position 0)
    vc[0, 0, 0] = f32_to_bf16_bits([0.0, 2.0])    # v0
    kv = orc.OracleKV(kc, vc)
    out = orc.attn_block(dims, ly, np.ones((1, 2)), [1], kv)
    # at position 1 the pair rotates by angle 1 (i = 0): q' = 2(cos1, sin1),
    # k_new' = bf16(0.5 (cos1, sin1)) -> scores s0 = q'.k0/sqrt2, s1 = q'.k1'/sqrt2
    c, s = math.cos(1.0), math.sin(1.0)
    q = np.array([2 * c, 2 * s])
    k1 = np.array([bf16_value(orc.double_to_bf16(0.5 * c)), bf16_value(orc.double_to_bf16(0.5 * s))])
    s0 = q @ np.array([1.0, 0.0]) / math.sqrt(2)
    s1 = q @ k1 / math.sqrt(2)
    a0 = 1 / (1 + math.exp(s1 - s0))
    o = a0 * np.array([0.0, 2.0]) + (1 - a0) * np.array([1.0, 0.0])
    np.testing.assert_allclose(out[0], 1.0 + o, rtol=1e-12)


# ---------------------------------------------------------------- MoE block and router


def test_router_zero_logits_equal_bias_and_tie_break(orc):
    d, E, k = 16, 8, 3
    ly = mk_layer(orc, d, E, 8, 0, orc.F32, router_zero=True)
    dims = orc.make_dims(d, E, k, 8, 0, orc.F32)
    h = np.random.default_rng(8).standard_normal((2, d))
    logits, ids, w, margin = orc.route(dims, ly, h)
    np.testing.assert_array_equal(logits, 0.0)
    np.testing.assert_array_equal(ids, [[0, 1, 2], [0, 1, 2]])
    np.testing.assert_allclose(w, 1 / 3, rtol=1e-15)
    np.testing.assert_array_equal(margin, 0.0)
    bias = np.arange(E, dtype=np.float32) * 0.25
    ly_b = mk_layer(orc, d, E, 8, 0, orc.F32, router_zero=True, bias=bias)
    logits, ids, w, margin = orc.route(dims, ly_b, h)
    np.testing.assert_array_equal(logits, np.tile(bias.astype(np.float64), (2, 1)))
    np.testing.assert_array_equal(ids, [[7, 6, 5]] * 2)
    np.testing.assert_allclose(margin, 0.25, rtol=1e-15)


def test_moe_zero_gate_is_residual_identity(orc):
    d, E, k, F = 32, 8, 2, 16
    for dtype in (orc.F32, orc.BF16):
        ly = mk_layer(orc, d, E, F, 1, dtype, gate_zero=True)
        dims = orc.make_dims(d, E, k, F, 1, dtype)
        h = np.random.default_rng(9).standard_normal((3, d))
        _, ids, w, _ = orc.route(dims, ly, h)
        out = orc.moe_block(dims, ly, h, ids, w)
        np.testing.assert_array_equal(out, h)


def dense_swiglu(orc, ly, x):
    """Textbook dense SwiGLU FFN of expert 0, in numpy."""
    Wg, Wu, Wd = (widen(orc, a) for a in (ly.w_gate[0], ly.w_up[0], ly.w_down[0]))
    g = Wg @ x
    return Wd @ ((g / (1 + np.exp(-g))) * (Wu @ x))


@pytest.mark.parametrize("k", [2, 8])
def test_moe_identical_experts_reduce_to_dense_ffn(orc, k):
    """With identical experts the combine sum_e w_e y equals y (weights sum to
    one), so the block is h + dense SwiGLU(RMSNorm(h)), whatever the router;
    with k = E every expert is used."""
    d, E, F = 24, 8, 12
    ly = mk_layer(orc, d, E, F, 0, orc.F32, identical=True, std=0.2)
    dims = orc.make_dims(d, E, k, F, 0, orc.F32)
    rng = np.random.default_rng(11)
    h = rng.standard_normal((4, d))
    _, ids, w, _ = orc.route(dims, ly, h)
    out = orc.moe_block(dims, ly, h, ids, w)
    g2 = widen(orc, ly.arrays["g2"])
    for r in range(4):
        x = h[r] / np.sqrt(np.mean(h[r] ** 2) + 1e-6) * g2
        np.testing.assert_allclose(out[r], h[r] + dense_swiglu(orc, ly, x), rtol=1e-12, atol=1e-14)


def test_moe_dense_then_mask_equals_sparse(orc):
    d, E, k, F = 16, 8, 3, 8
    ly = mk_layer(orc, d, E, F, 1, orc.F32, std=0.3)
    dims = orc.make_dims(d, E, k, F, 1, orc.F32)
    rng = np.random.default_rng(12)
    h = rng.standard_normal((2, d))
    logits, ids, w, _ = orc.route(dims, ly, h)
    out = orc.moe_block(dims, ly, h, ids, w)
    g2 = widen(orc, ly.arrays["g2"])
    for r in range(2):
        x = h[r] / np.sqrt(np.mean(h[r] ** 2) + 1e-6) * g2
        p = np.exp(logits[r] - logits[r].max())
        p /= p.sum()
        mask = np.zeros(E)
        top = np.argsort(-logits[r], kind="stable")[:k]
        mask[top] = p[top] / p[top].sum()
        ys = np.stack([orc.expert(ly.w_gate[e], ly.w_up[e], ly.w_down[e], x) for e in range(E)])
        shared = orc.expert(ly.s_gate[0], ly.s_up[0], ly.s_down[0], x)
        np.testing.assert_allclose(out[r], h[r] + mask @ ys + shared, rtol=1e-12, atol=1e-14)


def test_moe_zero_routed_down_leaves_shared_only(orc):
    d, E, k, F = 16, 4, 2, 8
    ly = mk_layer(orc, d, E, F, 1, orc.F32, down_zero=True, std=0.3)
    dims = orc.make_dims(d, E, k, F, 1, orc.F32)
    h = np.random.default_rng(13).standard_normal((1, d))
    _, ids, w, _ = orc.route(dims, ly, h)
    out = orc.moe_block(dims, ly, h, ids, w)
    g2 = widen(orc, ly.arrays["g2"])
    x = h[0] / np.sqrt(np.mean(h[0] ** 2) + 1e-6) * g2
    Wg, Wu, Wd = (widen(orc, a) for a in (ly.s_gate[0], ly.s_up[0], ly.s_down[0]))
    gg = Wg @ x
    np.testing.assert_allclose(out[0], h[0] + Wd @ ((gg / (1 + np.exp(-gg))) * (Wu @ x)), rtol=1e-12)


def test_moe_missing_unselected_expert_is_not_touched(orc):
    """Only the selected experts are read: the others may be absent."""
    d, E, k, F = 16, 8, 2, 8
    ly = mk_layer(orc, d, E, F, 0, orc.F32)
    dims = orc.make_dims(d, E, k, F, 0, orc.F32)
    h = np.random.default_rng(14).standard_normal((1, d))
    _, ids, w, _ = orc.route(dims, ly, h)
    full = orc.moe_block(dims, ly, h, ids, w)
    keep = set(ids[0])
    ly.set_experts([a if e in keep else None for e, a in enumerate(ly.w_gate)],
                   [a if e in keep else None for e, a in enumerate(ly.w_up)],
                   [a if e in keep else None for e, a in enumerate(ly.w_down)])
    np.testing.assert_array_equal(orc.moe_block(dims, ly, h, ids, w), full)
    ly.set_experts([None] * E, [None] * E, [None] * E)
    with pytest.raises(RuntimeError):
        orc.moe_block(dims, ly, h, ids, w)


# ---------------------------------------------------------------- whole step


def tiny_stack(orc, L=2, d=32, E=8, k=2, F=16, n_shared=1, dtype=0, attn=False, seed=0):
    rng = np.random.default_rng(seed)
    layers = []
    for _ in range(L):
        ly = mk_layer(orc, d, E, F, n_shared, dtype, rng=rng, std=0.2)
        if attn:
            H, G, hd = 4, 2, 8
            ly.arrays.update(g1=ly.arrays["g2"].copy(),
                             wq=(rng.standard_normal((H * hd, d)) * 0.2).astype(np.float32),
                             wk=(rng.standard_normal((G * hd, d)) * 0.2).astype(np.float32),
                             wv=(rng.standard_normal((G * hd, d)) * 0.2).astype(np.float32),
                             wo=(rng.standard_normal((d, H * hd)) * 0.2).astype(np.float32))
            ly._refresh()
        layers.append(ly)
    if attn:
        dims = orc.make_dims(d, E, k, F, n_shared, dtype, n_heads=4, n_kv_heads=2, head_dim=8, rope_theta=1e4)
    else:
        dims = orc.make_dims(d, E, k, F, n_shared, dtype)
    return dims, layers


def test_forward_equals_staged_calls(orc):
    dims, layers = tiny_stack(orc)
    h = np.random.default_rng(15).standard_normal((2, 32)).astype(np.float32)
    out, tr = orc.forward(dims, layers, h)
    x = h.astype(np.float64)
    for l, ly in enumerate(layers):
        lg, ids, w, mg = orc.route(dims, ly, x)
        np.testing.assert_array_equal(ids, tr["ids"][l])
        x = orc.moe_block(dims, ly, x, ids, w)
    np.testing.assert_array_equal(out, x.astype(np.float32))


def test_forward_batch_invariance(orc):
    dims, layers = tiny_stack(orc, seed=3)
    h = np.random.default_rng(16).standard_normal((4, 32)).astype(np.float32)
    out, _ = orc.forward(dims, layers, h)
    for r in range(4):
        o1, _ = orc.forward(dims, layers, h[r:r + 1])
        np.testing.assert_array_equal(o1[0], out[r])


def attn_stack_with_cache(orc, M, rows_per_seq, past, seed):
    dims, layers = tiny_stack(orc, attn=True, seed=seed)
    rng = np.random.default_rng(seed + 100)
    n_seq = M // rows_per_seq
    cap = past + rows_per_seq + 2
    kvs = []
    for _ in layers:
        k = (rng.standard_normal((n_seq, 2, cap, 8))).astype(np.float32)
        v = (rng.standard_normal((n_seq, 2, cap, 8))).astype(np.float32)
        tobf = lambda a: ((a.view(np.uint32) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
        kvs.append(orc.OracleKV(tobf(k), tobf(v)))
    return dims, layers, kvs


def test_verify_rows_equal_sequential_decode(orc):
    """A verify pass of R rows at positions p..p+R-1 equals R single-row
    decode steps in sequence (each writes its row before the next attends)."""
    R, past = 4, 6
    dims, layers, kvs = attn_stack_with_cache(orc, R, R, past, seed=21)
    _, _, kvs_seq = attn_stack_with_cache(orc, R, R, past, seed=21)
    h = np.random.default_rng(22).standard_normal((R, 32)).astype(np.float32)
    out, _ = orc.forward(dims, layers, h, positions=[past + r for r in range(R)], kvs=kvs, rows_per_seq=R)
    for r in range(R):
        o1, _ = orc.forward(dims, layers, h[r:r + 1], positions=[past + r], kvs=kvs_seq, rows_per_seq=1)
        np.testing.assert_allclose(o1[0], out[r], rtol=1e-6, atol=1e-6)
    for a, b in zip(kvs, kvs_seq):
        np.testing.assert_array_equal(a.k, b.k)
        np.testing.assert_array_equal(a.v, b.v)


def test_speculative_rollback_leaves_no_trace(orc):
    """Speculative decoding: a verify pass at p..p+R-1 whose drafts after the
    first are rejected is followed by a pass at p+2.  Its rows write their own
    K/V at p+2.. before attending, so the rejected drafts left at p+2, p+3 are
    never read: the second pass is bit-identical to one over a cache that
    never held them."""
    R, past = 4, 6
    dims, layers, kvs = attn_stack_with_cache(orc, R, R, past, seed=41)
    _, _, fresh = attn_stack_with_cache(orc, R, R, past, seed=41)
    rng = np.random.default_rng(42)
    h1 = rng.standard_normal((R, 32)).astype(np.float32)
    h2 = rng.standard_normal((R, 32)).astype(np.float32)
    orc.forward(dims, layers, h1, positions=[past + r for r in range(R)], kvs=kvs, rows_per_seq=R)
    p1 = past + 2  # token p and one draft accepted
    after = [orc.OracleKV(kv.k.copy(), kv.v.copy()) for kv in kvs]
    out_a, _ = orc.forward(dims, layers, h2, positions=[p1 + r for r in range(R)], kvs=after, rows_per_seq=R)
    clean = [orc.OracleKV(kv.k.copy(), kv.v.copy()) for kv in kvs]
    for c, f0 in zip(clean, fresh):
        c.k[:, :, p1:past + R] = f0.k[:, :, p1:past + R]
        c.v[:, :, p1:past + R] = f0.v[:, :, p1:past + R]
    out_b, _ = orc.forward(dims, layers, h2, positions=[p1 + r for r in range(R)], kvs=clean, rows_per_seq=R)
    np.testing.assert_array_equal(out_a, out_b)
    # the rejected positions did hold the drafts (the check above is not vacuous)
    assert not np.array_equal(kvs[0].k[:, :, p1:past + R], fresh[0].k[:, :, p1:past + R])


def test_batched_sequences_equal_single(orc):
    """Rows of different sequences do not interact."""
    M, past = 3, 5
    dims, layers, kvs = attn_stack_with_cache(orc, M, 1, past, seed=31)
    h = np.random.default_rng(32).standard_normal((M, 32)).astype(np.float32)
    out, _ = orc.forward(dims, layers, h, positions=[past] * M, kvs=kvs, rows_per_seq=1)
    for r in range(M):
        _, _, kv1 = attn_stack_with_cache(orc, M, 1, past, seed=31)
        sub = [orc.OracleKV(kv.k[r:r + 1].copy(), kv.v[r:r + 1].copy()) for kv in kv1]
        o1, _ = orc.forward(dims, layers, h[r:r + 1], positions=[past], kvs=sub, rows_per_seq=1)
        np.testing.assert_array_equal(o1[0], out[r])


def test_route_margin_brute_force(orc):
    """margin = k-th largest minus (k+1)-th largest logit (sorted by numpy)."""
    d, E = 16, 8
    rng = np.random.default_rng(40)
    for k in (1, 2, 3, 7, 8):
        ly = mk_layer(orc, d, E, 8, 0, orc.F32, rng=rng, std=0.5)
        dims = orc.make_dims(d, E, k, 8, 0, orc.F32)
        h = rng.standard_normal((3, d))
        logits, ids, _, margin = orc.route(dims, ly, h)
        for r in range(3):
            srt = np.sort(logits[r])[::-1]
            expect = math.inf if k == E else srt[k - 1] - srt[k]
            assert margin[r] == expect
            assert set(ids[r]) == set(np.argsort(-logits[r], kind="stable")[:k])


def test_moe_norm_uses_its_own_gain(orc):
    """With a silent attention block (all projections zero) and a zero
    attention gain, the layer equals the MoE-only layer: the MoE block must
    normalise with its own gain, not the attention one."""
    d, E, k, F = 32, 8, 2, 16
    dims_m, layers = tiny_stack(orc, L=1, d=d, E=E, k=k, F=F, seed=41)
    ly = layers[0]
    H, G, hd = 4, 2, 8
    ly_a = orc.OracleLayer(ly.arrays["g2"], ly.arrays["wr"], None, ly.w_gate, ly.w_up, ly.w_down,
                           ly.s_gate, ly.s_up, ly.s_down, g1=np.zeros(d, np.float32),
                           wq=np.zeros((H * hd, d), np.float32), wk=np.zeros((G * hd, d), np.float32),
                           wv=np.zeros((G * hd, d), np.float32), wo=np.zeros((d, H * hd), np.float32))
    dims_a = orc.make_dims(d, E, k, F, 1, orc.F32, n_heads=H, n_kv_heads=G, head_dim=hd, rope_theta=1e4)
    kv = orc.OracleKV(np.zeros((1, G, 4, hd), np.uint16), np.zeros((1, G, 4, hd), np.uint16))
    h = np.random.default_rng(42).standard_normal((1, d)).astype(np.float32)
    out_a, _ = orc.forward(dims_a, [ly_a], h, positions=[2], kvs=[kv])
    out_m, _ = orc.forward(dims_m, [ly], h)
    np.testing.assert_array_equal(out_a, out_m)
    assert not np.array_equal(out_m, h)


# ---------------------------------------------------------------- MLA attention
# The reading: multi-head latent attention as published (DeepSeek-V2 report,
# section 2.1), in the absorbed form a decode step uses (oracle.h).


def _bf16_random(rng, shape, scale=1.0):
    """bf16 bit patterns of N(0, scale^2) draws (truncated float32: exact values)."""
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _mha_row(q_nope, q_rope, c, k_r, W_uk, W_uv, scale):
    """Textbook attention of one head over explicit keys and values built from
    the latents: key_j = (W_uk c_j, k_r_j), value_j = W_uv c_j."""
    keys = np.concatenate([c @ W_uk.T, k_r], axis=1)  # [P][d_nope + Dr]
    vals = c @ W_uv.T                                  # [P][d_v]
    s = scale * (keys @ np.concatenate([q_nope, q_rope]))
    a = np.exp(s - s.max())
    a /= a.sum()
    return a @ vals


def test_mla_absorbed_equals_explicit_heads(orc):
    """The absorbed form over the latent cache, projected by W_UV, equals
    per-head attention over explicitly decompressed keys and values (the
    identity MLA decode rests on).  Catches a dropped rotary part of the
    score, a wrong scale, values that include the rotary columns, and an
    off-by-one in the attended range."""
    rng = np.random.default_rng(11)
    H, Dc, Dr, dn, dv, n_seq, cap = 3, 24, 8, 12, 10, 2, 11
    cache = _bf16_random(rng, (n_seq, cap, Dc + Dr))
    cf = _bf16_to_f64(cache)
    W_uk = rng.standard_normal((H, dn, Dc)) * 0.3
    W_uv = rng.standard_normal((H, dv, Dc)) * 0.3
    positions = [4, 10, 0, 7]  # rows 0, 1 in sequence 0; rows 2, 3 in sequence 1
    rps, scale = 2, 1.0 / math.sqrt(dn + Dr)
    q_nope = rng.standard_normal((len(positions), H, dn))
    q_rope = rng.standard_normal((len(positions), H, Dr))
    q = np.concatenate([np.einsum("hnc,rhn->rhc", W_uk, q_nope), q_rope], axis=2)
    out = orc.mla_attention(q, cache, positions, Dc, scale, rows_per_seq=rps)
    for r, p in enumerate(positions):
        seq = r // rps
        c, k_r = cf[seq, :p + 1, :Dc], cf[seq, :p + 1, Dc:]
        for h in range(H):
            want = _mha_row(q_nope[r, h], q_rope[r, h], c, k_r, W_uk[h], W_uv[h], scale)
            np.testing.assert_allclose(W_uv[h] @ out[r, h], want, rtol=1e-11, atol=1e-12)


def test_mla_zero_query_averages_the_latents(orc):
    """q = 0: every score is 0, the weights are uniform over positions
    0..pos, and the output is the mean of those latents (closed form).
    Catches a softmax over the whole capacity or including position pos + 1."""
    rng = np.random.default_rng(12)
    Dc, Dr, cap = 16, 4, 9
    cache = _bf16_random(rng, (1, cap, Dc + Dr))
    cf = _bf16_to_f64(cache)
    for p in (0, 3, cap - 1):
        out = orc.mla_attention(np.zeros((1, 2, Dc + Dr)), cache, [p], Dc, 0.7)
        want = cf[0, :p + 1, :Dc].mean(axis=0)
        np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)
        np.testing.assert_array_equal(out[0, 0], out[0, 1])


def test_mla_first_position_returns_its_latent(orc):
    """At position 0 the only weight is 1: the output is the latent part of
    cache row 0 exactly, whatever the query."""
    rng = np.random.default_rng(13)
    Dc, Dr = 16, 4
    cache = _bf16_random(rng, (1, 5, Dc + Dr))
    out = orc.mla_attention(rng.standard_normal((1, 3, Dc + Dr)) * 5, cache, [0], Dc, 1.3)
    for h in range(3):
        np.testing.assert_array_equal(out[0, h], _bf16_to_f64(cache)[0, 0, :Dc])


def test_mla_reads_no_position_after_its_own(orc):
    """Cache rows after a row's position do not change its output (bitwise);
    the row at its position does."""
    rng = np.random.default_rng(14)
    Dc, Dr, cap, p = 16, 4, 12, 6
    cache = _bf16_random(rng, (1, cap, Dc + Dr))
    q = rng.standard_normal((1, 2, Dc + Dr))
    base = orc.mla_attention(q, cache, [p], Dc, 0.5)
    later = cache.copy()
    later[0, p + 1:] = _bf16_random(rng, (cap - p - 1, Dc + Dr))
    np.testing.assert_array_equal(orc.mla_attention(q, later, [p], Dc, 0.5), base)
    own = cache.copy()
    own[0, p] = _bf16_random(rng, (Dc + Dr,))
    assert not np.array_equal(orc.mla_attention(q, own, [p], Dc, 0.5), base)


def test_mla_dominant_score_selects_its_row(orc):
    """A query aligned with one cache row and a large scale: that row's weight
    is 1 to double precision, so the output is its latent (the softmax is
    taken with the maximum subtracted; without it the exponentials overflow)."""
    rng = np.random.default_rng(15)
    Dc, Dr, cap, p, j = 16, 4, 10, 8, 5
    cache = _bf16_random(rng, (1, cap, Dc + Dr))
    cf = _bf16_to_f64(cache)
    q = cf[0, j][None, None, :] * 1.0
    gaps = cf[0, j] @ cf[0, j] - cf[0, :p + 1] @ cf[0, j]
    gaps[j] = np.inf
    scale = 800.0 / gaps.min()  # every other score is at least 800 below row j's
    out = orc.mla_attention(q, cache, [p], Dc, scale)
    np.testing.assert_allclose(out[0, 0], cf[0, j, :Dc], rtol=0, atol=1e-12 * np.abs(cf[0, j, :Dc]).max())
