"""Pins for the oracle's shared expert (dense_mlp).

- Brute force on a tiny problem: every gate/up/down sum in exact rationals, the BF16
  roundings of the pages' buffers applied stage by stage.
- One-hot weights with non-square shapes: each output is a closed form of one gate and
  one up input, so a transposed operand, swapped gate/up or a wrong index fails.
- The routed layer with one expert, top_k 1 and weight 1, whose NVFP4 weights decode to
  the dense weights, gives the same bits (a different code path: dequant, align, gather,
  combine).
- Rows are independent (sampled checks at full size rely on it).
"""

from fractions import Fraction
import math

import numpy as np
import pytest
import scipy.special

from oracle import codecs, moe
import workloads as wl


def _bf16(bits):
    return codecs.bf16_bits_to_f64(bits)


def _tiny(seed, t=3, h=8, i=5, scale=1.0):
    rng = np.random.default_rng(seed)
    x = _bf16(wl.bf16_normal(rng, (t, h)))
    g = _bf16(wl.bf16_normal(rng, (i, h))) * scale
    u = _bf16(wl.bf16_normal(rng, (i, h))) * scale
    d = _bf16(wl.bf16_normal(rng, (h, i)))
    return x, g, u, d


def _dot(row, col):
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(row, col)), Fraction(0))


def _swiglu_float(g, u, limit):
    gc = min(g, limit)
    uc = min(max(u, -limit), limit)
    return gc / (1.0 + math.exp(-gc)) * uc


@pytest.mark.parametrize("scale", [1.0, 8.0])  # 8: many gate/up values beyond the clamp
def test_dense_mlp_brute_force_exact(scale):
    x, g, u, d = _tiny(3, scale=scale)
    limit = 7.0
    out, mid = moe.dense_mlp(x, g, u, d, limit, "exact")
    t, h = x.shape
    i_w = g.shape[0]
    for r in range(t):
        act = []
        for j in range(i_w):
            gv, uv = _dot(x[r], g[j]), _dot(x[r], u[j])
            assert mid["gate"][r, j] == float(gv) and mid["up"][r, j] == float(uv)
            act.append(_swiglu_float(float(gv), float(uv), limit))
        assert np.allclose(mid["act"][r], act, rtol=1e-14, atol=0)
        for c in range(h):
            ref = sum(a * float(d[c, j]) for j, a in enumerate(act))
            assert out[r, c] == pytest.approx(ref, rel=1e-12, abs=1e-15)


def test_dense_mlp_brute_force_bf16_buffers():
    x, g, u, d = _tiny(4, t=4, h=16, i=6, scale=2.0)
    out, mid = moe.dense_mlp(x, g, u, d, 7.0, "bf16w")
    t, h = x.shape
    for r in range(t):
        for j in range(g.shape[0]):
            # the exact sums are doubles here (few short BF16 products), so rounding them
            # to BF16 is deterministic: compare bits
            assert mid["gate"][r, j] == codecs.round_bf16(float(_dot(x[r], g[j])))
            assert mid["up"][r, j] == codecs.round_bf16(float(_dot(x[r], u[j])))
        # the activation: one BF16 rounding of the clamped SwiGLU (within one BF16 ulp of
        # the brute-force value, whose last double bit may differ)
        act = np.array([_swiglu_float(mid["gate"][r, j], mid["up"][r, j], 7.0)
                        for j in range(g.shape[0])])
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(act), 1e-300))) - 7)
        assert np.all(np.abs(mid["act"][r] - act) <= ulp)
        assert np.all(codecs.round_bf16(mid["act"][r]) == mid["act"][r])
        for c in range(h):  # the output: the exact down sum of that activation, rounded
            assert out[r, c] == codecs.round_bf16(float(_dot(mid["act"][r], d[c])))


def test_dense_mlp_one_hot_closed_form():
    rng = np.random.default_rng(11)
    t, h, i_w, limit = 7, 24, 10, 3.0
    x = _bf16(wl.bf16_normal(rng, (t, h))) * 2.0
    p = rng.permutation(h)[:i_w]  # gate row j picks x[:, p[j]]
    q = rng.permutation(h)[:i_w]  # up row j picks 2 x[:, q[j]]
    g = np.zeros((i_w, h))
    g[np.arange(i_w), p] = 1.0
    u = np.zeros((i_w, h))
    u[np.arange(i_w), q] = 2.0
    d = np.zeros((h, i_w))
    d[np.arange(h), np.arange(h) % i_w] = 1.0  # output column c copies act[:, c % I]
    out, _ = moe.dense_mlp(x, g, u, d, limit, "exact")
    gv = np.minimum(x[:, p], limit)
    uv = np.clip(2.0 * x[:, q], -limit, limit)
    act = gv * scipy.special.expit(gv) * uv
    assert np.allclose(out, act[:, np.arange(h) % i_w], rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("mode", ["exact", "bf16w"])
def test_dense_mlp_equals_routed_layer_with_one_expert(mode):
    rng = np.random.default_rng(12)
    t, h, mi = 9, 64, 32
    x = _bf16(wl.bf16_normal(rng, (t, h)))
    gu = wl.random_nvfp4(rng, 2 * mi, h)
    dn = wl.random_nvfp4(rng, h, mi)
    s2gu, s2dn = np.float32(0.75), np.float32(1.25)
    # the routed layer's weights as the dense MLP's operands (the layer decodes them in
    # the same mode)
    w_gu = moe.dequant(gu[0], gu[1], float(s2gu), mode)
    w_dn = moe.dequant(dn[0], dn[1], float(s2dn), mode)
    ids = np.zeros((t, 1), np.int32)
    wts = np.ones((t, 1), np.float32)
    ref, _ = moe.moe_layer(x, ids, wts, [gu], [dn], np.array([s2gu]), np.array([s2dn]),
                           mi, 7.0, mode)
    out, _ = moe.dense_mlp(x, w_gu[:mi], w_gu[mi:], w_dn, 7.0, mode)
    if mode == "bf16w":
        assert np.array_equal(out, ref)
    else:
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_dense_mlp_rows_are_independent():
    w = wl.custom("dense_rows", 77, rows=12, num_experts=1, top_k=1, hidden=64,
                  moe_intermediate=32)
    x = _bf16(wl.activations(w))
    g, u, d = (_bf16(b) for b in wl.shared_expert(w))
    full, _ = moe.dense_mlp(x, g, u, d, 7.0, "bf16w")
    rows = [0, 5, 11]
    part, _ = moe.dense_mlp(x[rows], g, u, d, 7.0, "bf16w")
    assert np.array_equal(part, full[rows])


def test_shared_expert_recipe_shapes_and_scale():
    w = wl.WORKLOADS["layer_e64"]
    g, u, d = wl.shared_expert(w)
    assert g.shape == (768, 2048) and u.shape == (768, 2048) and d.shape == (2048, 768)
    assert g.dtype == np.uint16
    assert abs(np.std(_bf16(g)) * math.sqrt(2048) - 1.0) < 0.01
    assert abs(np.std(_bf16(d)) * math.sqrt(768) - 1.0) < 0.01
    assert not np.array_equal(g, u)
