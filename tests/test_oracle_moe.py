"""Pins for the oracle's dequant, align, grouped GEMM, SwiGLU, combine and layer.

Each test checks the oracle against something other than itself: one-hot layout
patterns with known answers, torch's own FP8/FP32/BF16 arithmetic, numpy's stable
argsort, scipy's logistic function, closed forms, and brute-force loops in exact
rational arithmetic on tiny inputs.
"""

from fractions import Fraction
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import codecs, moe
import workloads as wl

E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX FP4 (tests/golden/ocp_formats.json)


def _spec_nibble_value(q):
    v = E2M1_SPEC[q & 7]
    return -v if q & 8 else v


# ------------------------------------------------------------------------------ dequant

def _pack(nib):
    """[N, K] nibbles -> [N, K/2] bytes, even k in the low nibble (written out per byte)."""
    n, k = nib.shape
    out = np.zeros((n, k // 2), dtype=np.uint8)
    for j in range(k // 2):
        out[:, j] = (nib[:, 2 * j] & 0xF) | ((nib[:, 2 * j + 1] & 0xF) << 4)
    return out


def test_dequant_one_hot_layout():
    # Row n has a single 1.0 (nibble 2) at k = pi(n); scale 1.0 (0x38), scale2 = 1.
    rng = np.random.default_rng(0)
    n_rows, k_total = 48, 96
    pi = rng.integers(0, k_total, n_rows)
    nib = np.zeros((n_rows, k_total), dtype=np.uint8)
    nib[np.arange(n_rows), pi] = 2
    packed = _pack(nib)
    # check the byte/nibble convention directly on the raw bytes as well
    for n in range(n_rows):
        byte = packed[n, pi[n] // 2]
        assert byte == (0x02 if pi[n] % 2 == 0 else 0x20)
    scales = np.full((n_rows, k_total // 16), 0x38, dtype=np.uint8)
    for mode in ("exact", "bf16w"):
        w = moe.dequant(packed, scales, 1.0, mode)
        expect = np.zeros((n_rows, k_total))
        expect[np.arange(n_rows), pi] = 1.0
        assert np.array_equal(w, expect)


def test_dequant_scale_index_pattern():
    # Distinct power-of-two scale per (row, group): 2**((n + 3 g) % 9 - 4); all nibbles 1.0.
    n_rows, k_total = 20, 128
    nib = np.full((n_rows, k_total), 2, dtype=np.uint8)
    exps = np.array([[(n + 3 * g) % 9 - 4 for g in range(k_total // 16)] for n in range(n_rows)])
    codes = ((exps + 7) << 3).astype(np.uint8)  # E4M3FN: exponent field, mantissa 0
    w = moe.dequant(_pack(nib), codes, 0.5, "exact")
    for n in range(n_rows):
        for k in range(k_total):
            assert w[n, k] == 0.5 * 2.0 ** exps[n, k // 16]


def test_dequant_matches_torch_fp32_arithmetic():
    # Same formula evaluated by torch: codebook value (spec table) times torch's FP8
    # decode in FP32, times scale2 in FP32, then torch's BF16 conversion.
    rng = np.random.default_rng(3)
    n_rows, k_total = 64, 256
    packed, scales = wl.random_nvfp4(rng, n_rows, k_total)
    scales[0, 0] = 0x00  # zero scale
    scales[1, 1] = 0x01  # smallest subnormal
    scales[2, 2] = 0x7E  # 448
    for s2 in (np.float32(1.3719), np.float32(0.51), np.float32(1.0)):
        nib = np.zeros((n_rows, k_total), dtype=np.int64)
        nib[:, 0::2] = packed & 0xF
        nib[:, 1::2] = packed >> 4
        v = torch.tensor([[_spec_nibble_value(int(q)) for q in row] for row in nib],
                         dtype=torch.float32)
        d = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float32)
        d = d.repeat_interleave(16, dim=1)
        w32 = (v * d) * torch.tensor(float(s2), dtype=torch.float32)
        got_exact = moe.dequant(packed, scales, float(s2), "exact")
        assert np.array_equal(got_exact, w32.double().numpy())
        got_bits = moe.dequant_bf16_bits(packed, scales, float(s2))
        ref_bits = w32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got_bits, ref_bits)


def test_dequant_every_code_and_nibble_matches_torch():
    # Row n: E4M3 code n in every block (zero, subnormal, negative, 448 and the two NaN
    # codes included), nibbles (k + n) % 16; against torch's FP8 decode and FP32/BF16
    # arithmetic of the same formula, NaN where torch gives NaN.
    k_total = 64
    nib = ((np.arange(k_total)[None, :] + np.arange(256)[:, None]) % 16).astype(np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k_total // 16, axis=1)
    packed = _pack(nib)
    v = torch.tensor([[_spec_nibble_value(int(q)) for q in row] for row in nib],
                     dtype=torch.float32)
    d = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float32)
    for s2 in (np.float32(1.3719), np.float32(0.51)):
        w32 = (v * d.repeat_interleave(16, dim=1)) * torch.tensor(float(s2), dtype=torch.float32)
        ref = w32.to(torch.bfloat16).double().numpy()
        got = moe.dequant(packed, scales, float(s2), "bf16w")
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        assert np.array_equal(np.isnan(got).all(axis=1), np.isin(np.arange(256), [0x7F, 0xFF]))
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok], ref[ok])


def test_dequant_product_order_matters():
    # (v * d) * s2 and v * (d * s2) differ after BF16 rounding for a few inputs per
    # million; the oracle must follow the grouped GEMM's order (scale2 multiplied into
    # the dequant product), so find such an input with torch and check the oracle on it.
    rng = np.random.default_rng(5)
    count = 1 << 23
    v = torch.tensor([1.5, 3.0, 6.0], dtype=torch.float32)[torch.from_numpy(rng.integers(0, 3, count))]
    codes = rng.integers(0x20, 0x50, count).astype(np.uint8)
    d = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    s2 = torch.from_numpy(rng.uniform(0.5, 2, count).astype(np.float32))
    a = ((v * d) * s2).to(torch.bfloat16)
    b = (v * (d * s2)).to(torch.bfloat16)
    diff = torch.nonzero(a != b).flatten()
    assert diff.numel() > 0
    i = int(diff[0])
    q = {1.5: 0x3, 3.0: 0x5, 6.0: 0x7}[float(v[i])]
    packed = np.full((1, 8), q | (q << 4), dtype=np.uint8)
    scales = np.full((1, 1), codes[i], dtype=np.uint8)
    got = moe.dequant(packed, scales, float(s2[i]), "bf16w")
    assert np.all(got == float(a[i])) and float(a[i]) != float(b[i])


# ------------------------------------------------------------------------------ align

def _align_by_argsort(ids, num_experts):
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < num_experts)
    key = np.where(valid, flat, num_experts)  # invalid slots sort last
    perm = np.argsort(key, kind="stable")
    n_valid = int(valid.sum())
    perm = perm[:n_valid]
    ttp = np.full(flat.size, -1, dtype=np.int64)
    ttp[perm] = np.arange(n_valid)
    offsets = np.concatenate([[0], np.cumsum(np.bincount(flat[valid], minlength=num_experts))])
    st = np.full(flat.size, -1)
    se = np.full(flat.size, -1)
    st[:n_valid] = perm // ids.shape[1]
    se[:n_valid] = flat[perm]
    return offsets, st, se, ttp.reshape(ids.shape)


@pytest.mark.parametrize("rows,top_k,num_experts,bad", [
    (64, 8, 16, 0.0), (256, 8, 64, 0.0), (37, 3, 5, 0.1), (1, 1, 1, 0.0),
    (200, 6, 300, 0.05), (16, 8, 256, 0.2)])
def test_align_matches_stable_argsort(rows, top_k, num_experts, bad):
    rng = np.random.default_rng(rows * 1000 + num_experts)
    ids = np.stack([rng.permutation(max(num_experts, top_k))[:top_k] for _ in range(rows)])
    ids = ids.astype(np.int32)
    mask = rng.random(ids.shape) < bad
    ids[mask] = rng.choice([-1, num_experts, num_experts + 7, -5], size=int(mask.sum()))
    got = moe.align(ids, num_experts)
    offsets, st, se, ttp = _align_by_argsort(ids, num_experts)
    assert np.array_equal(got["expert_offsets"], offsets)
    assert np.array_equal(got["sorted_token_ids"], st)
    assert np.array_equal(got["sorted_expert_ids"], se)
    assert np.array_equal(got["token_to_perm"], ttp)
    n_valid = int(((ids >= 0) & (ids < num_experts)).sum())
    assert got["n_invalid"] == ids.size - n_valid
    # invariants: slot counts sum to the valid slots (rows*top_k with no invalid ids),
    # expert ids non-decreasing, segments ascending in token, token_to_perm a bijection
    assert got["expert_offsets"][-1] == n_valid
    assert np.all(np.diff(got["sorted_expert_ids"][:n_valid]) >= 0)
    for e in range(num_experts):
        lo, hi = got["expert_offsets"][e], got["expert_offsets"][e + 1]
        assert np.all(np.diff(got["sorted_token_ids"][lo:hi]) >= 0)
        assert np.all(got["sorted_expert_ids"][lo:hi] == e)
    t = got["token_to_perm"].reshape(-1)
    assert sorted(t[t >= 0].tolist()) == list(range(n_valid))


def test_align_brute_force_tiny():
    ids = np.array([[2, 0], [0, 1], [2, 2], [-1, 0]], dtype=np.int32)
    got = moe.align(ids, 3)
    # by hand: slots t=0..7 -> experts [2,0,0,1,2,2,-1,0]
    assert got["expert_offsets"].tolist() == [0, 3, 4, 7]
    assert got["sorted_token_ids"].tolist() == [0, 1, 3, 1, 0, 2, 2, -1]
    assert got["sorted_expert_ids"].tolist() == [0, 0, 0, 1, 2, 2, 2, -1]
    assert got["token_to_perm"].tolist() == [[4, 0], [1, 3], [5, 6], [-1, 2]]
    assert got["n_invalid"] == 1


# ------------------------------------------------------------------------------ GEMM

def _tiny_problem(seed, rows=6, top_k=2, num_experts=4, n=16, k=32, null=()):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    x_bits = wl.bf16_normal(rng, (rows, k))
    experts = []
    for e in range(num_experts):
        experts.append(None if e in null else wl.random_nvfp4(rng, n, k))
    s2 = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    return ids, x_bits, experts, s2


def _exact_weight(packed, scales, s2, n, k, bf16w):
    """Brute force one weight: torch FP32 arithmetic, optional torch BF16 rounding."""
    byte = int(packed[n, k // 2])
    q = (byte >> 4) if (k % 2) else (byte & 0xF)
    v = torch.tensor(_spec_nibble_value(q), dtype=torch.float32)
    d = torch.tensor([int(scales[n, k // 16])], dtype=torch.uint8).view(torch.float8_e4m3fn)
    w = (v * d.to(torch.float32)[0]) * torch.tensor(float(s2), dtype=torch.float32)
    if bf16w:
        w = w.to(torch.bfloat16)
    return Fraction(float(w))


@pytest.mark.parametrize("mode", ["exact", "bf16w"])
def test_grouped_gemm_brute_force_exact_rationals(mode):
    ids, x_bits, experts, s2 = _tiny_problem(21, null=(1,))
    rows, top_k = ids.shape
    n, k = 16, 32
    x = codecs.bf16_bits_to_f64(x_bits)
    al = moe.align(ids, len(experts))
    out = np.full((rows * top_k, n), -7.0)
    moe.grouped_gemm(x, al["sorted_token_ids"], experts, s2, al["expert_offsets"], out, mode)
    xt = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    for s in range(rows * top_k):
        e = int(al["sorted_expert_ids"][s])
        tok = int(al["sorted_token_ids"][s])
        if experts[e] is None:
            assert np.all(out[s] == -7.0)  # null expert: row untouched
            continue
        packed, scales = experts[e]
        for nn in range(n):
            acc = sum(Fraction(float(xt[tok, kk])) *
                      _exact_weight(packed, scales, s2[e], nn, kk, mode == "bf16w")
                      for kk in range(k))
            assert out[s, nn] == pytest.approx(float(acc), rel=1e-13, abs=1e-13)


def test_grouped_gemm_all_ones_is_row_sum():
    rows, k, n = 9, 64, 32
    rng = np.random.default_rng(4)
    x_bits = wl.bf16_normal(rng, (rows, k))
    x = codecs.bf16_bits_to_f64(x_bits)
    packed = np.full((n, k // 2), 0x22, dtype=np.uint8)  # both nibbles 1.0
    scales = np.full((n, k // 16), 0x38, dtype=np.uint8)
    offsets = np.array([0, 4, 4, rows])
    out = np.zeros((rows, n))
    moe.grouped_gemm(x, None, [(packed, scales), None, (packed, scales)],
                     np.ones(3, np.float32), offsets, out, "bf16w")
    xt = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double()
    ref = xt.sum(dim=1).numpy()
    assert np.allclose(out, ref[:, None], rtol=1e-15, atol=1e-15)


def test_grouped_gemm_one_hot_picks_gathered_column():
    rng = np.random.default_rng(8)
    rows, k, n, num_experts = 10, 64, 32, 3
    x = codecs.bf16_bits_to_f64(wl.bf16_normal(rng, (rows, k)))
    experts, pis = [], []
    for e in range(num_experts):
        pi = rng.integers(0, k, n)
        nib = np.zeros((n, k), np.uint8)
        nib[np.arange(n), pi] = 2
        experts.append((_pack(nib), np.full((n, k // 16), 0x38, np.uint8)))
        pis.append(pi)
    gather = rng.integers(0, rows, 15)
    offsets = np.array([0, 5, 9, 15])
    out = np.zeros((15, n))
    moe.grouped_gemm(x, gather, experts, np.ones(num_experts, np.float32), offsets, out, "exact")
    for e in range(num_experts):
        for s in range(offsets[e], offsets[e + 1]):
            assert np.array_equal(out[s], x[gather[s], pis[e]])


# ------------------------------------------------------------------------------ SwiGLU

def test_swiglu_closed_forms():
    limit = 7.0
    silu_l = limit * scipy.special.expit(limit)  # 6.99361...
    g = np.array([7.0, 9.0, 100.0, 0.0, -3.0, 1.0, 1.0, 1.0])
    u = np.array([2.0, -1.5, 3.0, 5.0, 2.0, 8.0, -9.0, 0.0])
    got = moe.swiglu_clamp(g, u, limit)
    assert got[0] == pytest.approx(silu_l * 2.0, rel=1e-15)
    assert got[1] == pytest.approx(silu_l * -1.5, rel=1e-15)
    assert got[2] == pytest.approx(silu_l * 3.0, rel=1e-15)
    assert got[3] == 0.0
    assert got[4] == pytest.approx(-3.0 * scipy.special.expit(-3.0) * 2.0, rel=1e-15)
    s1 = scipy.special.expit(1.0)
    assert got[5] == pytest.approx(s1 * 7.0, rel=1e-15)  # up clamps to +L
    assert got[6] == pytest.approx(s1 * -7.0, rel=1e-15)  # up clamps to -L
    assert got[7] == 0.0
    assert silu_l == pytest.approx(6.9936226, abs=1e-7)


def test_swiglu_matches_scipy_expit():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(10000) * 6
    u = rng.standard_normal(10000) * 6
    ref = np.minimum(g, 7.0) * scipy.special.expit(np.minimum(g, 7.0)) * np.clip(u, -7, 7)
    assert np.allclose(moe.swiglu_clamp(g, u, 7.0), ref, rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------------------ combine

def test_combine_copy_identity_and_skip():
    rng = np.random.default_rng(6)
    e_out = rng.standard_normal((12, 10))
    # top_k=1, weight 1 -> rows copied through the permutation
    perm = rng.permutation(12).reshape(12, 1)
    out = moe.combine(e_out, perm, np.ones((12, 1)))
    assert np.array_equal(out, e_out[perm[:, 0]])
    # identity token_to_perm over [rows, top_k] = slot-major combine
    rows, top_k = 4, 3
    w = rng.random((rows, top_k))
    ident = np.arange(rows * top_k).reshape(rows, top_k)
    got = moe.combine(e_out, ident, w)
    for r in range(rows):
        ref = sum(w[r, j] * e_out[r * top_k + j] for j in range(top_k))
        assert np.allclose(got[r], ref, rtol=1e-15, atol=1e-15)
    # skipped slots (-1) add nothing; shared output is added
    ttp = ident.copy()
    ttp[1, 2] = -1
    shared = rng.standard_normal((rows, 10))
    got = moe.combine(e_out, ttp, w, shared)
    ref1 = w[1, 0] * e_out[3] + w[1, 1] * e_out[4] + shared[1]
    assert np.allclose(got[1], ref1, rtol=1e-15, atol=1e-15)
    # identical rows with equal weights: row * sum(w)
    same = np.tile(e_out[:1], (12, 1))
    got = moe.combine(same, ident, np.full((rows, top_k), 0.25))
    assert np.allclose(got, np.tile(e_out[:1] * 0.75, (rows, 1)), rtol=1e-15)


# ------------------------------------------------------------------------------ layer

def _brute_layer(ids, wts, x_bits, gate_up, down, s2gu, s2dn, mi, limit, bf16w):
    """Per token, per slot: the expert's FFN straight from the definition, no sorting."""
    def rnd(v):
        return float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16)) if bf16w else v

    xt = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    rows, top_k = ids.shape
    hidden = xt.shape[1]
    out = np.zeros((rows, hidden))
    for r in range(rows):
        for j in range(top_k):
            e = int(ids[r, j])
            if not (0 <= e < len(gate_up)) or gate_up[e] is None:
                continue
            pgu, sgu = gate_up[e]
            h = []
            for nn in range(2 * mi):
                acc = sum(Fraction(float(xt[r, kk])) *
                          _exact_weight(pgu, sgu, s2gu[e], nn, kk, bf16w) for kk in range(hidden))
                h.append(rnd(float(acc)))
            act = []
            for i in range(mi):
                g = min(h[i], limit)
                u = min(max(h[mi + i], -limit), limit)
                act.append(rnd(g / (1.0 + math.exp(-g)) * u))
            pdn, sdn = down[e]
            for hh in range(hidden):
                acc = sum(Fraction(act[i]) * _exact_weight(pdn, sdn, s2dn[e], hh, i, bf16w)
                          for i in range(mi))
                out[r, hh] += float(wts[r, j]) * rnd(float(acc))
    return out


@pytest.mark.parametrize("workers", [1, 3])
@pytest.mark.parametrize("mode", ["exact", "bf16w"])
def test_layer_brute_force(mode, workers):
    rng = np.random.default_rng(31)
    rows, top_k, num_experts, hidden, mi = 5, 2, 4, 32, 16
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    ids[3, 1] = -1  # one unfilled slot
    wts = rng.random((rows, top_k)).astype(np.float32)
    x_bits = wl.bf16_normal(rng, (rows, hidden))
    gate_up, down = [], []
    for e in range(num_experts):
        if e == 2:  # a remote expert: null in both tables
            gate_up.append(None)
            down.append(None)
            continue
        gate_up.append(wl.random_nvfp4(rng, 2 * mi, hidden))
        down.append(wl.random_nvfp4(rng, hidden, mi))
    s2gu = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    s2dn = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    x = codecs.bf16_bits_to_f64(x_bits)
    got, _ = moe.moe_layer(x, ids, wts, gate_up, down, s2gu, s2dn, mi, 7.0, mode,
                           workers=workers)
    ref = _brute_layer(ids, wts, x_bits, gate_up, down, s2gu, s2dn, mi, 7.0, mode == "bf16w")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_layer_ep_halves_sum_to_full():
    # Running with complementary halves of the table null sums to the full-table output
    # (the per-GPU partial sums of an expert-parallel split, before an all-reduce).
    rng = np.random.default_rng(41)
    rows, top_k, num_experts, hidden, mi = 12, 3, 6, 32, 16
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    wts = rng.random((rows, top_k)).astype(np.float32)
    x = codecs.bf16_bits_to_f64(wl.bf16_normal(rng, (rows, hidden)))
    gu = [wl.random_nvfp4(rng, 2 * mi, hidden) for _ in range(num_experts)]
    dn = [wl.random_nvfp4(rng, hidden, mi) for _ in range(num_experts)]
    s2 = np.ones(num_experts, np.float32)
    full, _ = moe.moe_layer(x, ids, wts, gu, dn, s2, s2, mi, 7.0, "exact")
    half = num_experts // 2
    lo_gu = [w if e < half else None for e, w in enumerate(gu)]
    lo_dn = [w if e < half else None for e, w in enumerate(dn)]
    hi_gu = [w if e >= half else None for e, w in enumerate(gu)]
    hi_dn = [w if e >= half else None for e, w in enumerate(dn)]
    a, _ = moe.moe_layer(x, ids, wts, lo_gu, lo_dn, s2, s2, mi, 7.0, "exact")
    b, _ = moe.moe_layer(x, ids, wts, hi_gu, hi_dn, s2, s2, mi, 7.0, "exact")
    assert np.allclose(a + b, full, rtol=1e-13, atol=1e-12)


def test_pages_error_table_is_self_consistent():
    # The only reproducible fact in the pages' microtest table: all four rows share one
    # reference infinity norm (max_abs / ratio ~ 442), so 0.998566 is half a BF16 ulp
    # of the outputs in [256, 512) and 2.0 is one ulp.
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pages_error_table.json")) as f:
        t = json.load(f)
    norms = [r["max_abs"] / r["max_abs_over_ref_inf"] for r in t["rows"]]
    assert max(norms) / min(norms) < 1.001
    assert 256 <= norms[0] < 512


# ------------------------------------------------------------------------------- router

def test_router_no_bias_is_argsort_of_logits_and_softmax_of_selected():
    rng = np.random.default_rng(21)
    lg = rng.standard_normal((40, 33)).astype(np.float32)
    ids, wts = moe.router_topk(lg, 6)
    want_ids = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :6]
    assert np.array_equal(ids, want_ids)
    sel = np.take_along_axis(lg.astype(np.float64), want_ids, axis=1)
    assert np.allclose(wts, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)


def test_router_brute_force_small():
    # every subset of size k of 6 experts: the selection maximises the summed key, and
    # among equal sums takes the lexicographically smallest id set (ties to lower ids)
    import itertools
    rng = np.random.default_rng(22)
    for trial in range(30):
        lg = rng.integers(-3, 4, size=(1, 6)).astype(np.float32)  # many equal keys
        k = int(rng.integers(1, 6))
        ids, wts = moe.router_topk(lg, k)
        best = None
        for sub in itertools.combinations(range(6), k):
            # rank by the sorted key vector, then by ids: what "k largest, ties to lower id" means
            kv = sorted((-float(lg[0, e]), e) for e in sub)
            if best is None or kv < best[0]:
                best = (kv, sub)
        assert list(ids[0]) == [e for _, e in best[0]], (lg, k)
        z = [math.exp(float(lg[0, e])) for e in ids[0]]
        assert np.allclose(wts[0], [v / sum(z) for v in z], rtol=1e-14)


def test_router_equal_logits_ties_and_weights():
    ids, wts = moe.router_topk(np.zeros((2, 8), np.float32), 3, routed_scale=2.5)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(wts, 2.5 / 3, rtol=1e-15)


def test_router_bias_changes_selection_not_weights():
    lg = np.array([[0.0, 0.0, 5.0, 1.0]], np.float32)
    bias = np.array([10.0, 0.0, 0.0, 0.0])
    ids, wts = moe.router_topk(lg, 1, bias=bias)
    assert ids.tolist() == [[0]] and wts[0, 0] == 1.0  # renormalised over one expert
    ids, wts = moe.router_topk(lg, 2, bias=bias, renormalize=False)
    p = scipy.special.softmax(lg[0].astype(np.float64))
    assert ids.tolist() == [[0, 2]]
    assert np.allclose(wts[0], [p[0], p[2]], rtol=1e-14)  # scores, not scores + bias


def test_router_no_renormalize_is_softmax_over_all_experts():
    rng = np.random.default_rng(23)
    lg = rng.standard_normal((5, 12)).astype(np.float32)
    ids, wts = moe.router_topk(lg, 4, renormalize=False, routed_scale=1.5)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(wts, 1.5 * np.take_along_axis(p, ids.astype(np.int64), axis=1), rtol=1e-14)


def test_router_top_k_beyond_experts_pads():
    ids, wts = moe.router_topk(np.array([[1.0, 3.0]], np.float32), 4)
    assert ids.tolist() == [[1, 0, -1, -1]] and wts[0, 2:].tolist() == [0.0, 0.0]
    assert math.isclose(wts[0, :2].sum(), 1.0, rel_tol=1e-15)


@pytest.mark.parametrize("name", ["single_gemm", "layer_e64", "long_prefill"])
def test_router_matches_workload_routing_recipe(name):
    # the workloads' FP32 routing recipe (top-k of logits, softmax over the selected ones)
    # is an independent implementation of the no-bias, renormalised case
    w = wl.WORKLOADS[name]
    ids, wts = moe.router_topk(wl.router_logits(w), w.top_k)
    want_ids, want_w = wl.routing(w)
    assert np.array_equal(ids, want_ids)
    assert np.allclose(wts, want_w, rtol=2e-6, atol=0)
