"""Pins for the oracle's number codecs against library routines and the format specs."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _spec():
    with open(os.path.join(GOLDEN, "ocp_formats.json")) as f:
        return json.load(f)


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_e4m3fn_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert _same(codecs.e4m3fn_decode(codes), ref)


def test_generic_decoder_matches_torch_e5m2_on_every_code():
    # The same decoder, with E5M2's parameters and IEEE specials, against torch: this
    # checks the generic exponent/mantissa/subnormal logic that E2M1 also goes through.
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float32).numpy()
    got = codecs.minifloat_decode(codes, exp_bits=5, man_bits=2, bias=15, nan_rule="ieee")
    assert _same(got, ref)


def test_e2m1_matches_ocp_table():
    spec = _spec()
    pos = np.array(spec["e2m1_positive_values_by_code"])
    got = codecs.e2m1_decode(np.arange(16))
    assert _same(got[:8], pos)
    assert _same(got[8:], -pos)  # bit 3 is the sign; nibble 8 is -0.0
    assert np.signbit(got[8])


def test_e4m3fn_spec_examples():
    for code, val in _spec()["e4m3fn_examples"].items():
        got = codecs.e4m3fn_decode(int(code, 16))
        want = np.nan if val == "nan" else float(val)
        assert _same(got, want), (code, got, want)


def _f32_edge_values():
    rng = np.random.default_rng(7)
    r = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    big = (rng.standard_normal(2000) * 1e30).astype(np.float32)
    tiny = (rng.standard_normal(2000) * 1e-39).astype(np.float32)  # FP32 subnormals
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    u = rng.integers(0, 2**31, size=4000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.3895314e38, 3.4028235e38,
                        -3.4028235e38, 1.0, -1.0, 1.00390625, 1.01171875], dtype=np.float32)
    return np.concatenate([r, big, tiny, ties, special])


def test_bf16_rne_matches_torch():
    x = _f32_edge_values()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_bits_from_f32(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(codecs.bf16_bits_to_f64(got[nan])))


def test_bf16_bits_to_f64_roundtrip_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(codecs.bf16_bits_to_f64(bits), ref)


def test_round_bf16_on_f32_values_matches_torch():
    x = _f32_edge_values()
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert _same(codecs.round_bf16(x.astype(np.float64)), ref)


def _bf16_nearest_exact(v: float) -> float:
    """Brute force: nearest BF16 to a finite float64 by exact rationals, ties to even."""
    if v == 0.0:
        return v
    f = Fraction(v)
    lo_bits = codecs.bf16_bits_from_f32(np.float32(v)).astype(np.int64)
    cands = []
    for b in range(int(lo_bits) - 2, int(lo_bits) + 3):
        if 0 <= (b & 0x7FFF) < 0x7F80:
            cands.append(b & 0xFFFF)
    best = None
    for b in cands:
        val = float(codecs.bf16_bits_to_f64(np.uint16(b)))
        d = abs(Fraction(val) - f)
        key = (d, b & 1)  # ties: even mantissa bit wins
        if best is None or key < best[0]:
            best = (key, val)
    return best[1]


def test_round_bf16_f64_brute_force():
    rng = np.random.default_rng(11)
    vals = rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))
    # values exactly halfway between two BF16 numbers, and a hair either side
    base = codecs.bf16_bits_to_f64(rng.integers(0x3000, 0x5000, 500).astype(np.uint16))
    half_ulp = np.ldexp(1.0, np.frexp(base)[1] - 9)
    vals = np.concatenate([vals, base + half_ulp, base + half_ulp * (1 + 2**-40),
                           base + half_ulp * (1 - 2**-40)])
    got = codecs.round_bf16(vals)
    for v, g in zip(vals, got):
        assert g == _bf16_nearest_exact(float(v)), v


@pytest.mark.parametrize("v,expect", [(3.3962e38, np.inf), (-3.3962e38, -np.inf),
                                      (3.3961e38, 3.3895313892515355e38)])
def test_round_bf16_overflow(v, expect):
    assert codecs.round_bf16(np.array([v]))[0] == expect
