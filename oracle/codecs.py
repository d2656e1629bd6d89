"""Number-format codecs for the oracle (test infrastructure only).

The pages name the formats but print neither codebook: the packed weight element is
"E2M1" decoded through a 16-value codebook, the block scale is "E4M3", and the
grouped GEMM stages each dequantised weight as a BF16 obtained by
``__float2bfloat16`` (forward_prefill_gemm module docs, "Layout compatibility" table,
rows "codebook" and "block scale"; section "What is NOT bit-identical", item 2).

Readings taken (each pinned in tests/test_oracle_codecs.py):
- E2M1 is the OCP Microscaling FP4 element: 1 sign, 2 exponent, 1 mantissa bit,
  bias 1, no infinities or NaNs.
- E4M3 is OCP FP8 E4M3FN: bias 7, no infinities, NaN only at S.1111.111.
- FP32 -> BF16 is round-to-nearest-even on the FP32 bit pattern, NaN -> quiet NaN.

Both minifloats go through one generic decoder written from the IEEE-style
definition (sign, biased exponent, implicit leading one, subnormals at exponent
field 0), so that the decoder that is checked against ``torch.float8_e4m3fn`` and
``torch.float8_e5m2`` on every code is the same one that decodes E2M1.
"""

from __future__ import annotations

import numpy as np


def minifloat_decode(codes, exp_bits: int, man_bits: int, bias: int, nan_rule: str):
    """Decode unsigned integer ``codes`` of a (1, exp_bits, man_bits) minifloat to float64.

    ``nan_rule``:
    - ``"none"``: every code is finite (OCP E2M1).
    - ``"fn"``: only the all-ones exponent *and* all-ones mantissa is NaN; the rest of
      the top binade is finite (OCP E4M3FN).
    - ``"ieee"``: all-ones exponent is Inf (mantissa 0) or NaN (OCP E5M2).
    """
    codes = np.asarray(codes, dtype=np.int64)
    sign = (codes >> (exp_bits + man_bits)) & 1
    e = (codes >> man_bits) & ((1 << exp_bits) - 1)
    m = codes & ((1 << man_bits) - 1)
    frac = m.astype(np.float64) / float(1 << man_bits)
    normal = (1.0 + frac) * np.power(2.0, (e - bias).astype(np.float64))
    subnormal = frac * 2.0 ** (1 - bias)
    mag = np.where(e == 0, subnormal, normal)
    e_max = (1 << exp_bits) - 1
    m_max = (1 << man_bits) - 1
    if nan_rule == "fn":
        mag = np.where((e == e_max) & (m == m_max), np.nan, mag)
    elif nan_rule == "ieee":
        mag = np.where(e == e_max, np.where(m == 0, np.inf, np.nan), mag)
    elif nan_rule != "none":
        raise ValueError(nan_rule)
    return np.where(sign == 1, -mag, mag)


def e2m1_decode(nibbles):
    """Value of an E2M1 nibble (0..15) as float64: bit 3 sign, bits 2..1 exponent, bit 0
    mantissa. Nibble 8 decodes to -0.0."""
    return minifloat_decode(nibbles, exp_bits=2, man_bits=1, bias=1, nan_rule="none")


def e4m3fn_decode(codes):
    """Value of an E4M3FN byte (0..255) as float64; 0x7F and 0xFF are NaN."""
    return minifloat_decode(codes, exp_bits=4, man_bits=3, bias=7, nan_rule="fn")


def bf16_bits_from_f32(x):
    """Round float32 values to BF16 with round-to-nearest-even; returns uint16 bit patterns.

    Works on the FP32 bit pattern: add 0x7FFF plus the lowest kept bit, keep the top 16
    bits. NaN maps to the quiet NaN 0x7FC0 with the input's sign dropped.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    out = np.where(np.isnan(f), 0x7FC0, rounded)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact float64 value of BF16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_bf16(x):
    """Round float64 values straight to the BF16 grid (round-to-nearest-even), as float64.

    Used for the BF16 buffers between the layer's steps, where the oracle's FP64 value
    stands in for the kernels' FP32 accumulator. BF16 keeps 8 significant bits; below
    2**-126 the grid spacing stays 2**-133 (subnormals); beyond the largest finite BF16
    (0x7F7F) the result is +-inf. NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, exp = np.frexp(x)  # x = mant * 2**exp, 0.5 <= |mant| < 1
    exp = np.maximum(exp, -125)  # fixed quantum 2**-133 in the subnormal range
    quantum_exp = exp - 8
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -quantum_exp)), quantum_exp)
        max_bf16 = float(np.ldexp(np.float64(0xFF), 127 - 7))  # 0x7F7F
        r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)
