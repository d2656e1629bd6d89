"""The gate_up grouped GEMM with the SwiGLU clamp fused into its epilogue.

The fused call must give the same bits as the two calls it replaces (grouped GEMM into a
[rows, 2 mi] buffer, then swiglu_clamp on its halves), for every shape the two calls
accept: mi not a multiple of the block's 64 gate columns, experts with more rows than
one pass, null entries (their rows are left alone), out-of-range gather indices, and
zero, subnormal, negative and NaN scale codes (every code goes through the same per-block
decode table). Its agreement with the oracle is checked at layer level
(tests/test_gpu_layer.py runs the layer fused and unfused); the table itself is checked
against the oracle on all 256 scale codes in tests/test_gpu_gemm.py.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import bf16_bits_host, bf16_dev, dev, upload_table

pytestmark = pytest.mark.gpu

POISON = -1  # 0xFFFF: a BF16 NaN


def _problem(seed, mi, k, counts, null, special):
    rng = np.random.default_rng(seed)
    e_n = len(counts)
    experts = []
    for e in range(e_n):
        if e in null:
            experts.append(None)
            continue
        packed, scales = wl.random_nvfp4(rng, 2 * mi, k)
        if special:  # zero, subnormal, max, negative and NaN scale codes
            flat = scales.reshape(-1)
            idx = rng.choice(flat.size, size=min(64, flat.size), replace=False)
            flat[idx] = rng.choice(np.array([0x00, 0x01, 0x07, 0x7E, 0x7F, 0x80, 0xB8], np.uint8),
                                   size=idx.size)
        experts.append((packed, scales))
    s2 = rng.uniform(0.5, 2.0, e_n).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t = max(int(offsets[-1]), 1) + 3
    x_bits = wl.bf16_normal(rng, (t, k))
    gather = rng.integers(0, t, max(int(offsets[-1]), 1)).astype(np.int32)
    if offsets[-1] > 2:
        gather[1] = t + 5  # out of range: reads a row of zeros
        gather[2] = -4
    return experts, s2, offsets, x_bits, gather


def _run_both(hip, experts, s2, offsets, x_bits, gather, mi, k, limit):
    rows = int(offsets[-1])
    table = upload_table(hip, experts, s2, 2 * mi, k)
    x = bf16_dev(x_bits)
    off = dev(offsets)
    g = dev(gather)
    # unfused: GEMM into [rows, 2 mi], then swiglu_clamp on its halves
    c = torch.empty((rows, 2 * mi), dtype=torch.bfloat16, device="cuda")
    c.view(torch.int16).fill_(POISON)
    hip.moe_w4a16_grouped_gemm(x, table, off, c, g, max_rows=rows)
    ref = torch.empty((rows, mi), dtype=torch.bfloat16, device="cuda")
    hip.swiglu_clamp(c[:, :mi], c[:, mi:], ref, limit)
    # fused, into a wider buffer (ld_act > mi) filled with NaN
    act_full = torch.empty((rows, mi + 24), dtype=torch.bfloat16, device="cuda")
    act_full.view(torch.int16).fill_(POISON)
    act = act_full[:, :mi]
    hip.moe_w4a16_grouped_gemm_swiglu(x, table, off, act, limit, g, max_rows=rows)
    torch.cuda.synchronize()
    return bf16_bits_host(ref), bf16_bits_host(act_full)


@pytest.mark.parametrize("mi,k,counts,null,special,seed", [
    (64, 256, [5, 0, 16, 3], (), False, 1),
    (80, 512, [17, 4, 0, 9], (1,), True, 2),           # mi % 64 = 16; a two-pass expert
    (16, 768, [1, 33, 2], (), True, 3),                # one gate tile; three passes
    (192, 1024, [8, 8, 8, 8, 8, 8], (0, 5), False, 4),
    (48, 256, [40], (), True, 5),
    (32, 512, [65, 0, 200, 64, 3], (3,), False, 6),  # experts past 64 rows: overflow blocks
])
def test_fused_matches_two_calls_bitwise(hip, mi, k, counts, null, special, seed):
    experts, s2, offsets, x_bits, gather = _problem(seed, mi, k, counts, null, special)
    ref, got_full = _run_both(hip, experts, s2, offsets, x_bits, gather, mi, k, 7.0)
    got = got_full[:, :mi]
    for e in range(len(counts)):
        lo, hi = offsets[e], offsets[e + 1]
        if experts[e] is None:  # null entry: rows not written
            assert np.all(got[lo:hi] == 0xFFFF)
            continue
        assert np.array_equal(got[lo:hi], ref[lo:hi]), (e, np.argwhere(got[lo:hi] != ref[lo:hi])[:3])
    assert np.all(got_full[:, mi:] == 0xFFFF)  # nothing written past mi


def test_fused_small_limit_clamps(hip):
    # a small limit makes the clamps bind on most elements
    experts, s2, offsets, x_bits, gather = _problem(9, 64, 512, [12, 7], (), False)
    ref, got_full = _run_both(hip, experts, s2, offsets, x_bits, gather, 64, 512, 0.25)
    assert np.array_equal(got_full[:, :64], ref)


def test_fused_prefill_subchunk_sampled_experts(hip):
    """Full gate_up shape (mi 2048, K 6144) for a few routed experts."""
    w = wl.WORKLOADS["prefill_subchunk"]
    rng = np.random.default_rng(11)
    mi, k = w.moe_intermediate, w.hidden
    counts = [9, 0, 21, 1]
    experts = [wl.random_nvfp4(rng, 2 * mi, k) if c else None for c in counts]
    s2 = rng.uniform(0.5, 2.0, len(counts)).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x_bits = wl.bf16_normal(rng, (int(offsets[-1]), k))
    gather = rng.permutation(int(offsets[-1])).astype(np.int32)
    ref, got_full = _run_both(hip, experts, s2, offsets, x_bits, gather, mi, k, w.limit)
    assert np.array_equal(got_full[:, :mi], ref)


def test_fused_rejects_bad_arguments(hip):
    rng = np.random.default_rng(1)
    packed, scales = wl.random_nvfp4(rng, 2 * 24, 256)  # mi = 24: not a multiple of 16
    table = upload_table(hip, [(packed, scales)], np.ones(1, np.float32), 48, 256)
    x = bf16_dev(wl.bf16_normal(rng, (4, 256)))
    off = dev(np.array([0, 4], np.int32))
    act = torch.empty((4, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hip.MoeError):
        hip.moe_w4a16_grouped_gemm_swiglu(x, table, off, act, 7.0, max_rows=4)
    packed, scales = wl.random_nvfp4(rng, 32, 256)
    table = upload_table(hip, [(packed, scales)], np.ones(1, np.float32), 32, 256)
    act = torch.empty((4, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hip.MoeError):
        hip.moe_w4a16_grouped_gemm_swiglu(x, table, off, act, 0.0, max_rows=4)  # limit <= 0
    # the binding refuses an act narrower than mi before calling the library
    with pytest.raises(ValueError):
        hip.moe_w4a16_grouped_gemm_swiglu(x, table, off, act[:, :8], 7.0, max_rows=4)
