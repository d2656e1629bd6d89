"""The grouped W4A16 GEMM and its weight decode on the GPU against the oracle.

- Decode: bit-exact against the oracle's BF16-weight dequant, special scales included.
- Layout pins: one-hot weights and power-of-two scale patterns give exact answers.
- Numerics: against the BF16-weight oracle within the gate (max_abs / ||ref||_inf <= 5e-3)
  and a per-element FP32 accumulation bound; against the exact oracle, reported.
- Edge cases: null experts untouched, empty experts, ragged N (partial tiles), experts
  with more rows than one pass, out-of-range gather indices, max_rows cut-off.
- Full size: the 256-expert prefill sub-chunk shapes, every expert and row.
- Every E4M3 scale code through the GEMM's own decode table, bit-exact (identity rows).
"""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import codecs, moe
from gpu_util import (GATE, ORACLE_WORKERS, LazyExperts, bf16_bits_host, bf16_dev, dev, f64,
                      oracle_threads, rel_err, rel_err_rows, upload_table, workload_tables)

pytestmark = pytest.mark.gpu


def _pack(nib):
    """[N, K] nibbles -> [N, K/2] bytes, even k in the low nibble."""
    return (nib[:, 0::2] & 0xF) | ((nib[:, 1::2] & 0xF) << 4)


# ----------------------------------------------------------------------------- decode

def _dequant_gpu(hip, packed, scales, s2):
    n, half = packed.shape
    out = torch.empty((n, 2 * half), dtype=torch.bfloat16, device="cuda")
    hip.moe_w4a16_dequant_bf16(dev(packed), dev(scales), float(s2), out)
    torch.cuda.synchronize()
    return bf16_bits_host(out)


def _same_bits(got, ref):
    gn = np.isnan(codecs.bf16_bits_to_f64(got))
    rn = np.isnan(codecs.bf16_bits_to_f64(ref))
    assert np.array_equal(gn, rn)
    bad = (got != ref) & ~gn
    assert not bad.any(), f"{bad.sum()} mismatches, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("s2", [1.0, 0.7310585, 1.9999999, 0.5, 3.3e-36, 2.5e36, -1.25, 1e-40])
def test_dequant_bit_exact_random(hip, s2):
    rng = np.random.default_rng(17)
    packed, scales = wl.random_nvfp4(rng, 96, 512)
    # every E4M3 code somewhere: zero, subnormals, max, NaN, negative scales
    scales.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)
    ref = moe.dequant_bf16_bits(packed, scales, s2)
    _same_bits(_dequant_gpu(hip, packed, scales, s2), ref)


def test_dequant_bit_exact_all_nibbles_all_scales(hip):
    # every (nibble, scale code) pair with a non-power-of-two scale2
    codes = np.arange(256, dtype=np.uint8)
    nib = np.tile(np.arange(16, dtype=np.uint8), (256, 2))  # [256, 32]
    packed = _pack(nib)
    scales = np.stack([codes, codes], axis=1)  # one code per row
    for s2 in (1.3719, 0.51, 1.0 + 2 ** -23):
        _same_bits(_dequant_gpu(hip, packed, scales, s2), moe.dequant_bf16_bits(packed, scales, s2))


# ----------------------------------------------- every scale code through the GEMM

def code_per_row_expert(k: int):
    """An NVFP4 projection of 256 rows: row n uses E4M3 code n for every 16-k block, and
    its nibbles run (k + n) % 16, so every block holds all 16 nibbles."""
    n_idx = np.arange(256)[:, None]
    nib = ((np.arange(k)[None, :] + n_idx) % 16).astype(np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k // 16, axis=1)
    return _pack(nib), np.ascontiguousarray(scales)


def _same_values(got, ref):
    """Equal values (+0 == -0) and NaN at the same places."""
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn), f"NaN at {np.argwhere(gn != rn)[:4].tolist()}"
    bad = (got != ref) & ~gn
    assert not bad.any(), f"{bad.sum()} mismatches, first at {np.argwhere(bad)[0].tolist()}"


@pytest.mark.parametrize("null_pad", [0, 60])  # 2 experts: 32-row passes; 62: 16-row passes
@pytest.mark.parametrize("s2", [(1.3719, 0.51), (1.0, 1.0 + 2 ** -23)])
def test_every_scale_code_through_the_gemm_bit_exact(hip, null_pad, s2):
    """All 256 E4M3 codes (zero, subnormal, negative, the largest, NaN) times all 16 nibbles
    through the GEMM's own per-block decode table: identity activation rows (row t is one
    at k = t) make output [s, n] the decoded weight w[n, t], which BF16 holds exactly, so
    the GEMM output must equal the oracle's BF16-weight dequant value for value."""
    k = 256
    ex = code_per_row_expert(k)
    experts = [ex, ex] + [None] * null_pad
    s2v = np.array(list(s2) + [1.0] * null_pad, np.float32)
    x_bits = np.where(np.eye(k, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    offsets = np.array([0, 256, 512] + [512] * null_pad, np.int32)
    gather = np.concatenate([np.arange(256), np.arange(256)]).astype(np.int32)
    got = _gemm(hip, x_bits, experts, s2v, offsets, 256, k, gather)
    ref = _oracle(x_bits, experts, s2v, offsets, 256, gather, "bf16w")
    # the definition: row s of expert e is column gather[s] of its BF16-weight dequant
    for e in range(2):
        w = moe.dequant(ex[0], ex[1], float(s2v[e]), "bf16w")
        assert np.array_equal(np.isnan(ref[256 * e:256 * (e + 1)]), np.isnan(w.T))
    _same_values(got, ref)


@pytest.mark.parametrize("null_pad", [0, 60])
def test_every_scale_code_through_the_fused_gemm(hip, null_pad):
    """The SwiGLU-fused kernel's decode table on all 256 codes: gate row j has code j,
    up rows are all 1.0 (code 0x38, nibble 2); identity activations make the gate value
    the decoded weight itself. The result equals the oracle's SwiGLU of those values to
    half a BF16 ulp (NaN where the gate weight is NaN)."""
    k, mi, limit = 256, 256, 7.0
    gate_p, gate_s = code_per_row_expert(k)
    up_p = np.full((mi, k // 2), 0x22, np.uint8)
    up_s = np.full((mi, k // 16), 0x38, np.uint8)
    ex = (np.concatenate([gate_p, up_p]), np.concatenate([gate_s, up_s]))
    experts = [ex, ex] + [None] * null_pad
    s2v = np.array([1.3719, 0.51] + [1.0] * null_pad, np.float32)
    table = upload_table(hip, experts, s2v, 2 * mi, k)
    x_bits = np.where(np.eye(k, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    offsets = np.array([0, 256, 512] + [512] * null_pad, np.int32)
    gather = np.concatenate([np.arange(256), np.arange(256)]).astype(np.int32)
    act = torch.full((512, mi), -3.0, dtype=torch.bfloat16, device="cuda")
    hip.moe_w4a16_grouped_gemm_swiglu(bf16_dev(x_bits), table, dev(offsets), act, limit,
                                      dev(gather), max_rows=512)
    torch.cuda.synchronize()
    got = f64(act)
    c = _oracle(x_bits, experts, s2v, offsets, 2 * mi, gather, "bf16w")
    c = codecs.round_bf16(c)
    ref = moe.swiglu_clamp(c[:, :mi], c[:, mi:], limit)
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn)
    ok = ~rn
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref[ok]), 2.0 ** -126))[1] - 8)
    assert np.all(np.abs(got[ok] - ref[ok]) <= ulp * 0.5 * (1 + 2 ** -4) + 1e-38)


def test_every_scale_code_through_the_union_gemv(hip):
    """The union GEMV's decode table on all 256 codes: 16 rows routed to one expert, row r
    one-hot at k = 16 i + r in call i, so 16 calls read every decoded weight back exactly."""
    k = 256
    ex = code_per_row_expert(k)
    experts, s2v = [ex], np.array([1.3719], np.float32)
    table = upload_table(hip, experts, s2v, 256, k)
    rows = 16
    ids = np.zeros((rows, 1), np.int32)
    i32 = dict(dtype=torch.int32, device="cuda")
    u_eid, u_slot = torch.empty(rows, **i32), torch.empty(rows * rows, **i32)
    hip.moe_row_union(dev(ids), 1, u_eid, u_slot)
    w = moe.dequant(ex[0], ex[1], float(s2v[0]), "bf16w")
    for i in range(k // rows):
        x_bits = np.zeros((rows, k), np.uint16)
        x_bits[np.arange(rows), 16 * i + np.arange(rows)] = 0x3F80
        c = torch.full((rows, 256), -3.0, dtype=torch.bfloat16, device="cuda")
        hip.moe_w4a16_gemv_union(bf16_dev(x_bits), table, u_eid, u_slot, c, rows, 1)
        torch.cuda.synchronize()
        ref = np.full((rows, 256), np.nan)
        un = moe.row_union(ids, 1)
        moe.union_gemv(codecs.bf16_bits_to_f64(x_bits), False, experts, s2v, un["u_eid"],
                       un["u_slot"], 1, ref, "bf16w")
        assert np.array_equal(np.isnan(ref), np.isnan(w[:, 16 * i:16 * i + rows].T))
        _same_values(f64(c), ref)


# ------------------------------------------------------------------------ GEMM runner

def _gemm(hip, x_bits, experts, s2, offsets, n, k, gather=None, rows=None, fill=-3.0,
          c_rows=None, table=None):
    """Run the GPU GEMM; returns the output as float64 (rows not written keep ``fill``)."""
    if table is None:
        table = upload_table(hip, experts, s2, n, k)
    rows = int(offsets[-1]) if rows is None else rows
    c_rows = rows if c_rows is None else c_rows
    c = torch.full((max(c_rows, 1), n), fill, dtype=torch.bfloat16, device="cuda")
    g = None if gather is None else dev(np.asarray(gather, np.int32))
    hip.moe_w4a16_grouped_gemm(bf16_dev(x_bits), table, dev(np.asarray(offsets, np.int32)), c,
                               g, max_rows=rows)
    torch.cuda.synchronize()
    return f64(c)


def _oracle(x_bits, experts, s2, offsets, n, gather, mode, rows=None):
    rows = int(offsets[-1]) if rows is None else rows
    out = np.full((rows, n), np.nan)
    moe.grouped_gemm(codecs.bf16_bits_to_f64(x_bits), gather, experts, s2, offsets, out, mode)
    return out


def _acc_bound(x_bits, experts, s2, offsets, gather, k):
    """Per-element bound on FP32 accumulation plus BF16 output rounding."""
    ax = np.abs(codecs.bf16_bits_to_f64(x_bits))
    rows = int(offsets[-1])
    s = None
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        if hi <= lo or experts[e] is None:
            continue
        ex = experts[e]
        if s is None:
            s = np.zeros((rows, ex[0].shape[0]))
        w = np.abs(moe.dequant(ex[0], ex[1], float(s2[e]), "bf16w"))
        src = np.arange(lo, hi) if gather is None else np.asarray(gather)[lo:hi]
        s[lo:hi] = ax[src] @ w.T
    gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    return gamma * s


def _check_gemm(got, ref, bound, exact=None):
    mask = ~np.isnan(ref)
    err = np.abs(got - ref)
    # half a BF16 ulp of the FP32 result (whose magnitude is at most |ref| + bound) plus
    # the accumulation bound
    lim = np.ldexp(1.0, np.frexp(np.abs(ref) + bound)[1] - 8) * 0.5 + bound * 1.001 + 1e-30
    assert np.all(err[mask] <= lim[mask]), float(np.max((err - lim)[mask]))
    r = rel_err(got[mask], ref[mask])
    assert r <= GATE, r
    return r


# ------------------------------------------------------------------------ layout pins

def test_one_hot_layout_is_exact(hip):
    # W_e[n, k] = 1 at k = pi_e(n): y[s, n] = a[g(s), pi_e(n)] exactly. Pins N-major order,
    # even-low nibble order, K/2 byte and K/16 scale indexing, the global-id table, the
    # gather and the output row.
    rng = np.random.default_rng(3)
    t, e_n, n, k = 40, 5, 48, 512
    x_bits = wl.bf16_normal(rng, (t, k))
    experts, pis = [], []
    for e in range(e_n):
        pi = rng.integers(0, k, n)
        nib = np.zeros((n, k), np.uint8)
        nib[np.arange(n), pi] = 2 if e % 2 == 0 else 10  # +1.0 / -1.0
        experts.append((_pack(nib), np.full((n, k // 16), 0x38, np.uint8)))
        pis.append(pi)
    counts = [7, 0, 19, 40, 5]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    gather = rng.integers(0, t, offsets[-1])
    got = _gemm(hip, x_bits, experts, np.ones(e_n, np.float32), offsets, n, k, gather)
    x = codecs.bf16_bits_to_f64(x_bits)
    for e in range(e_n):
        for s in range(offsets[e], offsets[e + 1]):
            sign = 1.0 if e % 2 == 0 else -1.0
            assert np.array_equal(got[s], sign * x[gather[s], pis[e]]), (e, s)


def test_power_of_two_scale_pattern_is_exact(hip):
    # One 1.0 per row at k = pi(n) with a distinct power-of-two block scale per (n, k/16)
    # and scale2 = 2**-3: y = a[g, pi(n)] * 2**(f(n, pi(n)/16) - 3) exactly.
    rng = np.random.default_rng(4)
    t, n, k = 16, 32, 768
    x_bits = wl.bf16_normal(rng, (t, k))
    pi = rng.integers(0, k, n)
    nib = np.zeros((n, k), np.uint8)
    nib[np.arange(n), pi] = 2
    exps = (np.arange(n)[:, None] * 5 + np.arange(k // 16)[None, :] * 3) % 13 - 6
    codes = ((exps + 7) << 3).astype(np.uint8)
    ex = [(_pack(nib), codes)]
    offsets = np.array([0, t])
    got = _gemm(hip, x_bits, ex, np.array([0.125], np.float32), offsets, n, k)
    x = codecs.bf16_bits_to_f64(x_bits)
    want = x[:, pi] * np.exp2(exps[np.arange(n), pi // 16] - 3)[None, :]
    assert np.array_equal(got, want)


def test_all_ones_gives_row_sums(hip):
    rng = np.random.default_rng(5)
    t, n, k = 20, 64, 1024
    x_bits = wl.bf16_normal(rng, (t, k))
    ex = [(np.full((n, k // 2), 0x22, np.uint8), np.full((n, k // 16), 0x38, np.uint8))]
    offsets = np.array([0, t])
    got = _gemm(hip, x_bits, ex, np.ones(1, np.float32), offsets, n, k)
    ref = _oracle(x_bits, ex, np.ones(1, np.float32), offsets, n, None, "bf16w")
    _check_gemm(got, ref, _acc_bound(x_bits, ex, np.ones(1), offsets, None, k))
    assert np.all(got == got[:, :1])  # every weight row is the same


# --------------------------------------------------------------------------- numerics

def _routed_problem(w: wl.Workload):
    ids, _ = wl.routing(w)
    al = moe.align(ids, w.num_experts)
    x_bits = wl.activations(w)
    return al, x_bits


def test_single_gemm_workload_vs_oracle(hip):
    w = wl.WORKLOADS["single_gemm"]
    al, x_bits = _routed_problem(w)
    n, k = wl.gate_up_shape(w)
    experts = LazyExperts(w, "gate_up")
    s2 = wl.scale2_gate_up(w)
    offsets, gather = al["expert_offsets"], al["sorted_token_ids"]
    got = _gemm(hip, x_bits, experts, s2, offsets, n, k, gather)
    ref = _oracle(x_bits, experts, s2, offsets, n, gather, "bf16w")
    r = _check_gemm(got, ref, _acc_bound(x_bits, experts, s2, offsets, gather, k))
    exact = _oracle(x_bits, experts, s2, offsets, n, gather, "exact")
    r_exact = rel_err(got, exact)
    print(f"single_gemm: vs bf16w {r:.6f}, vs exact {r_exact:.6f}")
    # the BF16 weight operand moves the result by about 2**-9 per weight, no more
    assert r_exact < 2 * GATE


@pytest.mark.parametrize("n,k,counts,null,seed", [
    (16, 256, [3, 0, 1, 33, 16], (), 0),            # one wave's rows, one pass and two
    (144, 768, [70, 1, 0, 15, 32, 9], (2,), 1),     # partial block of rows, long expert
    (400, 512, [5, 64, 0, 17], (0,), 2),            # ragged N tiles, exactly two passes
    (256, 2048, [129, 0, 2], (), 3),                # five passes
    # experts past 64 rows: one block per 64 of them (64 fits one; 65, 128, 193 overflow),
    # a null expert with overflow chunks keeps its rows
    (48, 256, [64, 65, 0, 128, 193, 1, 130], (3,), 4),
])
def test_ragged_shapes_and_nulls(hip, n, k, counts, null, seed):
    rng = np.random.default_rng(seed)
    t = 50
    x_bits = wl.bf16_normal(rng, (t, k))
    experts = [None if e in null else wl.random_nvfp4(rng, n, k) for e in range(len(counts))]
    s2 = rng.uniform(0.5, 2, len(counts)).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    gather = rng.integers(0, t, offsets[-1])
    got = _gemm(hip, x_bits, experts, s2, offsets, n, k, gather)
    ref = _oracle(x_bits, experts, s2, offsets, n, gather, "bf16w")
    for e in null:  # rows of null experts keep the caller's values
        assert np.all(got[offsets[e]:offsets[e + 1]] == -3.0)
    _check_gemm(got, ref, _acc_bound(x_bits, experts, s2, offsets, gather, k))


def test_no_gather_and_row_cut_off(hip):
    rng = np.random.default_rng(6)
    n, k = 64, 512
    counts = [10, 20, 30]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    x_bits = wl.bf16_normal(rng, (offsets[-1], k))
    experts = [wl.random_nvfp4(rng, n, k) for _ in counts]
    s2 = np.ones(3, np.float32)
    ref = _oracle(x_bits, experts, s2, offsets, n, None, "bf16w")
    got = _gemm(hip, x_bits, experts, s2, offsets, n, k)
    _check_gemm(got, ref, _acc_bound(x_bits, experts, s2, offsets, None, k))
    # max_rows = 35 < offsets[-1]: rows >= 35 are never written
    got = _gemm(hip, x_bits, experts, s2, offsets, n, k, rows=35, c_rows=60)
    assert np.all(got[35:] == -3.0)
    assert rel_err(got[:35], ref[:35]) <= GATE


@pytest.mark.parametrize("fused", [False, True])
def test_unused_experts_change_no_bits(hip, fused):
    """Experts of 40, 50 and 33 rows average over 24 rows: the GEMM passes over 32 rows
    at a time (two row tiles per decoded weight). Ten unused experts appended to the
    table lower the average, and the GEMM then passes over 16 rows. Each output element
    sums the same products in the same order either way: the bits must not change."""
    rng = np.random.default_rng(12)
    n, k = 96, 512
    counts = [40, 50, 33]
    x_bits = wl.bf16_normal(rng, (130, k))
    experts = [wl.random_nvfp4(rng, n, k) for _ in counts]
    s2 = rng.uniform(0.5, 2, 13).astype(np.float32)
    gather = rng.integers(0, 130, sum(counts)).astype(np.int32)
    outs = []
    for extra in (0, 10):
        offsets = np.concatenate([[0], np.cumsum(counts + [0] * extra)]).astype(np.int32)
        table = upload_table(hip, experts + [None] * extra, s2[:3 + extra], n, k)
        rows = int(offsets[-1])
        x, g, off = bf16_dev(x_bits), dev(gather), dev(offsets)
        if fused:
            c = torch.full((rows, n // 2), -3.0, dtype=torch.bfloat16, device="cuda")
            hip.moe_w4a16_grouped_gemm_swiglu(x, table, off, c, 7.0, g, max_rows=rows)
        else:
            c = torch.full((rows, n), -3.0, dtype=torch.bfloat16, device="cuda")
            hip.moe_w4a16_grouped_gemm(x, table, off, c, g, max_rows=rows)
        torch.cuda.synchronize()
        outs.append(bf16_bits_host(c).copy())
    assert np.array_equal(outs[0], outs[1])
    if not fused:
        offsets = np.concatenate([[0], np.cumsum(counts)])
        ref = _oracle(x_bits, experts, s2, offsets, n, gather, "bf16w")
        _check_gemm(codecs.bf16_bits_to_f64(outs[0]), ref,
                    _acc_bound(x_bits, experts, s2, offsets, gather, k))


def test_many_experts_without_room_for_overflow_rows(hip):
    """65500 experts: the grid rows for overflow chunks would pass the 65535 limit, so the
    launch falls back to one block row per expert taking all of its rows (here 150 rows,
    three passes past 64). Three live experts at the ends and the middle of the table."""
    rng = np.random.default_rng(9)
    n, k, e_n = 32, 256, 65500
    counts = np.zeros(e_n, np.int64)
    live = {0: 150, 30000: 5, e_n - 1: 70}
    for e, c in live.items():
        counts[e] = c
    offsets = np.concatenate([[0], np.cumsum(counts)])
    experts = [None] * e_n
    for e in live:
        experts[e] = wl.random_nvfp4(rng, n, k)
    s2 = rng.uniform(0.5, 2, e_n).astype(np.float32)
    x_bits = wl.bf16_normal(rng, (offsets[-1], k))
    got = _gemm(hip, x_bits, experts, s2, offsets, n, k)
    ref = _oracle(x_bits, experts, s2, offsets, n, None, "bf16w")
    _check_gemm(got, ref, _acc_bound(x_bits, experts, s2, offsets, None, k))


def test_row_cut_off_inside_an_overflow_chunk(hip):
    """Experts of 150 and 100 rows (past 64: more blocks per expert), max_rows cutting the
    second expert's rows inside its first chunk and the first expert's third chunk whole."""
    rng = np.random.default_rng(8)
    n, k = 32, 256
    counts = [150, 100]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    x_bits = wl.bf16_normal(rng, (offsets[-1], k))
    experts = [wl.random_nvfp4(rng, n, k) for _ in counts]
    s2 = np.array([0.75, 1.5], np.float32)
    ref = _oracle(x_bits, experts, s2, offsets, n, None, "bf16w")
    for rows in (130, 180, 250):
        got = _gemm(hip, x_bits, experts, s2, offsets, n, k, rows=rows, c_rows=250)
        assert np.all(got[rows:] == -3.0)
        assert rel_err(got[:rows], ref[:rows]) <= GATE


def test_out_of_range_gather_reads_zeros(hip):
    rng = np.random.default_rng(7)
    n, k, t = 32, 256, 8
    x_bits = wl.bf16_normal(rng, (t, k))
    ex = [wl.random_nvfp4(rng, n, k)]
    gather = np.array([0, -1, 3, t, 7, 100000])
    got = _gemm(hip, x_bits, ex, np.ones(1, np.float32), np.array([0, 6]), n, k, gather)
    assert np.all(got[[1, 3, 5]] == 0.0)
    ok = [0, 2, 4]
    ref = _oracle(x_bits, ex, np.ones(1, np.float32), np.array([0, 3]), n,
                  gather[ok], "bf16w")
    assert rel_err(got[ok], ref) <= GATE


def test_rejects_bad_shapes(hip):
    table = upload_table(hip, [wl.random_nvfp4(np.random.default_rng(0), 32, 256)],
                         [1.0], 32, 256)
    a = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    table.k = 200  # not a multiple of 256
    with pytest.raises(hip.MoeError):
        hip.moe_w4a16_grouped_gemm(a, table, off, c)
    table.k, table.n = 256, 24  # not a multiple of 16
    with pytest.raises(hip.MoeError):
        hip.moe_w4a16_grouped_gemm(a, table, off, c)


# ------------------------------------------------------------------ full-size samples

@pytest.mark.timeout(900)
@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_prefill_subchunk_gemms_every_expert(hip, which):
    """The 256-expert, 256-row sub-chunk GEMMs at full size in the bench's launch
    configuration (all 2048 sorted rows, every expert), against the oracle over the whole
    output and row by row."""
    w = wl.WORKLOADS["prefill_subchunk"]
    ids, _ = wl.routing(w)
    al = moe.align(ids, w.num_experts)
    offsets = al["expert_offsets"]
    n, k = wl.gate_up_shape(w) if which == "gate_up" else wl.down_shape(w)
    gu, dn, gt, dt = workload_tables(hip, w)
    experts, table = (gu, gt) if which == "gate_up" else (dn, dt)
    s2 = wl.scale2_gate_up(w) if which == "gate_up" else wl.scale2_down(w)
    if which == "gate_up":
        x_bits, gather = wl.activations(w), al["sorted_token_ids"]
    else:  # the down GEMM reads its rows in order; seeded BF16 rows stand in for act
        x_bits = wl.bf16_normal(np.random.default_rng(99), (offsets[-1], k))
        gather = None
    got = _gemm(hip, x_bits, experts, s2, offsets, n, k, gather, fill=0.0, table=table)
    ref = np.full(got.shape, np.nan)
    with oracle_threads():
        moe.grouped_gemm(codecs.bf16_bits_to_f64(x_bits), gather, experts, s2, offsets, ref,
                         "bf16w", workers=ORACLE_WORKERS)
    assert not np.isnan(ref).any()  # every expert of the table has rows here
    r, rr = rel_err(got, ref), rel_err_rows(got, ref)
    print(f"{which}: {r:.2e} (worst row {rr:.2e})")
    assert r <= GATE and rr <= GATE
