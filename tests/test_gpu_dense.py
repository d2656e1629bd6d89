"""The shared expert's BF16 GEMMs (moe_dense_gemm_bf16, moe_dense_gate_up_swiglu_bf16)
against the oracle's dense_mlp.

- moe_dense_gemm_bf16 against the oracle's BF16-rounded product (dense_mlp's gate
  stage) over shapes that reach every tile shape the launcher picks, ragged rows, a
  column-tile count that does not divide by 8, strided views and K = 0.
- The gate/up form gives the bits of two plain GEMMs followed by swiglu_clamp, and the
  oracle's activation within the gate, including clamped values.
- The shared expert (both calls) at the layer workloads' full sizes, and the routed
  layer with the shared expert in its combine, against the oracle.
- The split-K form (with a workspace) against the oracle, repeated calls give the same
  bits, one workspace serves calls of two shapes in turn, and its gate/up form gives the
  bits of the two plain split-K GEMMs followed by swiglu_clamp.
- Nothing outside the output rows and columns is written; bad arguments raise.

Tolerance: the parity gate, max |gpu - oracle| / max |oracle| <= 5e-3 against the FP64
oracle with the pages' BF16 buffers (FP32 accumulation in another order moves an output
by at most about one BF16 ulp of the largest value, 2^-8 of it).
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import GATE, bf16_bits_host, bf16_dev, f64, rel_err, workload_tables
from oracle import codecs, moe

pytestmark = pytest.mark.gpu

POISON = -1  # 0xFFFF: a BF16 NaN


def _bf16(bits):
    return codecs.bf16_bits_to_f64(bits)


def _operands(seed, m, n, k, w_scale=1.0):
    rng = np.random.default_rng(seed)
    a = wl.bf16_normal(rng, (m, k))
    b = wl.bf16_normal_scaled(rng, (n, k), w_scale / np.sqrt(max(k, 1)))
    return a, b


def _gemm_ref(a_bits, b_bits):
    """The oracle's BF16 product a @ b^T (dense_mlp's gate stage)."""
    a, b = _bf16(a_bits), _bf16(b_bits)
    zeros = np.zeros((b.shape[1], b.shape[0]))
    _, mid = moe.dense_mlp(a, b, b, zeros, 7.0, "bf16w")
    return mid["gate"]


def _padded(rows, cols, pad_r=0, pad_c=0):
    """A POISON-filled [rows + pad_r, cols + pad_c] buffer and its [rows, cols] view."""
    buf = torch.empty((rows + pad_r, cols + pad_c), dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(POISON)
    return buf, buf[:rows, :cols]


def _untouched(buf, rows, cols):
    bits = bf16_bits_host(buf)
    mask = np.ones(bits.shape, bool)
    mask[:rows, :cols] = False
    return bool(np.all(bits[mask] == 0xFFFF))


# (m, n, k): every tile shape the launcher picks on a 256-CU part, ragged row tiles,
# 5 column tiles (no XCD grouping), one 16-column tile.
GEMM_SHAPES = [
    (1, 16, 64), (5, 48, 128), (16, 256, 512), (17, 80, 192), (33, 512, 256), (64, 768, 2048),
    (100, 2048, 768), (256, 2048, 128), (256, 6144, 64), (20, 32768, 64), (5, 32768, 64),
    (4096, 512, 128),
]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_dense_gemm_vs_oracle(hip, m, n, k):
    a_bits, b_bits = _operands(m * 7 + n + k, m, n, k)
    buf, c = _padded(m, n, 3, 16)
    hip.moe_dense_gemm_bf16(bf16_dev(a_bits), bf16_dev(b_bits), c)
    torch.cuda.synchronize()
    got = f64(c)
    ref = _gemm_ref(a_bits, b_bits)
    assert rel_err(got, ref) <= GATE
    # most outputs carry the oracle's exact bits (FP32 sums round the same way)
    assert np.mean(got == ref) > 0.97
    assert _untouched(buf, m, n)


def test_dense_gemm_strided_views_and_k_zero(hip):
    m, n, k = 40, 96, 320
    a_bits, b_bits = _operands(5, m, n, k)
    a_full = torch.zeros((m, k + 24), dtype=torch.bfloat16, device="cuda")
    a_full[:, 8:8 + k] = bf16_dev(a_bits)
    b_full = torch.zeros((n, k + 8), dtype=torch.bfloat16, device="cuda")
    b_full[:, :k] = bf16_dev(b_bits)
    buf, c = _padded(m, n, 0, 12)
    hip.moe_dense_gemm_bf16(a_full[:, 8:8 + k], b_full[:, :k], c)
    torch.cuda.synchronize()
    assert rel_err(f64(c), _gemm_ref(a_bits, b_bits)) <= GATE
    assert _untouched(buf, m, n)
    # K = 0: the empty sum
    hip.moe_dense_gemm_bf16(a_full[:, :0], b_full[:, :0], c)
    torch.cuda.synchronize()
    assert np.all(f64(c) == 0.0) and _untouched(buf, m, n)
    # M = 0 and N = 0 enqueue nothing
    hip.moe_dense_gemm_bf16(a_full[:0, :k], b_full[:, :k], c[:0])
    hip.moe_dense_gemm_bf16(a_full[:, :k], b_full[:0, :k], c[:, :0])


def _check_against_oracle(a_bits, g_bits, u_bits, gate, up, act, limit, w_scale):
    """The gate/up form against the oracle's dense_mlp. G and U (the GEMM outputs the fused
    form reproduces bit for bit) at the parity gate; the activation at the gate when the
    weights are unscaled. With scaled weights most outputs sit at the clamp and reach
    ~49: there one BF16 rounding flip of U (the pages' BF16 buffer; FP32 and FP64 sums
    round to neighbours now and then) moves an output by silu(7) * ulp(U) ~ 0.22, up to
    one BF16 ulp of the largest output (2^-7 of it, above the 5e-3 gate), so the
    activation is checked elementwise within the bound from one such flip of G and of U
    plus the output rounding."""
    zeros = np.zeros((8, g_bits.shape[0]))
    _, mid = moe.dense_mlp(_bf16(a_bits), _bf16(g_bits), _bf16(u_bits), zeros, limit, "bf16w")
    assert rel_err(f64(gate), mid["gate"]) <= GATE
    assert rel_err(f64(up), mid["up"]) <= GATE
    got = f64(act)
    if w_scale <= 4:
        assert rel_err(got, mid["act"]) <= GATE
    else:
        assert np.mean(np.abs(mid["gate"]) > limit) > 0.05  # the clamp was exercised
        ulp = lambda v: 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126))) - 7)
        silu_max = limit / (1.0 + np.exp(-limit))
        # silu' <= 1.1 everywhere; |clamped U| <= limit; FP32 swiglu: a few 2^-24
        bound = 0.5 * ulp(mid["act"]) + silu_max * ulp(np.clip(mid["up"], -limit, limit)) \
            + 1.1 * limit * ulp(np.minimum(mid["gate"], limit)) + 1e-6 * np.abs(mid["act"])
        assert np.all(np.abs(got - mid["act"]) <= bound)
        assert rel_err(got, mid["act"]) <= 2.0 ** -7 + 2.0 ** -9


# (m, inter, k, weight scale): every tile shape of the gate/up form on a 256-CU part;
# scales 6 and 8 push many gate and up values past the clamp.
@pytest.mark.parametrize("m,inter,k,w_scale", [
    (1, 16, 64, 1.0), (19, 48, 192, 6.0), (1, 6144, 128, 1.0), (17, 6144, 64, 6.0),
    (33, 2048, 192, 1.0), (33, 4096, 64, 8.0), (256, 2048, 256, 1.0), (100, 768, 2048, 8.0),
    (4096, 256, 128, 1.0),
])
def test_gate_up_swiglu_bits_and_oracle(hip, m, inter, k, w_scale):
    rng_seed = m + inter + k
    a_bits, g_bits = _operands(rng_seed, m, inter, k, w_scale)
    _, u_bits = _operands(rng_seed + 1, m, inter, k, w_scale)
    a, g, u = bf16_dev(a_bits), bf16_dev(g_bits), bf16_dev(u_bits)
    limit = 7.0
    buf, act = _padded(m, inter, 2, 8)
    hip.moe_dense_gate_up_swiglu_bf16(a, g, u, act, limit)
    # the two plain GEMMs, then swiglu_clamp
    gate = torch.empty((m, inter), dtype=torch.bfloat16, device="cuda")
    up = torch.empty_like(gate)
    ref_act = torch.empty_like(gate)
    hip.moe_dense_gemm_bf16(a, g, gate)
    hip.moe_dense_gemm_bf16(a, u, up)
    hip.swiglu_clamp(gate, up, ref_act, limit)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(act), bf16_bits_host(ref_act))
    assert _untouched(buf, m, inter)
    _check_against_oracle(a_bits, g_bits, u_bits, gate, up, act, limit, w_scale)


# Split-K form (with a workspace): (m, n, k) with K split 4, 2 and 1 ways, ragged row and
# column tiles, a column-tile count that does not divide by 8, the shared expert's shapes,
# and 64-k steps per split of every remainder modulo 6 (the register-staged loop runs six
# steps per trip with three register sets; 1, 3, 5, 8, 11, 12, 16 and 24 steps here).
# Grids of at most one block per CU take the LDS-direct kernel; (520, 8192, 512) has 320
# blocks and takes the register-staged one.
SPLITK_SHAPES = [
    (1, 16, 64), (17, 80, 192), (130, 272, 1024), (100, 2048, 768), (300, 4096, 512),
    (256, 2048, 6144), (256, 6144, 2048), (33, 48, 4096), (40, 96, 320), (70, 160, 704),
    (520, 8192, 512),
]


@pytest.mark.parametrize("m,n,k", SPLITK_SHAPES)
def test_dense_gemm_split_k_vs_oracle(hip, m, n, k):
    a_bits, b_bits = _operands(m * 5 + n + k, m, n, k)
    a, b = bf16_dev(a_bits), bf16_dev(b_bits)
    ws = hip.dense_workspace(m, n, k)
    buf, c = _padded(m, n, 3, 16)
    hip.moe_dense_gemm_bf16(a, b, c, workspace=ws)
    torch.cuda.synchronize()
    got = f64(c)
    ref = _gemm_ref(a_bits, b_bits)
    assert rel_err(got, ref) <= GATE
    assert np.mean(got == ref) > 0.97
    assert _untouched(buf, m, n)
    # deterministic: a second call over a workspace full of the first call's partials
    first = bf16_bits_host(c).copy()
    hip.moe_dense_gemm_bf16(a, b, c, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(c), first)


def test_dense_split_k_workspace_shared_by_two_shapes(hip):
    """One workspace for the gate/up form and the plain GEMM of another shape, in turns
    (stream-ordered), three times: the same bits each time and the oracle's values."""
    m, inter, k = 200, 1024, 1536
    a_bits, g_bits = _operands(41, m, inter, k)
    _, u_bits = _operands(42, m, inter, k)
    _, d_bits = _operands(43, m, k, inter)
    a, g, u, d = (bf16_dev(x) for x in (a_bits, g_bits, u_bits, d_bits))
    ws = torch.zeros(max(hip.moe_dense_workspace_bytes(m, inter, k, True),
                         hip.moe_dense_workspace_bytes(m, k, inter, False)),
                     dtype=torch.uint8, device="cuda")
    act = torch.empty((m, inter), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    runs = []
    for _ in range(3):
        hip.moe_dense_gate_up_swiglu_bf16(a, g, u, act, 7.0, workspace=ws)
        hip.moe_dense_gemm_bf16(act, d, out, workspace=ws)
        torch.cuda.synchronize()
        runs.append((bf16_bits_host(act).copy(), bf16_bits_host(out).copy()))
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0]) and np.array_equal(r[1], runs[0][1])
    ref, mid = moe.dense_mlp(_bf16(a_bits), _bf16(g_bits), _bf16(u_bits), _bf16(d_bits), 7.0,
                             "bf16w")
    assert rel_err(f64(act), mid["act"]) <= GATE
    assert rel_err(f64(out), ref) <= GATE


@pytest.mark.parametrize("m,inter,k,w_scale", [
    (33, 48, 192, 6.0), (19, 16, 1024, 6.0), (100, 768, 2048, 8.0), (256, 2048, 6144, 1.0),
    (520, 4096, 512, 1.0),  # 320 blocks: the register-staged kernel
])
def test_gate_up_swiglu_split_k_bits_and_oracle(hip, m, inter, k, w_scale):
    a_bits, g_bits = _operands(m + inter + k + 1, m, inter, k, w_scale)
    _, u_bits = _operands(m + inter + k + 2, m, inter, k, w_scale)
    a, g, u = bf16_dev(a_bits), bf16_dev(g_bits), bf16_dev(u_bits)
    limit = 7.0
    ws = hip.dense_workspace(m, inter, k, swiglu=True)
    buf, act = _padded(m, inter, 2, 8)
    hip.moe_dense_gate_up_swiglu_bf16(a, g, u, act, limit, workspace=ws)
    # the two plain split-K GEMMs (one workspace, stream-ordered), then swiglu_clamp
    ws_plain = hip.dense_workspace(m, inter, k)
    gate = torch.empty((m, inter), dtype=torch.bfloat16, device="cuda")
    up = torch.empty_like(gate)
    ref_act = torch.empty_like(gate)
    hip.moe_dense_gemm_bf16(a, g, gate, workspace=ws_plain)
    hip.moe_dense_gemm_bf16(a, u, up, workspace=ws_plain)
    hip.swiglu_clamp(gate, up, ref_act, limit)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(act), bf16_bits_host(ref_act))
    assert _untouched(buf, m, inter)
    _check_against_oracle(a_bits, g_bits, u_bits, gate, up, act, limit, w_scale)


def test_dense_split_k_workspace_errors(hip):
    m, n, k = 64, 128, 1024
    a = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((m, n), dtype=torch.bfloat16, device="cuda")
    need = hip.moe_dense_workspace_bytes(m, n, k)
    small = torch.zeros(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(hip.MoeError) as e:  # MOE_ECAPACITY
        hip.moe_dense_gemm_bf16(a, b, c, workspace=small)
    assert e.value.status == 2
    big = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(hip.MoeError):  # not 256-byte aligned
        hip.moe_dense_gemm_bf16(a, b, c, workspace=big[16:16 + need])


def _shared_on_device(hip, w, scale=1.0):
    g, u, d = wl.shared_expert(w, scale)
    return (g, u, d), hip.SharedExpert(bf16_dev(g), bf16_dev(u), bf16_dev(d), w.rows)


@pytest.mark.parametrize("name", ["layer_e64", "prefill_subchunk"])
def test_shared_expert_full_size_vs_oracle(hip, name):
    w = wl.WORKLOADS[name]
    (g, u, d), se = _shared_on_device(hip, w)
    x_bits = wl.activations(w)
    out = se(bf16_dev(x_bits), w.limit)
    torch.cuda.synchronize()
    ref, mid = moe.dense_mlp(_bf16(x_bits), _bf16(g), _bf16(u), _bf16(d), w.limit, "bf16w")
    assert rel_err(f64(se.act[:w.rows]), mid["act"]) <= GATE
    assert rel_err(f64(out), ref) <= GATE


def test_shared_expert_few_rows(hip):
    # the verify-sweep width: 8 rows of the small-M workload's sizes
    w = wl.WORKLOADS["small_m"]
    (g, u, d), se = _shared_on_device(hip, w, scale=3.0)
    x_bits = wl.activations(w)
    out = se(bf16_dev(x_bits), w.limit)
    torch.cuda.synchronize()
    ref, _ = moe.dense_mlp(_bf16(x_bits), _bf16(g), _bf16(u), _bf16(d), w.limit, "bf16w")
    assert rel_err(f64(out), ref) <= GATE


def test_layer_with_shared_expert_vs_oracle(hip):
    w = wl.WORKLOADS["layer_e64"]
    gu, dn, gt, dt = workload_tables(hip, w)
    (g, u, d), se = _shared_on_device(hip, w)
    x_bits = wl.activations(w)
    ids, wts = wl.routing(w)
    ws = hip.Workspace(w.rows, w.top_k, w.num_experts, w.hidden, w.moe_intermediate)
    out = torch.empty((w.rows, w.hidden), dtype=torch.bfloat16, device="cuda")
    x = bf16_dev(x_bits)
    hip.moe_layer(x, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), gt, dt,
                  w.moe_intermediate, w.limit, ws, out, shared=se)
    torch.cuda.synchronize()
    xf = _bf16(x_bits)
    shared_ref, _ = moe.dense_mlp(xf, _bf16(g), _bf16(u), _bf16(d), w.limit, "bf16w")
    ref, _ = moe.moe_layer(xf, ids, wts, gu, dn, wl.scale2_gate_up(w),
                           wl.scale2_down(w), w.moe_intermediate, w.limit, "bf16w",
                           shared=shared_ref)
    assert rel_err(f64(out), ref) <= GATE


def test_dense_bad_arguments(hip):
    a = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((32, 128), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hip.MoeError):  # N not a multiple of 16
        hip.moe_dense_gemm_bf16(a, b[:24], c[:, :24])
    with pytest.raises(hip.MoeError):  # K not a multiple of 64
        hip.moe_dense_gemm_bf16(a[:, :96], b[:, :96], c)
    with pytest.raises(hip.MoeError):  # a misaligned by one element
        hip.moe_dense_gemm_bf16(a.view(-1)[1:1 + 4 * 64].view(4, 64), b[:, :64], c)
    with pytest.raises(hip.MoeError):  # limit must be positive
        hip.moe_dense_gate_up_swiglu_bf16(a, b, b, c, 0.0)
    with pytest.raises(ValueError):  # shape mismatch caught by the binding
        hip.moe_dense_gemm_bf16(a, b, c[:, :16])
