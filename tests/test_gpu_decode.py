"""The decode / verify path on the GPU against the oracle: moe_row_union (bit-exact),
moe_w4a16_gemv_union and its SwiGLU-fused form (one-hot layout pins exact, per-element
FP32 accumulation bound, fused == unfused bits), and the whole layer through the union.
"""

import types

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import codecs, moe
from gpu_util import GATE, LazyExperts, bf16_bits_host, bf16_dev, dev, f64, rel_err, upload_table

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------- row union

def _union_gpu(hip, ids, num_experts, present=None):
    rows, top_k = ids.shape
    t = rows * top_k
    i32 = dict(dtype=torch.int32, device="cuda")
    u_eid = torch.full((t,), -7, **i32)
    u_slot = torch.full((t * rows,), -7, **i32)
    perm = torch.full((t,), -7, **i32)
    cnt = torch.full((2,), -7, **i32)
    table = None
    if present is not None:  # a stand-in table: only its pointer array is read
        ptrs = np.where(present, 0x1000, 0).astype(np.int64)
        table = types.SimpleNamespace(num_experts=num_experts, packed_ptrs=dev(ptrs))
    hip.moe_row_union(dev(ids.astype(np.int32)), num_experts, u_eid, u_slot, perm, cnt,
                      present=table)
    torch.cuda.synchronize()
    return (u_eid.cpu().numpy(), u_slot.cpu().numpy().reshape(t, rows), perm.cpu().numpy(),
            cnt.cpu().numpy())


@pytest.mark.parametrize("rows,top_k,num_experts,seed", [
    (1, 8, 256, 0), (8, 8, 256, 1), (8, 8, 16, 2), (5, 3, 7, 3), (16, 8, 64, 4),
    (128, 8, 256, 5), (1024, 1, 40, 6), (64, 16, 2048, 7),
    # more than 64 ids with expert ids past the LDS map (8192): the pairwise-scan kernel
    (100, 2, 1 << 20, 13), (9, 8, 9000, 14),
    # at most 64 ids (the one-wave kernel): one id per row, one row of 64, a single
    # expert, heavy repeats, ids of 20 bits
    (64, 1, 3, 8), (1, 64, 100, 9), (2, 32, 1, 10), (7, 9, 5, 11), (4, 16, 1 << 20, 12)])
def test_row_union_bit_exact(hip, rows, top_k, num_experts, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, num_experts + 2, size=(rows, top_k)).astype(np.int32)
    if rows > 1:
        ids[1] = ids[0][::-1]
    if top_k > 2:
        ids[0, 2] = ids[0, 1]  # a repeat inside a row: not covered
    u_eid, u_slot, perm, cnt = _union_gpu(hip, ids, num_experts)
    ref = moe.row_union(ids, num_experts)
    assert np.array_equal(u_eid, ref["u_eid"])
    assert np.array_equal(u_slot, ref["u_slot"])
    assert np.array_equal(perm, ref["slot_perm"].reshape(-1))
    assert cnt.tolist() == [ref["n_union"], ref["n_uncovered"]]


@pytest.mark.parametrize("rows,top_k,num_experts,seed", [
    (8, 8, 256, 20), (3, 5, 11, 21), (16, 8, 64, 22), (128, 8, 256, 23)])
def test_row_union_present_mask_bit_exact(hip, rows, top_k, num_experts, seed):
    """Experts absent from a table (null entries) are left out, in the one-wave kernel
    (at most 64 ids) and the block-wide one."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, num_experts + 1, size=(rows, top_k)).astype(np.int32)
    ids[1] = ids[0][::-1]
    present = rng.random(num_experts) < 0.5
    u_eid, u_slot, perm, cnt = _union_gpu(hip, ids, num_experts, present)
    ref = moe.row_union(ids, num_experts, present)
    assert np.array_equal(u_eid, ref["u_eid"])
    assert np.array_equal(u_slot, ref["u_slot"])
    assert np.array_equal(perm, ref["slot_perm"].reshape(-1))
    assert cnt.tolist() == [ref["n_union"], ref["n_uncovered"]]


def test_row_union_softmax_routing_and_limits(hip):
    w = wl.WORKLOADS["small_m"]
    ids, _ = wl.routing(w)
    u_eid, u_slot, perm, cnt = _union_gpu(hip, ids, w.num_experts)
    ref = moe.row_union(ids, w.num_experts)
    assert np.array_equal(u_eid, ref["u_eid"]) and np.array_equal(u_slot, ref["u_slot"])
    assert cnt[1] == 0 and np.array_equal(perm, np.arange(ids.size))
    i32 = dict(dtype=torch.int32, device="cuda")
    with pytest.raises(hip.MoeError):  # more than one workgroup of ids
        big = torch.zeros((129, 8), **i32)
        hip.moe_row_union(big, 16, torch.empty(129 * 8, **i32), torch.empty(129 * 8 * 129, **i32))
    empty = torch.zeros((0, 8), **i32)
    hip.moe_row_union(empty, 16, torch.empty(1, **i32), torch.empty(1, **i32))  # no-op


# --------------------------------------------------------------------------- union GEMV

def _problem(seed, rows, top_k, num_experts, n, k, null=(), repeat=False):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    if rows > 2:
        ids[2, 0] = -1  # an unfilled slot
    if repeat and top_k > 1:
        ids[0, 1] = ids[0, 0]
    experts = [None if e in null else wl.random_nvfp4(rng, n, k) for e in range(num_experts)]
    s2 = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    return rng, ids, experts, s2


def _gemv_gpu(hip, a_bits, per_slot, experts, s2, ids, n, k, fill=-3.0):
    rows, top_k = ids.shape
    num_experts = len(experts)
    table = upload_table(hip, experts, s2, n, k)
    u_eid, u_slot, _, _ = _union_gpu(hip, ids, num_experts)
    c = torch.full((rows * top_k, n), fill, dtype=torch.bfloat16, device="cuda")
    hip.moe_w4a16_gemv_union(bf16_dev(a_bits), table, dev(u_eid), dev(u_slot.reshape(-1)), c,
                             rows, top_k, a_per_slot=per_slot)
    torch.cuda.synchronize()
    return f64(c), table, u_eid, u_slot


def _oracle_gemv(a_bits, per_slot, experts, s2, ids, n, mode="bf16w", fill=np.nan):
    rows, top_k = ids.shape
    un = moe.row_union(ids, len(experts))
    out = np.full((rows * top_k, n), fill)
    moe.union_gemv(codecs.bf16_bits_to_f64(a_bits), per_slot, experts, s2, un["u_eid"],
                   un["u_slot"], top_k, out, mode)
    return out


def _abs_bound(a_bits, per_slot, experts, s2, ids, n, k):
    """gamma_K * sum_k |a w| per element: the FP32 accumulation bound, any order."""
    rows, top_k = ids.shape
    s_abs = np.full((rows * top_k, n), np.nan)
    un = moe.row_union(ids, len(experts))
    a_abs = np.abs(codecs.bf16_bits_to_f64(a_bits))
    for p in range(un["n_union"]):
        e = int(un["u_eid"][p])
        if experts[e] is None:
            continue
        w = np.abs(moe.dequant(experts[e][0], experts[e][1], float(s2[e]), "bf16w"))
        for r in range(rows):
            j = int(un["u_slot"][p, r])
            if j >= 0:
                t = r * top_k + j
                s_abs[t] = a_abs[t if per_slot else r] @ w.T
    gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    return gamma * s_abs


def _check(got, ref, bound):
    mask = ~np.isnan(ref)
    err = np.abs(got - ref)
    lim = np.ldexp(1.0, np.frexp(np.abs(ref) + bound)[1] - 8) * 0.5 + bound * 1.001 + 1e-30
    assert np.all(err[mask] <= lim[mask]), float(np.max((err - lim)[mask]))
    assert rel_err(got[mask], ref[mask]) <= GATE


@pytest.mark.parametrize("rows,top_k,num_experts,n,k,per_slot", [
    (8, 8, 32, 256, 512, False),     # K = 2 steps: no K split
    (8, 8, 32, 256, 2048, True),     # 8 steps: two waves split K
    (3, 4, 9, 48, 6144, False),      # 24 steps: four waves split K; N not a block multiple
    (16, 2, 40, 160, 2304, True),    # 16 rows, 9 steps, ragged groups
    (1, 8, 300, 64, 768, False),     # one row: every entry has one token
    # at most 8 rows: activations staged per wave in LDS, 2 tokens per load (1, 2, 4 loads)
    (2, 8, 64, 96, 6144, True),      # one load per step, four waves split K
    (4, 8, 16, 128, 1024, True),     # two loads per step, no K split
    (5, 6, 20, 80, 4096, False),     # four loads per step, an odd token count
    # the most ids a launch takes (512 entries' metadata in LDS), staged and direct
    (8, 64, 600, 32, 512, False),
    (16, 32, 560, 32, 256, True),
])
def test_gemv_union_vs_oracle(hip, rows, top_k, num_experts, n, k, per_slot):
    rng, ids, experts, s2 = _problem(rows * 100 + k, rows, top_k, num_experts, n, k,
                                     null=(3, 5), repeat=True)
    a_bits = wl.bf16_normal(rng, (rows * top_k if per_slot else rows, k))
    got, _, _, _ = _gemv_gpu(hip, a_bits, per_slot, experts, s2, ids, n, k, fill=-3.0)
    ref = _oracle_gemv(a_bits, per_slot, experts, s2, ids, n)
    _check(got, ref, _abs_bound(a_bits, per_slot, experts, s2, ids, n, k))
    # rows no entry writes (unfilled, repeated or null-expert slots) keep the caller's value
    assert np.all(got[np.isnan(ref)] == -3.0)


@pytest.mark.parametrize("k", [512, 2048, 6144])
def test_gemv_union_one_hot_layout_is_exact(hip, k):
    # W_e[n, k] = 1 at k = pi_e(n) (nibble 2, scale code 0x38 = 1.0, scale2 1): every output
    # is one input element, exactly. Pins the lane -> k mapping, the scale dword, the row
    # gather and the (row, slot) output layout of every K split.
    rng = np.random.default_rng(k)
    rows, top_k, num_experts, n = 6, 4, 10, 96
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    experts, pis = [], []
    for e in range(num_experts):
        pi = rng.integers(0, k, n)
        nib = np.zeros((n, k), np.uint8)
        nib[np.arange(n), pi] = 2
        packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        experts.append((packed, np.full((n, k // 16), 0x38, np.uint8)))
        pis.append(pi)
    for per_slot in (False, True):
        a_bits = wl.bf16_normal(rng, (rows * top_k if per_slot else rows, k))
        got, _, _, _ = _gemv_gpu(hip, a_bits, per_slot, experts, np.ones(num_experts), ids, n, k)
        a = codecs.bf16_bits_to_f64(a_bits)
        for r in range(rows):
            for j in range(top_k):
                e, t = int(ids[r, j]), r * top_k + j
                assert np.array_equal(got[t], a[t if per_slot else r, pis[e]])


def test_gemv_union_swiglu_is_unfused_bits(hip):
    rng, ids, experts, s2 = _problem(61, 8, 8, 24, 2 * 160, 6144, null=(7,))
    mi = 160
    # gate_up weights with magnitudes that drive values past the clamp
    a_bits = codecs.bf16_bits_from_f32((rng.standard_normal((8, 6144)) * 3).astype(np.float32))
    plain, table, u_eid, u_slot = _gemv_gpu(hip, a_bits, False, experts, s2, ids, 2 * mi, 6144)
    act = torch.full((64, mi), -5.0, dtype=torch.bfloat16, device="cuda")
    hip.moe_w4a16_gemv_union_swiglu(bf16_dev(a_bits), table, dev(u_eid),
                                    dev(u_slot.reshape(-1)), act, 7.0, 8, 8)
    ref = torch.full((64, mi), -5.0, dtype=torch.bfloat16, device="cuda")
    c = torch.tensor(plain, dtype=torch.bfloat16, device="cuda")  # exact: plain is BF16
    covered = torch.tensor(~np.isnan(_oracle_gemv(a_bits, False, experts, s2, ids, 2 * mi)[:, 0]),
                           device="cuda")
    hip.swiglu_clamp(c[:, :mi], c[:, mi:], ref, 7.0)
    torch.cuda.synchronize()
    got_b, ref_b = bf16_bits_host(act), bf16_bits_host(ref)
    cov = covered.cpu().numpy()
    assert np.array_equal(got_b[cov], ref_b[cov])
    assert np.all(f64(act)[~cov] == -5.0)


def test_gemv_union_argument_errors(hip):
    rng, ids, experts, s2 = _problem(3, 4, 2, 4, 32, 256)
    table = upload_table(hip, experts, s2, 32, 256)
    i32 = dict(dtype=torch.int32, device="cuda")
    a = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((34, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hip.MoeError):  # more rows than one matrix-core tile
        hip.moe_w4a16_gemv_union(a, table, torch.zeros(34, **i32), torch.zeros(34 * 17, **i32),
                                 c, 17, 2)
    # rows == 0 enqueues nothing
    hip.moe_w4a16_gemv_union(a, table, torch.zeros(1, **i32), torch.zeros(1, **i32), c, 0, 2)


# --------------------------------------------------------------------------- layer

def _decode_layer(hip, w, ids, wts, x_bits, gt, dt, fused=True):
    rows, top_k = ids.shape
    ws = hip.DecodeWorkspace(rows, top_k, w.hidden, w.moe_intermediate)
    for t in (ws.gate_up, ws.act, ws.expert_out):
        t.view(torch.int16).fill_(-1)  # NaN: a row read before it is written poisons the output
    out = torch.empty((rows, w.hidden), dtype=torch.bfloat16, device="cuda")
    hip.moe_layer_decode(bf16_dev(x_bits), dev(ids), dev(wts), gt, dt, w.moe_intermediate,
                         w.limit, ws, out, fused=fused)
    torch.cuda.synchronize()
    return f64(out), ws


@pytest.mark.parametrize("fused", [True, False])
def test_decode_layer_small_m_vs_oracle(hip, fused):
    """8 rows over 256 experts (hidden 6144, mi 2048), experts [128, 256) null: every
    output row of the union path against the oracle's decode layer."""
    w = wl.WORKLOADS["small_m"]
    ids, wts = wl.routing(w)
    x_bits = wl.activations(w)
    live = sorted({int(e) for e in ids.reshape(-1) if not w.is_null(int(e))})
    gu, dn = LazyExperts(w, "gate_up"), LazyExperts(w, "down")
    gt = upload_table(hip, gu, wl.scale2_gate_up(w), *wl.gate_up_shape(w), only=set(live))
    dt = upload_table(hip, dn, wl.scale2_down(w), *wl.down_shape(w), only=set(live))
    got, ws = _decode_layer(hip, w, ids, wts, x_bits, gt, dt, fused)
    ref, inter = moe.moe_layer_decode(codecs.bf16_bits_to_f64(x_bits), ids, wts, gu, dn,
                                      wl.scale2_gate_up(w), wl.scale2_down(w),
                                      w.moe_intermediate, w.limit, "bf16w")
    assert rel_err(got, ref) <= GATE
    # the layer's union leaves out the experts absent from the table (the combine skips
    # their slots, so no zero-first step is needed); the oracle's layer keeps them and adds
    # their zeros: the same outputs
    present = np.isin(np.arange(w.num_experts), live)
    un = moe.row_union(ids, w.num_experts, present)
    assert np.array_equal(ws.u_eid.cpu().numpy(), un["u_eid"])
    assert np.array_equal(ws.slot_perm.cpu().numpy()[:ids.size], un["slot_perm"].reshape(-1))
    for r in range(w.rows):  # a row whose experts are all null gets exactly zero
        if all(w.is_null(int(e)) for e in ids[r]):
            assert np.all(got[r] == 0.0)


def test_decode_layer_matches_sorted_layer_ragged(hip):
    """5 rows, top_k 3, 12 experts with two absent and an unfilled slot: the union path and
    the sorted path both against the oracle (the oracle's two layers agree by their pins)."""
    w = wl.custom("decode_ragged", 91, rows=5, num_experts=12, top_k=3, hidden=512,
                  moe_intermediate=256)
    ids, wts = wl.routing(w)
    ids = ids.copy()
    ids[1, 2] = -1
    x_bits = wl.activations(w)
    null = (4, 9)
    gu, dn = LazyExperts(w, "gate_up", null), LazyExperts(w, "down", null)
    gt = upload_table(hip, gu, wl.scale2_gate_up(w), *wl.gate_up_shape(w))
    dt = upload_table(hip, dn, wl.scale2_down(w), *wl.down_shape(w))
    got, _ = _decode_layer(hip, w, ids, wts, x_bits, gt, dt)
    ws = hip.Workspace(5, 3, w.num_experts, w.hidden, w.moe_intermediate)
    out = torch.empty((5, w.hidden), dtype=torch.bfloat16, device="cuda")
    hip.moe_layer(bf16_dev(x_bits), dev(ids), dev(wts), gt, dt, w.moe_intermediate, w.limit, ws,
                  out)
    torch.cuda.synchronize()
    gu_l = [gu[e] for e in range(w.num_experts)]
    dn_l = [dn[e] for e in range(w.num_experts)]
    ref, _ = moe.moe_layer_decode(codecs.bf16_bits_to_f64(x_bits), ids, wts, gu_l, dn_l,
                                  wl.scale2_gate_up(w), wl.scale2_down(w), w.moe_intermediate,
                                  w.limit, "bf16w")
    assert rel_err(got, ref) <= GATE
    assert rel_err(f64(out), ref) <= GATE


@pytest.mark.parametrize("rows,cut", [(8, 3), (12, 4), (16, 2)])
def test_gemv_union_row_result_independent_of_sharing(hip, rows, cut):
    """Which rows share a sweep never changes what a row gets: the same rows run as one
    union and split into two unions give the same bits for every (row, slot). The cuts
    also cross the launch forms (activations staged in LDS for at most 8 rows, with 1, 2
    or 4 loads per step; loaded directly above 8)."""
    rng, ids, experts, s2 = _problem(71 + rows, rows, 8, 24, 256, 2048)
    a_bits = wl.bf16_normal(rng, (rows, 2048))
    whole, _, _, _ = _gemv_gpu(hip, a_bits, False, experts, s2, ids, 256, 2048)
    lo, _, _, _ = _gemv_gpu(hip, a_bits[:cut], False, experts, s2, ids[:cut], 256, 2048)
    hi, _, _, _ = _gemv_gpu(hip, a_bits[cut:], False, experts, s2, ids[cut:], 256, 2048)
    split = np.concatenate([lo, hi])
    assert np.array_equal(np.isnan(whole), np.isnan(split))
    assert np.array_equal(whole, split)


@pytest.mark.parametrize("rows,a_rows,per_slot", [(6, 4, False), (12, 9, False), (5, 11, True)])
def test_gemv_union_source_rows_past_a_read_zeros(hip, rows, a_rows, per_slot):
    """Through the C ABI (the binding refuses a short ``a``): a source row at or past
    a_rows reads zeros, so its covered outputs are exactly 0 and the others are those of
    the full problem. Six and five rows take the LDS-staged activations, twelve the
    direct loads."""
    import ctypes

    top_k, num_experts, n, k = 4, 10, 64, 512
    rng, ids, experts, s2 = _problem(300 + rows, rows, top_k, num_experts, n, k)
    src_rows = rows * top_k if per_slot else rows
    assert a_rows < src_rows
    a_bits = wl.bf16_normal(rng, (src_rows, k))
    a_bits[a_rows:] = 0  # what the kernel must read past a_rows
    table = upload_table(hip, experts, s2, n, k)
    u_eid, u_slot, _, _ = _union_gpu(hip, ids, num_experts)
    a_dev = bf16_dev(np.ascontiguousarray(a_bits[:a_rows]))
    u_eid_d, u_slot_d = dev(u_eid), dev(u_slot.reshape(-1))
    c = torch.full((rows * top_k, n), -3.0, dtype=torch.bfloat16, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    lib = hip.load()
    rc = lib.moe_w4a16_gemv_union(
        p(a_dev), k, a_rows, int(per_slot), p(table.packed_ptrs), p(table.scale_ptrs),
        p(table.scale2), p(u_eid_d), p(u_slot_d), rows, top_k, num_experts, p(c), n, n, k,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.moe_w4a16_last_error().decode()
    torch.cuda.synchronize()
    got = f64(c)
    ref = _oracle_gemv(a_bits, per_slot, experts, s2, ids, n)
    _check(got, ref, _abs_bound(a_bits, per_slot, experts, s2, ids, n, k))
    srcs = np.array([t if per_slot else t // top_k for t in range(rows * top_k)])
    zero = (srcs >= a_rows) & ~np.isnan(ref[:, 0])
    assert zero.any() and np.all(got[zero] == 0.0)
