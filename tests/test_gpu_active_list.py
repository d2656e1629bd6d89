"""The grouped GEMMs given moe_align's active-expert list (a launch with fewer rows than
experts visits only the listed experts) against the same GEMMs without it: the same bits,
element for element, in the gate_up, fused gate_up + SwiGLU and down forms, with null
experts, invalid ids, an expert whose rows run into overflow chunks, one row, and a list
that is shuffled and padded with out-of-range entries. Untouched rows keep their poison
on both sides. The unlisted GEMMs are held to the oracle in test_gpu_gemm.py, and the
routed layer at 8 rows and 256 experts (which takes the list) in test_gpu_layer.py.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import align_buffers, bf16_dev, workload_tables

pytestmark = pytest.mark.gpu

E = 256


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _align(hip, ids_np):
    rows, top_k = ids_np.shape
    b = align_buffers(rows, top_k, E)
    hip.moe_align(torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).cuda(), E,
                  b["sorted_token_ids"], b["sorted_expert_ids"], b["expert_offsets"],
                  b["token_to_perm"], b["active_experts"], b["counters"])
    return b


def _gemms(hip, w, b, active=None, counters=None, max_rows=None):
    """(gate_up, act, down output) bits of the three grouped GEMM forms over sorted rows
    (the first ``max_rows`` of them; all by default)."""
    _, _, gt, dt = _tables(hip, w)
    s = w.rows * w.top_k
    cut = s if max_rows is None else max_rows
    mi, hidden = w.moe_intermediate, w.hidden
    kw = dict(active_experts=active, counters=counters)
    x = bf16_dev(wl.activations(w))
    bf16 = dict(dtype=torch.bfloat16, device="cuda")
    gu = torch.full((s, 2 * mi), -3.0, **bf16)
    hip.moe_w4a16_grouped_gemm(x, gt, b["expert_offsets"], gu, b["sorted_token_ids"],
                               max_rows=cut, **kw)
    act = torch.full((s, mi), -3.0, **bf16)
    hip.moe_w4a16_grouped_gemm_swiglu(x, gt, b["expert_offsets"], act, w.limit,
                                      b["sorted_token_ids"], max_rows=cut, **kw)
    out = torch.full((s, hidden), -3.0, **bf16)
    hip.moe_w4a16_grouped_gemm(act, dt, b["expert_offsets"], out, None, max_rows=cut, **kw)
    torch.cuda.synchronize()
    return _bits(gu), _bits(act), _bits(out)


_LIVE = {}


def _tables(hip, w):
    return workload_tables(hip, w, only=_LIVE[w.name])


def _workload(name, seed, rows, top_k, ids_np=None):
    w = wl.custom(name, seed, rows=rows, num_experts=E, top_k=top_k, hidden=1024,
                  moe_intermediate=512, null_from=200)
    if ids_np is None:
        ids_np, _ = wl.routing(w)
    _LIVE[name] = {int(e) for e in ids_np.reshape(-1) if 0 <= e < E and not w.is_null(int(e))}
    return w, ids_np


def _heavy_ids(rows, top_k, seed):
    """Every row routes to expert 3 (its rows run past one 64-row block: overflow
    chunks); the other choices are distinct per row, some null (>= 200), some invalid."""
    rng = np.random.default_rng(seed)
    ids = np.empty((rows, top_k), np.int32)
    for r in range(rows):
        ids[r] = np.concatenate([[3], rng.choice(np.arange(4, E), top_k - 1, replace=False)])
    ids[rng.random((rows, top_k)) < 0.05] = -1
    ids[rng.random((rows, top_k)) < 0.05] = E + 44
    return ids


CASES = [
    ("act_softmax_8", 8, 8, None),   # 64 slots, ~60 experts of 256
    ("act_one_row", 1, 8, None),
    ("act_heavy_100x2", 100, 2, "heavy"),  # 200 slots; expert 3 has ~95 rows
    ("act_31x8", 31, 8, None),       # 248 slots: just under the expert count
]


@pytest.mark.parametrize("name,rows,top_k,ids", CASES)
def test_listed_launch_has_the_same_bits(hip, name, rows, top_k, ids):
    ids_np = _heavy_ids(rows, top_k, 5) if ids == "heavy" else None
    w, ids_np = _workload(name, 70 + rows, rows, top_k, ids_np)
    b = _align(hip, ids_np)
    n_active = int(b["counters"][0])
    assert 0 < n_active <= rows * top_k < E
    ref = _gemms(hip, w, b)
    got = _gemms(hip, w, b, b["active_experts"], b["counters"])
    for r, g in zip(ref, got):
        assert np.array_equal(g, r)
    # the rows of live experts were written (not all poison)
    off = b["expert_offsets"].cpu().numpy()
    live_rows = sum(int(off[e + 1] - off[e]) for e in _LIVE[name])
    assert live_rows > 0 and (got[2] != _bits(torch.tensor(-3.0, dtype=torch.bfloat16))).any()


def test_shuffled_list_with_out_of_range_entries(hip):
    """The list's order does not matter and entries outside [0, E) are skipped."""
    w, ids_np = _workload("act_softmax_8", 78, 8, 8)
    b = _align(hip, ids_np)
    n_active = int(b["counters"][0])
    listed = b["active_experts"][:n_active].cpu().numpy()
    rng = np.random.default_rng(3)
    pad = [-1, E, E + 1000, -70000][:max(0, w.rows * w.top_k - n_active)]
    mixed = np.concatenate([rng.permutation(listed), pad]).astype(np.int32)
    mixed = rng.permutation(mixed).astype(np.int32)
    active = torch.full((E,), -9, dtype=torch.int32, device="cuda")
    active[:mixed.size] = torch.from_numpy(mixed).cuda()
    counters = torch.tensor([mixed.size, 0], dtype=torch.int32, device="cuda")
    ref = _gemms(hip, w, b)
    got = _gemms(hip, w, b, active, counters)
    for r, g in zip(ref, got):
        assert np.array_equal(g, r)


def test_row_cut_off_below_the_list_length(hip):
    """max_rows = 35 of 64 sorted rows with ~56 listed experts: the grid's 35 expert rows
    take the first 35 entries; the experts past them start at row 35 or later."""
    w, ids_np = _workload("act_softmax_8", 78, 8, 8)
    b = _align(hip, ids_np)
    assert int(b["counters"][0]) > 35
    ref = _gemms(hip, w, b, max_rows=35)
    got = _gemms(hip, w, b, b["active_experts"], b["counters"], max_rows=35)
    poison = _bits(torch.tensor(-3.0, dtype=torch.bfloat16))
    for r, g in zip(ref, got):
        assert np.array_equal(g, r)
        assert (g[35:] == poison).all()


def test_no_valid_ids_writes_nothing(hip):
    """Every id invalid: the list is empty, every block exits, both sides keep the poison."""
    w, ids_np = _workload("act_none", 79, 4, 8, np.full((4, 8), -1, np.int32))
    b = _align(hip, ids_np)
    assert int(b["counters"][0]) == 0
    got = _gemms(hip, w, b, b["active_experts"], b["counters"])
    poison = _bits(torch.tensor(-3.0, dtype=torch.bfloat16))
    for g in got:
        assert (g == poison).all()


def test_list_arguments_go_together(hip):
    w, ids_np = _workload("act_one_row", 71, 1, 8)
    b = _align(hip, ids_np)
    with pytest.raises(ValueError):
        _gemms(hip, w, b, b["active_experts"], None)
    with pytest.raises(ValueError):
        _gemms(hip, w, b, b["active_experts"][:E - 1], b["counters"])
