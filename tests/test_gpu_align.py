"""moe_align on the GPU against the oracle's counting sort: bit-exact on every output."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import moe
from gpu_util import align_buffers, dev

pytestmark = pytest.mark.gpu


def _run(hip, ids: np.ndarray, num_experts: int):
    rows, top_k = ids.shape
    b = align_buffers(rows, top_k, num_experts)
    hip.moe_align(dev(ids.astype(np.int32)), num_experts, **b)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in b.items()}


def _check(got, ids, num_experts):
    ref = moe.align(ids, num_experts)
    s = ids.size
    assert np.array_equal(got["expert_offsets"], ref["expert_offsets"])
    if s:
        assert np.array_equal(got["sorted_token_ids"][:s], ref["sorted_token_ids"])
        assert np.array_equal(got["sorted_expert_ids"][:s], ref["sorted_expert_ids"])
        assert np.array_equal(got["token_to_perm"][:s], ref["token_to_perm"].reshape(-1))
    counts = np.diff(ref["expert_offsets"])
    active = np.nonzero(counts)[0]
    assert np.array_equal(got["active_experts"][:active.size], active)
    assert np.all(got["active_experts"][active.size:] == -1)
    assert got["counters"].tolist() == [active.size, ref["n_invalid"]]


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_align_workload_routing(hip, name):
    w = wl.WORKLOADS[name]
    ids, _ = wl.routing(w)
    for c in range(w.n_chunks):
        chunk = ids[c * w.chunk:(c + 1) * w.chunk]
        _check(_run(hip, chunk, w.num_experts), chunk, w.num_experts)
    if w.n_chunks > 1:  # the whole long prefill in one call as well
        _check(_run(hip, ids, w.num_experts), ids, w.num_experts)


@pytest.mark.parametrize("rows,top_k,num_experts,bad,seed", [
    (1, 1, 1, 0.0, 0), (3, 2, 5, 0.3, 1), (37, 3, 5, 0.1, 2), (64, 8, 16, 0.0, 3),
    (200, 6, 300, 0.05, 4), (16, 8, 256, 0.2, 5), (1000, 8, 2048, 0.01, 6),
    (4097, 8, 256, 0.0, 7), (513, 4, 1025, 0.02, 8), (129, 8, 7, 0.5, 9),
    # at most 64 slots (the one-wave kernel): decode-sized batches, one row of 64, one
    # slot, a single expert, the largest expert count, mostly invalid ids
    (8, 8, 256, 0.1, 10), (1, 64, 300, 0.0, 11), (64, 1, 2048, 0.2, 12), (1, 1, 2048, 0.0, 13),
    (5, 7, 1, 0.0, 14), (2, 3, 2000, 0.5, 15), (9, 7, 64, 0.0, 16)])
def test_align_random_with_invalid_ids(hip, rows, top_k, num_experts, bad, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, num_experts, size=(rows, top_k)).astype(np.int32)  # repeats allowed
    mask = rng.random(ids.shape) < bad
    ids[mask] = rng.choice([-1, num_experts, num_experts + 9, -100], size=int(mask.sum()))
    _check(_run(hip, ids, num_experts), ids, num_experts)


def test_align_all_slots_one_expert_and_all_invalid(hip):
    ids = np.full((300, 8), 5, np.int32)
    _check(_run(hip, ids, 64), ids, 64)
    bad = np.full((10, 4), -1, np.int32)
    got = _run(hip, bad, 16)
    _check(got, bad, 16)
    assert np.all(got["sorted_token_ids"] == -1) and got["counters"][1] == 40
    # the same past 64 slots (the 1024-thread form): every id invalid, and one expert only
    bad = np.full((300, 8), 64, np.int32)
    got = _run(hip, bad, 64)
    _check(got, bad, 64)
    assert np.all(got["sorted_token_ids"] == -1) and got["counters"].tolist() == [0, 2400]
    one = np.zeros((100, 8), np.int32)
    got = _run(hip, one, 1)
    _check(got, one, 1)
    assert got["expert_offsets"].tolist() == [0, 800]


def test_align_empty_input(hip):
    ids = np.zeros((0, 8), np.int32)
    b = align_buffers(0, 8, 32)
    hip.moe_align(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 32, **b)
    torch.cuda.synchronize()
    assert np.all(b["expert_offsets"].cpu().numpy() == 0)
    assert b["counters"].cpu().tolist() == [0, 0]
    assert np.all(b["active_experts"].cpu().numpy() == -1)
    del ids


def test_align_is_deterministic(hip):
    ids, _ = wl.routing(wl.WORKLOADS["long_prefill"])
    a = _run(hip, ids, 256)
    for _ in range(3):
        b = _run(hip, ids, 256)
        for k in a:
            assert np.array_equal(a[k], b[k])


def test_align_rejects_bad_arguments(hip):
    b = align_buffers(4, 2, 8)
    ids = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(hip.MoeError):
        hip.moe_align(ids, 0, **b)
    with pytest.raises(hip.MoeError):
        hip.moe_align(ids, 4096, **{**b, "expert_offsets": torch.zeros(4097, dtype=torch.int32,
                                                                        device="cuda"),
                                    "active_experts": None})


@pytest.mark.parametrize("rows,top_k,num_experts,cols,ld,seed", [
    (8, 8, 256, 6144, 6144, 30),    # the one-wave form over the small-M expert_out
    (256, 8, 256, 2048, 2056, 31),  # the block form, a padded leading dimension
    (3, 2, 5, 8, 16, 32),           # tiny
    (37, 3, 5, 0, 8, 33)])          # no columns: moe_align alone
def test_align_zero(hip, rows, top_k, num_experts, cols, ld, seed):
    """moe_align_zero: the sort's outputs as moe_align's (bit-exact against the oracle), and
    exactly rows [0, rows * top_k) x columns [0, cols) of the buffer zeroed: the padding
    columns and the rows past them keep their values."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, num_experts, size=(rows, top_k)).astype(np.int32)
    ids[rng.random(ids.shape) < 0.1] = -1
    s = rows * top_k
    b = align_buffers(rows, top_k, num_experts)
    buf = torch.full((s + 3, ld), 7.0, dtype=torch.bfloat16, device="cuda")
    hip.moe_align(dev(ids), num_experts, **b, zero=buf[:s, :cols])
    torch.cuda.synchronize()
    _check({k: v.cpu().numpy() for k, v in b.items()}, ids, num_experts)
    host = buf.float().cpu().numpy()
    assert np.all(host[:s, :cols] == 0.0)
    assert np.all(host[:s, cols:] == 7.0) and np.all(host[s:] == 7.0)
