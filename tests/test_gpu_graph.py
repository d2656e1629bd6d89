"""The layer calls under HIP graph capture.

The library's calls only enqueue kernels on the caller's stream (no allocation, no host
synchronisation, no memset nodes: the zero-first step is a kernel), so a whole layer can
be captured once and replayed. Each replay is checked bit for bit against an eager run on
the same inputs, with new inputs copied into the captured tensors between replays and
eager library work and synchronisations in between (a replay that reused stale state, or
a node that only worked on the first replay, would show).
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import bf16_bits_host, bf16_dev, dev, workload_tables

pytestmark = pytest.mark.gpu


def _inputs(w, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(w.num_experts)[:w.top_k] for _ in range(w.rows)])
    wts = rng.random((w.rows, w.top_k)).astype(np.float32)
    return ids.astype(np.int32), wts, wl.bf16_normal(rng, (w.rows, w.hidden))


def _replays_match_eager(run, static, input_sets, out):
    """Capture ``run`` once, then for each input set: copy it into ``static``, replay,
    compare with an eager ``run`` on the same inputs; eager work between replays."""
    # warm up eagerly (first-call set-up happens outside the capture)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    results = []
    for inputs in input_sets:
        for t, v in zip(static, inputs):
            t.copy_(v)
        graph.replay()
        torch.cuda.synchronize()
        got = bf16_bits_host(out).copy()
        run()  # eager on the same inputs
        torch.cuda.synchronize()
        assert np.array_equal(got, bf16_bits_host(out))
        results.append(got)
    # the input sets differ, so do their outputs (a replay that redid nothing would fail)
    assert not np.array_equal(results[0], results[1])
    assert np.array_equal(results[0], results[2])


def test_layer_graph_replays(hip):
    """moe_layer with null experts (the zero-first kernel runs) and the split-K shared
    expert (two launches per GEMM) in its combine."""
    w = wl.custom("graph_layer", 91, rows=256, num_experts=32, top_k=4, hidden=1024,
                  moe_intermediate=512, null_from=24)
    gu, dn, gt, dt = workload_tables(hip, w)
    g, u, d = wl.shared_expert(w, 1.0)
    se = hip.SharedExpert(bf16_dev(g), bf16_dev(u), bf16_dev(d), w.rows)
    assert se.workspace is not None
    sets = [_inputs(w, s) for s in (1, 2, 1)]
    ids = dev(sets[0][0])
    wts = dev(sets[0][1])
    x = bf16_dev(sets[0][2])
    ws = hip.Workspace(w.rows, w.top_k, w.num_experts, w.hidden, w.moe_intermediate)
    out = torch.empty((w.rows, w.hidden), dtype=torch.bfloat16, device="cuda")

    def run():
        hip.moe_layer(x, ids, wts, gt, dt, w.moe_intermediate, w.limit, ws, out, shared=se)

    sets_dev = [(dev(i), dev(t), bf16_dev(xb)) for i, t, xb in sets]
    _replays_match_eager(run, (ids, wts, x), sets_dev, out)


def test_decode_layer_graph_replays(hip):
    """moe_layer_decode (row union, union GEMVs, combine) for 8 rows, half the experts
    absent."""
    w = wl.custom("graph_decode", 92, rows=8, num_experts=32, top_k=4, hidden=1024,
                  moe_intermediate=512, null_from=16)
    gu, dn, gt, dt = workload_tables(hip, w)
    sets = [_inputs(w, s) for s in (3, 4, 3)]
    ids = dev(sets[0][0])
    wts = dev(sets[0][1])
    x = bf16_dev(sets[0][2])
    dws = hip.DecodeWorkspace(w.rows, w.top_k, w.hidden, w.moe_intermediate)
    out = torch.empty((w.rows, w.hidden), dtype=torch.bfloat16, device="cuda")

    def run():
        hip.moe_layer_decode(x, ids, wts, gt, dt, w.moe_intermediate, w.limit, dws, out)

    sets_dev = [(dev(i), dev(t), bf16_dev(xb)) for i, t, xb in sets]
    _replays_match_eager(run, (ids, wts, x), sets_dev, out)


def test_layer_with_active_expert_list_graph_replays(hip):
    """moe_layer at 8 rows and 256 experts: the grouped GEMMs' grids hold one expert row
    per slot and take the experts from the sort's list on the device, so replays with
    other routing (another set of experts with rows) must follow it."""
    w = wl.custom("graph_listed", 94, rows=8, num_experts=256, top_k=8, hidden=1024,
                  moe_intermediate=512, null_from=160)
    sets = [_inputs(w, s) for s in (4, 5, 4)]
    live = {int(e) for s in sets for e in s[0].reshape(-1)}
    assert not live <= set(sets[0][0].reshape(-1).tolist())  # the sets route differently
    _, _, gt, dt = workload_tables(hip, w, only=live)
    ids = dev(sets[0][0])
    wts = dev(sets[0][1])
    x = bf16_dev(sets[0][2])
    ws = hip.Workspace(w.rows, w.top_k, w.num_experts, w.hidden, w.moe_intermediate)
    out = torch.empty((w.rows, w.hidden), dtype=torch.bfloat16, device="cuda")

    def run():
        hip.moe_layer(x, ids, wts, gt, dt, w.moe_intermediate, w.limit, ws, out)

    sets_dev = [(dev(i), dev(t), bf16_dev(xb)) for i, t, xb in sets]
    _replays_match_eager(run, (ids, wts, x), sets_dev, out)
