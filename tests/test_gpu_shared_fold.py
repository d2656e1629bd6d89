"""The shared expert's down projection reduced inside the combine (moe_dense_gemm_bf16_partials
+ moe_combine_partials) against the two-step path it replaces (moe_dense_gemm_bf16 in its
split-K form, then moe_combine with the BF16 shared term): the same bits, element for
element, at the prefill sub-chunk's size, with ragged rows, one, two and four K splits, the
top-8 and the generic combine kernels and excluded slots; the routed layer with a
SharedExpert gives the bits of the layer with the shared expert's BF16 output passed in;
bad arguments raise. The two-step path itself is held to the oracle in test_gpu_dense.py,
so these comparisons tie the folded path to the oracle too.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import bf16_dev, workload_tables

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _routed(seed, rows, top_k, hidden, excluded=0.1):
    """expert_out rows, token_to_perm (a permutation of the slots, some excluded) and
    weights, as a sorted layer would hand them to the combine."""
    rng = np.random.default_rng(seed)
    s = rows * top_k
    eo = bf16_dev(wl.bf16_normal(rng, (s, hidden)))
    ttp = rng.permutation(s).astype(np.int32)
    ttp[rng.random(s) < excluded] = -1
    wts = rng.random((rows, top_k)).astype(np.float32)
    return eo, torch.from_numpy(ttp).cuda(), torch.from_numpy(wts).cuda()


@pytest.mark.parametrize("rows,hidden,inter,top_k,ways", [
    (256, 6144, 2048, 8, 2),   # the prefill sub-chunk's shared expert
    (200, 1024, 512, 8, 1),    # ragged rows; K too short to split
    (130, 512, 4096, 6, 4),    # two row tiles, four splits, the generic combine kernel
    (384, 2048, 4096, 8, 2),   # three row tiles
    (520, 8192, 512, 8, 1)])   # 320 blocks: the register-staged kernel's row-major stores
def test_combine_partials_bits(hip, rows, hidden, inter, top_k, ways):
    rng = np.random.default_rng(rows + hidden)
    act = bf16_dev(wl.bf16_normal(rng, (rows, inter)))
    down = bf16_dev(wl.bf16_normal_scaled(rng, (hidden, inter), inter ** -0.5))
    eo, ttp, wts = _routed(rows, rows, top_k, hidden)
    assert hip.moe_dense_splitk_ways(rows, inter) == ways

    # the two-step path: the split-K down projection to BF16, then the combine
    ws = hip.dense_workspace(rows, hidden, inter)
    shared = torch.empty(rows, hidden, dtype=torch.bfloat16, device="cuda")
    hip.moe_dense_gemm_bf16(act, down, shared, workspace=ws)
    ref = torch.empty(rows, hidden, dtype=torch.bfloat16, device="cuda")
    hip.moe_combine(eo, ttp, wts, ref, shared)

    # folded: partials (poisoned first: every element must be written), then the combine
    buf = torch.full((ways * rows * hidden + 64,), float("nan"), dtype=torch.float32,
                     device="cuda")
    sp = hip.moe_dense_gemm_bf16_partials(act, down, buf)
    assert tuple(sp.partials.shape) == (ways, rows, hidden) and sp.ways == ways
    out = torch.full((rows, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    hip.moe_combine(eo, ttp, wts, out, sp)
    torch.cuda.synchronize()
    assert torch.isfinite(sp.partials).all()
    assert np.isnan(buf[ways * rows * hidden:].cpu().numpy()).all()  # nothing past the end
    assert np.array_equal(_bits(out), _bits(ref))
    # the partials' split-order FP32 sum, rounded to BF16, is the dense GEMM's output
    s = sp.partials[0].clone()
    for w in range(1, ways):
        s += sp.partials[w]
    assert np.array_equal(_bits(s.to(torch.bfloat16)), _bits(shared))


def test_layer_with_shared_expert_folds_with_the_same_bits(hip):
    """moe_layer with a SharedExpert (its down reduction inside the combine) against
    moe_layer with that shared expert's BF16 output passed in."""
    w = wl.custom("fold_layer", 93, rows=256, num_experts=32, top_k=8, hidden=1024,
                  moe_intermediate=512)
    _, _, gt, dt = workload_tables(hip, w)
    g, u, d = wl.shared_expert(w, 1.0)
    se = hip.SharedExpert(bf16_dev(g), bf16_dev(u), bf16_dev(d), w.rows)
    x = bf16_dev(wl.activations(w))
    ids, wts = wl.routing(w)
    ids, wts = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    ws = hip.Workspace(w.rows, w.top_k, w.num_experts, w.hidden, w.moe_intermediate)
    shared = se(x, w.limit).clone()
    assert isinstance(se.for_combine(x, w.limit), hip.SharedPartials)
    ref = torch.empty(w.rows, w.hidden, dtype=torch.bfloat16, device="cuda")
    hip.moe_layer(x, ids, wts, gt, dt, w.moe_intermediate, w.limit, ws, ref, shared=shared)
    out = torch.empty_like(ref)
    hip.moe_layer(x, ids, wts, gt, dt, w.moe_intermediate, w.limit, ws, out, shared=se)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))
    # below the split-K row count the shared expert hands over its BF16 output
    assert isinstance(se.for_combine(x[:64], w.limit), torch.Tensor)


def test_partials_bad_arguments(hip):
    act = torch.zeros(256, 512, dtype=torch.bfloat16, device="cuda")
    down = torch.zeros(1024, 512, dtype=torch.bfloat16, device="cuda")
    ways = hip.moe_dense_splitk_ways(256, 512)
    small = torch.zeros(ways * 256 * 1024 - 4, dtype=torch.float32, device="cuda")
    with pytest.raises(hip.MoeError) as e:  # MOE_ECAPACITY: the partials do not fit
        hip.moe_dense_gemm_bf16_partials(act, down, small)
    assert e.value.status == 2
    big = torch.zeros(ways * 256 * 1024 + 8, dtype=torch.float32, device="cuda")
    with pytest.raises(hip.MoeError):  # not 16-byte aligned
        hip.moe_dense_gemm_bf16_partials(act, down, big[1:])
    eo, ttp, wts = _routed(5, 4, 8, 1024)
    out = torch.empty(4, 1024, dtype=torch.bfloat16, device="cuda")
    lib = hip.load()
    p = torch.zeros(4 * 1024, dtype=torch.float32, device="cuda")
    nbytes = p.numel() * 4
    for bad_ways in (0, 65):
        rc = lib.moe_combine_partials(eo.data_ptr(), 1024, 32, ttp.data_ptr(), wts.data_ptr(),
                                      p.data_ptr(), bad_ways, nbytes, out.data_ptr(), 1024, 4,
                                      1024, 8, None)
        assert rc == 1  # MOE_EINVAL
    rc = lib.moe_combine_partials(eo.data_ptr(), 1024, 32, ttp.data_ptr(), wts.data_ptr(),
                                  None, 1, nbytes, out.data_ptr(), 1024, 4, 1024, 8, None)
    assert rc == 1
    # two splits of 4 x 1024 do not fit one's bytes: MOE_ECAPACITY, nothing read
    rc = lib.moe_combine_partials(eo.data_ptr(), 1024, 32, ttp.data_ptr(), wts.data_ptr(),
                                  p.data_ptr(), 2, nbytes, out.data_ptr(), 1024, 4, 1024, 8, None)
    assert rc == 2
    with pytest.raises(ValueError):  # partials of another row count
        hip.moe_combine(eo, ttp, wts, out, hip.SharedPartials(p.view(1, 2, 2048)))
