"""The device router (moe_router_topk) against the oracle's router_topk.

- Ids: without a bias the selection key is the FP32 logit on both sides, so the ids are
  compared bit for bit. With a bias the key is score + bias (the score needs an exp), so
  ids are compared where the oracle's keys are separated by more than the FP32 error of
  the key; elsewhere the GPU's picks must be valid (their keys within that error of the
  oracle's selected keys).
- Weights: FP32 softmax of the selected logits (or of all, without renormalisation),
  against the FP64 oracle within a relative bound of a few FP32 roundings and one exp.
- Edge cases: equal logits (ties to the lower id), top_k > E, the E and top_k limits, a
  row stride, empty input, bad arguments; the router's output fed to moe_align gives the
  oracle's routing buffers bit for bit.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import moe
from gpu_util import align_buffers, dev

pytestmark = pytest.mark.gpu

W_RTOL = 8e-6  # a few FP32 roundings plus the fast exp's error, relative


def _route(hip, logits, top_k, bias=None, routed_scale=1.0, renormalize=True, ld=None):
    rows, e = logits.shape
    if ld is not None:  # a row stride wider than E
        wide = np.full((rows, ld), np.nan, np.float32)
        wide[:, :e] = logits
        lt = dev(wide)[:, :e]
    else:
        lt = dev(np.ascontiguousarray(logits, np.float32))
    ids = torch.full((max(rows * top_k, 1),), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((max(rows * top_k, 1),), -7.0, dtype=torch.float32, device="cuda")
    hip.moe_router_topk(lt, top_k, ids, wts, None if bias is None else dev(bias.astype(np.float32)),
                        routed_scale, renormalize)
    torch.cuda.synchronize()
    return (ids.cpu().numpy()[:rows * top_k].reshape(rows, top_k),
            wts.cpu().numpy()[:rows * top_k].reshape(rows, top_k).astype(np.float64))


def _check_weights(got, ref):
    assert np.all(np.abs(got - ref) <= W_RTOL * np.abs(ref) + 1e-30), float(
        np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)))


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_router_workload_logits_bit_exact_ids(hip, name):
    w = wl.WORKLOADS[name]
    lg = wl.router_logits(w)
    ids, wts = _route(hip, lg, w.top_k)
    ref_ids, ref_w = moe.router_topk(lg, w.top_k)
    assert np.array_equal(ids, ref_ids)
    _check_weights(wts, ref_w)


@pytest.mark.parametrize("rows,e,k,seed", [(37, 5, 2, 1), (64, 64, 8, 2), (9, 300, 13, 3),
                                           (5, 2048, 64, 4), (3, 1, 1, 5), (50, 2000, 1, 6),
                                           (20, 1000, 8, 7), (11, 512, 6, 8)])
def test_router_shapes_and_limits(hip, rows, e, k, seed):
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((rows, e)) * 3).astype(np.float32)
    ids, wts = _route(hip, lg, k, ld=e + 3 if seed % 2 else None)
    ref_ids, ref_w = moe.router_topk(lg, k)
    assert np.array_equal(ids, ref_ids)
    _check_weights(wts, ref_w)


def test_router_ties_go_to_lower_ids(hip):
    lg = np.zeros((4, 40), np.float32)
    lg[1, 7] = lg[1, 3] = 1.0  # two equal maxima
    lg[2] = np.repeat(np.arange(10, dtype=np.float32), 4)  # groups of four equal logits
    ids, wts = _route(hip, lg, 6, routed_scale=2.5)
    ref_ids, ref_w = moe.router_topk(lg, 6, routed_scale=2.5)
    assert np.array_equal(ids, ref_ids)
    assert ids[0].tolist() == [0, 1, 2, 3, 4, 5] and ids[1][:2].tolist() == [3, 7]
    _check_weights(wts, ref_w)


def test_router_top_k_beyond_experts_pads(hip):
    lg = np.array([[0.5, -1.0, 2.0]] * 3, np.float32)
    ids, wts = _route(hip, lg, 5)
    assert ids.tolist() == [[2, 0, 1, -1, -1]] * 3
    assert np.all(wts[:, 3:] == 0.0)
    _check_weights(wts[:, :3], moe.router_topk(lg, 5)[1][:, :3])


def test_router_no_renormalize_and_scale(hip):
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((20, 96)).astype(np.float32)
    ids, wts = _route(hip, lg, 8, routed_scale=1.75, renormalize=False)
    ref_ids, ref_w = moe.router_topk(lg, 8, routed_scale=1.75, renormalize=False)
    assert np.array_equal(ids, ref_ids)
    _check_weights(wts, ref_w)


def test_router_with_bias(hip):
    rng = np.random.default_rng(9)
    rows, e, k = 64, 256, 8
    lg = rng.standard_normal((rows, e)).astype(np.float32)
    bias = (rng.standard_normal(e) * 0.01).astype(np.float32)  # same order as the scores
    ids, wts = _route(hip, lg, k, bias=bias)
    ref_ids, ref_w = moe.router_topk(lg, k, bias=bias.astype(np.float64))
    # keys score + bias, FP64; the GPU's FP32 keys (fast exp, a division, an add) are
    # within ~2e-6 of the row's largest |key|
    z = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    key = z / z.sum(axis=1, keepdims=True) + bias.astype(np.float64)[None, :]
    tol = 2e-6 * np.abs(key).max(axis=1)
    compared = 0
    for r in range(rows):
        ks = np.sort(key[r])[::-1]
        gaps = -np.diff(ks[:k + 1])
        if np.all(gaps > 2 * tol[r]):  # unambiguous: every pick and the cut-off
            assert ids[r].tolist() == ref_ids[r].tolist(), r
            _check_weights(wts[r], ref_w[r])
            compared += 1
        else:  # several valid answers: the GPU's picks must be near-maximal and distinct
            assert len(set(ids[r].tolist())) == k
            assert np.all(np.abs(key[r][ids[r]] - ks[:k]) <= 2 * tol[r])
    assert compared >= rows // 2


def test_router_feeds_align(hip):
    w = wl.WORKLOADS["layer_e64"]
    lg = wl.router_logits(w)
    lt = dev(lg)
    s = w.rows * w.top_k
    ids = torch.empty(s, dtype=torch.int32, device="cuda")
    wts = torch.empty(s, dtype=torch.float32, device="cuda")
    hip.moe_router_topk(lt, w.top_k, ids, wts)
    b = align_buffers(w.rows, w.top_k, w.num_experts)
    hip.moe_align(ids.view(w.rows, w.top_k), w.num_experts, b["sorted_token_ids"],
                  b["sorted_expert_ids"], b["expert_offsets"], b["token_to_perm"])
    torch.cuda.synchronize()
    al = moe.align(moe.router_topk(lg, w.top_k)[0], w.num_experts)
    assert np.array_equal(b["expert_offsets"].cpu().numpy(), al["expert_offsets"])
    assert np.array_equal(b["sorted_token_ids"].cpu().numpy(), al["sorted_token_ids"])
    assert np.array_equal(b["token_to_perm"].cpu().numpy(), al["token_to_perm"].reshape(-1))


def test_router_empty_and_bad_arguments(hip):
    ids = torch.empty(256, dtype=torch.int32, device="cuda")
    wts = torch.empty(256, dtype=torch.float32, device="cuda")
    hip.moe_router_topk(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 4, ids, wts)
    lt = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    for top_k, scale in ((0, 1.0), (65, 1.0), (4, float("inf"))):
        with pytest.raises(hip.MoeError):
            hip.moe_router_topk(lt, top_k, ids, wts, routed_scale=scale)
    big = torch.zeros((1, 2049), dtype=torch.float32, device="cuda")
    with pytest.raises(hip.MoeError):
        hip.moe_router_topk(big, 2, ids, wts)
