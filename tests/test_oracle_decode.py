"""Pins for the oracle's decode / verify path: row_union, union_gemv, moe_layer_decode.

The union table is checked against a hand-worked example and against a second
construction (numpy's unique with first indices); the union GEMV against exact rational
brute force; the layer against the per-token brute force of test_oracle_moe and against
the sorted (grouped) layer, which must give each covered slot the same value.
"""

import numpy as np
import pytest

from oracle import codecs, moe
import workloads as wl

from test_oracle_moe import _brute_layer, _exact_weight, _tiny_problem
from fractions import Fraction
import torch


# --------------------------------------------------------------------------- row_union

def test_row_union_hand_example():
    # rows: (3, 1), (1, 5), (unfilled, 3); E = 6. First appearances in flat order: 3, 1, 5.
    ids = np.array([[3, 1], [1, 5], [-1, 3]], dtype=np.int32)
    u = moe.row_union(ids, 6)
    assert u["u_eid"].tolist() == [3, 1, 5, -1, -1, -1]
    # entry 0 (expert 3): row 0 slot 0, row 2 slot 1; entry 1 (expert 1): row 0 slot 1,
    # row 1 slot 0; entry 2 (expert 5): row 1 slot 1.
    assert u["u_slot"].tolist() == [[0, -1, 1], [1, 0, -1], [-1, 1, -1],
                                    [-1, -1, -1], [-1, -1, -1], [-1, -1, -1]]
    assert u["slot_perm"].tolist() == [[0, 1], [2, 3], [-1, 5]]
    assert u["n_union"] == 3 and u["n_uncovered"] == 1


def test_row_union_present_mask_hand_example():
    # as above with expert 1 absent: its slots are not covered and open no entry
    ids = np.array([[3, 1], [1, 5], [-1, 3]], dtype=np.int32)
    present = np.array([True, False, True, True, True, True])
    u = moe.row_union(ids, 6, present)
    assert u["u_eid"].tolist() == [3, 5, -1, -1, -1, -1]
    assert u["u_slot"].tolist() == [[0, -1, 1], [-1, 1, -1], [-1, -1, -1],
                                    [-1, -1, -1], [-1, -1, -1], [-1, -1, -1]]
    assert u["slot_perm"].tolist() == [[0, -1], [-1, 3], [-1, 5]]
    assert u["n_union"] == 2 and u["n_uncovered"] == 3


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_row_union_absent_expert_is_an_invalid_id(seed):
    rng = np.random.default_rng(seed)
    e_n = 24
    ids = rng.integers(-1, e_n, size=(8, 6)).astype(np.int32)
    ids[2] = ids[1]
    present = rng.random(e_n) < 0.5
    masked = np.where((ids >= 0) & present[np.clip(ids, 0, e_n - 1)], ids, -1).astype(np.int32)
    a, b = moe.row_union(ids, e_n, present), moe.row_union(masked, e_n)
    for key in ("u_eid", "u_slot", "slot_perm", "n_union", "n_uncovered"):
        assert np.array_equal(a[key], b[key]), key


def _union_by_unique(ids, num_experts):
    """Second construction: dedupe each row, then numpy's unique with first indices."""
    rows, top_k = ids.shape
    cover = np.zeros(ids.shape, bool)
    for r in range(rows):
        seen = set()
        for j in range(top_k):
            e = int(ids[r, j])
            if 0 <= e < num_experts and e not in seen:
                cover[r, j] = True
                seen.add(e)
    flat = np.where(cover.reshape(-1), ids.reshape(-1), -1)
    vals, first = np.unique(flat[flat >= 0], return_index=True)
    pos_of_valid = np.flatnonzero(flat >= 0)
    order = np.argsort(pos_of_valid[first], kind="stable")
    u_eid = np.full(rows * top_k, -1)
    u_eid[:vals.size] = vals[order]
    u_slot = np.full((rows * top_k, rows), -1)
    for p, e in enumerate(vals[order]):
        for r in range(rows):
            hit = np.flatnonzero(cover[r] & (ids[r] == e))
            if hit.size:
                u_slot[p, r] = hit[0]
    perm = np.where(cover, np.arange(rows * top_k).reshape(rows, top_k), -1)
    return u_eid, u_slot, perm


@pytest.mark.parametrize("rows,top_k,num_experts,seed", [(1, 8, 256, 0), (8, 8, 256, 1),
                                                         (8, 8, 16, 2), (3, 4, 5, 3),
                                                         (16, 8, 64, 4), (2, 1, 3, 5)])
def test_row_union_matches_unique_first_index(rows, top_k, num_experts, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, num_experts + 2, size=(rows, top_k)).astype(np.int32)
    if rows > 1:
        ids[1, :] = ids[0, ::-1]  # shared experts across rows
    if top_k > 2:
        ids[0, 2] = ids[0, 1]  # a repeat inside a row
    u = moe.row_union(ids, num_experts)
    u_eid, u_slot, perm = _union_by_unique(ids, num_experts)
    assert np.array_equal(u["u_eid"], u_eid)
    assert np.array_equal(u["u_slot"], u_slot)
    assert np.array_equal(u["slot_perm"], perm)


def test_row_union_invariants_on_softmax_routing():
    w = wl.WORKLOADS["small_m"]
    ids, _ = wl.routing(w)
    u = moe.row_union(ids, w.num_experts)
    n = u["n_union"]
    assert n == np.unique(ids).size  # proper top-k: every slot covered, ids distinct per row
    assert np.all(u["u_eid"][n:] == -1) and np.unique(u["u_eid"][:n]).size == n
    covered = 0
    for p in range(n):
        for r in range(ids.shape[0]):
            j = u["u_slot"][p, r]
            if j >= 0:
                assert ids[r, j] == u["u_eid"][p]
                covered += 1
    assert covered == ids.size and u["n_uncovered"] == 0


# --------------------------------------------------------------------------- union_gemv

@pytest.mark.parametrize("mode", ["exact", "bf16w"])
@pytest.mark.parametrize("per_slot", [False, True])
def test_union_gemv_brute_force_exact_rationals(mode, per_slot):
    ids, x_bits, experts, s2 = _tiny_problem(23, rows=4, top_k=2, null=(2,))
    ids[3, 0] = -1
    rows, top_k = ids.shape
    n, k = 16, 32
    rng = np.random.default_rng(5)
    a_bits = wl.bf16_normal(rng, (rows * top_k, k)) if per_slot else x_bits
    a = codecs.bf16_bits_to_f64(a_bits)
    u = moe.row_union(ids, len(experts))
    out = np.full((rows * top_k, n), -7.0)
    moe.union_gemv(a, per_slot, experts, s2, u["u_eid"], u["u_slot"], top_k, out, mode)
    at = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    for r in range(rows):
        for j in range(top_k):
            t = r * top_k + j
            e = int(ids[r, j])
            if e < 0 or experts[e] is None:
                assert np.all(out[t] == -7.0)  # uncovered or remote: row untouched
                continue
            packed, scales = experts[e]
            src = t if per_slot else r
            for nn in range(n):
                acc = sum(Fraction(float(at[src, kk])) *
                          _exact_weight(packed, scales, s2[e], nn, kk, mode == "bf16w")
                          for kk in range(k))
                assert out[t, nn] == pytest.approx(float(acc), rel=1e-13, abs=1e-13)


def test_union_gemv_equals_grouped_gemm_per_slot():
    rng = np.random.default_rng(7)
    rows, top_k, num_experts, n, k = 8, 8, 32, 48, 64
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    experts = [None if e % 7 == 3 else wl.random_nvfp4(rng, n, k) for e in range(num_experts)]
    s2 = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    x = codecs.bf16_bits_to_f64(wl.bf16_normal(rng, (rows, k)))
    u = moe.row_union(ids, num_experts)
    got = np.full((rows * top_k, n), np.nan)
    moe.union_gemv(x, False, experts, s2, u["u_eid"], u["u_slot"], top_k, got, "bf16w")
    al = moe.align(ids, num_experts)
    ref = np.full((rows * top_k, n), np.nan)
    moe.grouped_gemm(x, al["sorted_token_ids"], experts, s2, al["expert_offsets"], ref, "bf16w")
    ttp = al["token_to_perm"].reshape(-1)
    np.testing.assert_allclose(got, ref[ttp], rtol=1e-12, atol=1e-12, equal_nan=True)


# --------------------------------------------------------------------------- layer

def _layer_problem(seed, rows, top_k, num_experts, hidden, mi, null=()):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(num_experts)[:top_k] for _ in range(rows)]).astype(np.int32)
    wts = rng.random((rows, top_k)).astype(np.float32)
    x_bits = wl.bf16_normal(rng, (rows, hidden))
    gate_up = [None if e in null else wl.random_nvfp4(rng, 2 * mi, hidden)
               for e in range(num_experts)]
    down = [None if e in null else wl.random_nvfp4(rng, hidden, mi) for e in range(num_experts)]
    s2gu = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    s2dn = rng.uniform(0.5, 2, num_experts).astype(np.float32)
    return ids, wts, x_bits, gate_up, down, s2gu, s2dn


@pytest.mark.parametrize("mode", ["exact", "bf16w"])
def test_decode_layer_brute_force(mode):
    ids, wts, x_bits, gu, dn, s2gu, s2dn = _layer_problem(33, 3, 2, 4, 32, 16, null=(1,))
    ids[2, 1] = -1
    got, _ = moe.moe_layer_decode(codecs.bf16_bits_to_f64(x_bits), ids, wts, gu, dn, s2gu, s2dn,
                                  16, 7.0, mode)
    ref = _brute_layer(ids, wts, x_bits, gu, dn, s2gu, s2dn, 16, 7.0, mode == "bf16w")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_decode_layer_equals_grouped_layer():
    ids, wts, x_bits, gu, dn, s2gu, s2dn = _layer_problem(35, 8, 8, 24, 64, 32, null=(3, 17))
    ids[5, 4] = -1
    x = codecs.bf16_bits_to_f64(x_bits)
    got, _ = moe.moe_layer_decode(x, ids, wts, gu, dn, s2gu, s2dn, 32, 7.0, "bf16w")
    ref, _ = moe.moe_layer(x, ids, wts, gu, dn, s2gu, s2dn, 32, 7.0, "bf16w")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
