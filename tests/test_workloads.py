"""The seeded input generators: determinism, shapes and the stated distributions."""

import numpy as np
import pytest

import workloads as wl
from oracle import moe


def test_generators_are_deterministic_per_expert():
    w = wl.WORKLOADS["layer_e64"]
    a1, s1 = wl.expert_gate_up(w, 5)
    a2, s2 = wl.expert_gate_up(w, 5)
    b, _ = wl.expert_gate_up(w, 6)
    assert np.array_equal(a1, a2) and np.array_equal(s1, s2)
    assert not np.array_equal(a1, b)
    assert a1.shape == (2 * 768, 2048 // 2) and s1.shape == (2 * 768, 2048 // 16)
    d, sd = wl.expert_down(w, 0)
    assert d.shape == (2048, 768 // 2) and sd.shape == (2048, 768 // 16)


def test_scale_codes_are_positive_and_in_range():
    rng = np.random.default_rng(0)
    _, codes = wl.random_nvfp4(rng, 256, 4096)
    from oracle.codecs import e4m3fn_decode
    v = e4m3fn_decode(codes)
    assert np.all(v >= 2.0 ** -4) and np.all(v <= 4.0)
    assert len(np.unique(codes)) == 49  # E4M3 codes reachable from [2^-4, 4]


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_routing_shapes_and_slot_counts(name):
    w = wl.WORKLOADS[name]
    ids, wts = wl.routing(w)
    assert ids.shape == (w.rows, w.top_k) and wts.shape == (w.rows, w.top_k)
    assert np.all((ids >= 0) & (ids < w.num_experts))
    assert np.all(np.sort(ids, axis=1)[:, 1:] != np.sort(ids, axis=1)[:, :-1])  # distinct per row
    assert np.allclose(wts.sum(axis=1), 1.0, atol=1e-6)
    for c in range(w.n_chunks):
        al = moe.align(ids[c * w.chunk:(c + 1) * w.chunk], w.num_experts)
        assert al["expert_offsets"][-1] == w.chunk * w.top_k  # slot counts sum to rows*top_k


def test_zipf_routing_is_skewed():
    w = wl.WORKLOADS["long_prefill"]
    ids, _ = wl.routing(w)
    load = np.bincount(ids[:256].reshape(-1), minlength=w.num_experts)
    assert load.max() > 150  # the hottest expert takes most rows of a sub-chunk
    assert (load > 0).sum() < 245
