"""Seeded synthetic inputs for the routed-MoE prefill path.

This module draws inputs only; it holds none of the path's arithmetic (no dequant,
no sorting, no products). Both the oracle-side tests and the GPU-side tests and bench
take their inputs from here, so both see identical bits.

Workloads (shapes and value distributions as the benchmark configurations state them):

=================  ====  =====  =====  ======  =====  ==========================
name               T     E      top_k  H (K)   mi     notes
=================  ====  =====  =====  ======  =====  ==========================
single_gemm        64    16     8      512     --     one GEMM, N=256, A-gather
layer_e64          256   64     8      2048    768    full layer, SwiGLU L=7
prefill_subchunk   256   256    8      6144    2048   full layer, uniform routing
long_prefill       4096  256    8      6144    2048   16 x 256-row sub-chunks, Zipf
small_m            8     256    8      6144    2048   experts [128, 256) null
=================  ====  =====  =====  ======  =====  ==========================

Value recipe (every workload):
- Packed NVFP4 bytes: uniform 0..255 (two independent uniform nibbles).
- Block scales: magnitudes drawn U[2**-4, 2**2] in FP32, encoded to E4M3FN
  (round-to-nearest-even, by torch's own float8 conversion); positive.
- scale2 per expert: U[0.5, 2] FP32.
- Activations: N(0, 1) FP32 rounded to BF16 by torch's conversion.
- Routing: FP32 logits N(0, 1) ``[T, E]``; top-k by logit descending, ties to the lower
  expert id; weights are the softmax over the selected logits (the renormalised
  top-k softmax), computed in FP64 and stored FP32.
- Zipf routing: ``logit[r, e] = -s * ln(rank_e) + Gumbel(0, 1)`` with ranks a seeded
  permutation of 1..E, so top-k is sampling without replacement with probability
  proportional to ``rank**-s`` (s = 1.1).
- Shared expert (layer workloads): one BF16 SwiGLU MLP of width ``mi``; gate and up
  ``[mi, H]``, down ``[H, mi]``, each N(0, 1) / sqrt(fan-in) in FP32 rounded to BF16, so
  the gate and up values of N(0, 1) rows are of order one (inside the clamp).

Seeds: one ``SeedSequence`` per (workload base seed, tensor tag, index), so any single
expert's weights can be regenerated on its own.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor tags for spawn keys
_TAG_X, _TAG_ROUTE, _TAG_GU, _TAG_DN, _TAG_S2GU, _TAG_S2DN, _TAG_ZIPF, _TAG_SHARED = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    rows: int
    num_experts: int
    top_k: int
    hidden: int
    moe_intermediate: int = 0  # 0: single GEMM workload
    gemm_n: int = 0  # single GEMM only
    limit: float = 7.0
    routing: str = "softmax"  # or "zipf"
    zipf_s: float = 1.1
    chunk_rows: int = 0  # >0: the rows run as sub-chunks of this many rows
    null_from: int = -1  # experts [null_from, E) have null table entries
    extra: dict = field(default_factory=dict)

    @property
    def n_chunks(self) -> int:
        return self.rows // self.chunk_rows if self.chunk_rows else 1

    @property
    def chunk(self) -> int:
        return self.chunk_rows if self.chunk_rows else self.rows

    def is_null(self, e: int) -> bool:
        return 0 <= self.null_from <= e


WORKLOADS = {
    "single_gemm": Workload("single_gemm", 1001, rows=64, num_experts=16, top_k=8,
                            hidden=512, gemm_n=256),
    "layer_e64": Workload("layer_e64", 1002, rows=256, num_experts=64, top_k=8,
                          hidden=2048, moe_intermediate=768),
    "prefill_subchunk": Workload("prefill_subchunk", 1003, rows=256, num_experts=256,
                                 top_k=8, hidden=6144, moe_intermediate=2048),
    "long_prefill": Workload("long_prefill", 1004, rows=4096, num_experts=256, top_k=8,
                             hidden=6144, moe_intermediate=2048, routing="zipf",
                             chunk_rows=256),
    "small_m": Workload("small_m", 1005, rows=8, num_experts=256, top_k=8, hidden=6144,
                        moe_intermediate=2048, null_from=128),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _to_bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_codes(values_f32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def random_nvfp4(rng: np.random.Generator, n: int, k: int):
    """One NVFP4 projection: packed uint8 ``[n, k/2]`` and E4M3 scale codes ``[n, k/16]``."""
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    mags = rng.uniform(2.0 ** -4, 4.0, size=(n, k // 16)).astype(np.float32)
    return packed, _to_e4m3_codes(mags)


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """BF16 bit patterns (uint16) of N(0, 1) FP32 draws."""
    return _to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def bf16_normal_scaled(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """BF16 bit patterns (uint16) of N(0, 1) FP32 draws times ``std`` (in FP32)."""
    return _to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def softmax_topk_routing(logits: np.ndarray, top_k: int):
    """Top-k ids by logit descending (ties to the lower id) and renormalised weights."""
    order = np.argsort(-logits.astype(np.float32), axis=1, kind="stable")[:, :top_k]
    sel = np.take_along_axis(logits.astype(np.float64), order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    wts = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), wts


def router_logits(w: Workload) -> np.ndarray:
    """FP32 router logits ``[T, E]`` of all rows: N(0, 1), or for Zipf routing
    ``-s ln(rank_e) + Gumbel(0, 1)`` with a seeded rank permutation."""
    rng = _rng(w.seed, _TAG_ROUTE)
    if w.routing == "softmax":
        return rng.standard_normal(size=(w.rows, w.num_experts), dtype=np.float32)
    if w.routing == "zipf":
        ranks = _rng(w.seed, _TAG_ZIPF).permutation(w.num_experts) + 1
        gumbel = rng.gumbel(size=(w.rows, w.num_experts))
        return (-w.zipf_s * np.log(ranks)[None, :] + gumbel).astype(np.float32)
    raise ValueError(w.routing)


def routing(w: Workload):
    """``(topk_ids int32 [T, top_k], topk_weights float32 [T, top_k])`` for all rows: the
    workload's routing recipe applied to router_logits(w)."""
    return softmax_topk_routing(router_logits(w), w.top_k)


def activations(w: Workload) -> np.ndarray:
    """BF16 bits ``[T, H]`` (for single_gemm: ``[T, K]``)."""
    return bf16_normal(_rng(w.seed, _TAG_X), (w.rows, w.hidden))


def gate_up_shape(w: Workload):
    if w.gemm_n:
        return w.gemm_n, w.hidden
    return 2 * w.moe_intermediate, w.hidden


def down_shape(w: Workload):
    return w.hidden, w.moe_intermediate


def expert_gate_up(w: Workload, e: int):
    """Fused gate_up projection of expert e (single_gemm: the one projection):
    packed ``[2*mi, H/2]``, scales ``[2*mi, H/16]``; gate rows first, then up rows."""
    n, k = gate_up_shape(w)
    return random_nvfp4(_rng(w.seed, _TAG_GU, e), n, k)


def expert_down(w: Workload, e: int):
    """Down projection of expert e: packed ``[H, mi/2]``, scales ``[H, mi/16]``."""
    n, k = down_shape(w)
    return random_nvfp4(_rng(w.seed, _TAG_DN, e), n, k)


def scale2_gate_up(w: Workload) -> np.ndarray:
    return _rng(w.seed, _TAG_S2GU).uniform(0.5, 2.0, size=w.num_experts).astype(np.float32)


def scale2_down(w: Workload) -> np.ndarray:
    return _rng(w.seed, _TAG_S2DN).uniform(0.5, 2.0, size=w.num_experts).astype(np.float32)


def shared_expert(w: Workload, scale: float = 1.0):
    """BF16 bits of the shared expert's ``(gate [mi, H], up [mi, H], down [H, mi])``:
    N(0, 1) * scale / sqrt(fan-in) FP32 draws rounded to BF16."""
    mi, h = w.moe_intermediate, w.hidden
    out = []
    for i, (n, k) in enumerate(((mi, h), (mi, h), (h, mi))):
        v = _rng(w.seed, _TAG_SHARED, i).standard_normal(size=(n, k), dtype=np.float32)
        out.append(_to_bf16_bits(v * np.float32(scale / np.sqrt(k))))
    return tuple(out)


def custom(name: str, seed: int, **kw) -> Workload:
    """A workload with other sizes, for parity tests that span tiles and ragged tails."""
    return Workload(name, seed, **kw)
