"""Helpers for the GPU parity tests: upload seeded inputs, read results back, error metrics.

Inputs come from ``workloads`` (the seeded generators both sides share); expected values
come only from ``oracle``. Nothing here computes any part of the path.
"""

from __future__ import annotations

import os

import numpy as np
import torch

import workloads as wl

# The parity gate: max |gpu - oracle| / max |oracle| against the BF16-weight oracle.
GATE = 5e-3

# Host threads for the oracle's per-expert loop at full size: at most 16 (a process may be
# given fewer CPUs than os.cpu_count() reports for the host).
ORACLE_WORKERS = max(1, min(16, os.cpu_count() or 1))


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits) -> torch.Tensor:
    """uint16 BF16 bit patterns -> a device bfloat16 tensor with those bits."""
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bf16_bits_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / scale) if scale > 0 else float(np.max(np.abs(got)))


def rel_err_rows(got, ref) -> float:
    """The gate taken row by row: max over rows of max |got - ref| / max |ref| in the row."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape and got.ndim == 2
    assert np.all(np.isfinite(got)), "non-finite output"
    scale = np.max(np.abs(ref), axis=1)
    err = np.max(np.abs(got - ref), axis=1)
    return float(np.max(np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)))


def ulp_bf16(v):
    """Spacing of BF16 numbers at |v| (8 significant bits; 2^-133 below 2^-126)."""
    return np.ldexp(1.0, np.frexp(np.maximum(np.abs(v), 2.0 ** -126))[1] - 8)


# Bounds for the layer's BF16 stores. The GPU sums in FP32 (in the matrix cores' order),
# the oracle in FP64; where the two sums straddle a rounding midpoint of a BF16 store, the
# stored values differ by one BF16 ulp (up to 2^-7 of the value). So each stored buffer
# may differ from the oracle's by one ulp per element, plus the spread of earlier flips
# through the next product (a few ulps of a BF16 input times its weights: at most ~2^-10
# of the row's largest value, far above what the FP32 sums contribute and far below what a
# wrong row, expert or scale would).

def act_bound(act_ref, c_ref, limit: float):
    """|act_gpu - act_ref| from one flip of the gate or the up value at the gate_up store
    (``c_ref``: the oracle's BF16 gate_up rows) carried through silu(g) u to first order
    (with 1.5x room for the second order), one flip at the act store, and a 2^-12 row
    floor for the FP32 exponential."""
    mi = act_ref.shape[1]
    g, u = c_ref[:, :mi], c_ref[:, mi:]
    gc = np.minimum(g, limit)
    uc = np.clip(u, -limit, limit)
    with np.errstate(over="ignore", invalid="ignore"):
        sig = 1.0 / (1.0 + np.exp(-gc))
        silu = gc * sig
        dsilu = sig * (1.0 + gc * (1.0 - sig))
    d_g = np.where(g < limit, np.abs(dsilu) * ulp_bf16(g) * np.abs(uc), 0.0)
    d_u = np.where(np.abs(u) < limit, np.abs(silu) * ulp_bf16(u), 0.0)
    floor = 2.0 ** -12 * np.max(np.abs(act_ref), axis=1, keepdims=True)
    return 1.5 * (np.nan_to_num(d_g) + np.nan_to_num(d_u)) + ulp_bf16(act_ref) + floor


def expert_out_bound(eo_ref):
    """|eo_gpu - eo_ref|: one flip at the expert_out store plus the act flips carried
    through the down product (2^-10 row floor)."""
    return ulp_bf16(eo_ref) + 2.0 ** -10 * np.max(np.abs(eo_ref), axis=1, keepdims=True)


def layer_out_bound(ref, eo_ref, token_to_perm, topk_weights):
    """|out_gpu - out_ref| per element: the output's own rounding (half an ulp, <= 2^-8 of
    it) plus, for each slot, its weight times one ulp (<= 2^-7) of the slot's expert_out
    value and that row's 2^-10 floor (expert_out_bound)."""
    ttp = np.asarray(token_to_perm).reshape(ref.shape[0], -1)
    wts = np.abs(np.asarray(topk_weights, np.float64)).reshape(ref.shape[0], -1)
    bound = 2.0 ** -8 * np.abs(ref)
    eo_row_max = np.max(np.abs(eo_ref), axis=1)
    for j in range(ttp.shape[1]):
        p = ttp[:, j]
        ok = p >= 0
        e = np.abs(eo_ref[np.where(ok, p, 0)])
        contrib = 2.0 ** -7 * e + 2.0 ** -10 * eo_row_max[np.where(ok, p, 0)][:, None]
        bound += np.where(ok, wts[:, j], 0.0)[:, None] * contrib
    return bound


def within(got, ref, bound) -> float:
    """Asserts |got - ref| <= bound everywhere (NaN nowhere) and returns the largest
    ratio |got - ref| / bound."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    ratio = np.abs(got - ref) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(ratio <= 1.0), (f"outside the bound at {tuple(int(i) for i in worst)}: "
                                  f"got {got[worst]}, ref {ref[worst]}, bound {bound[worst]}")
    return float(ratio.max())


def oracle_threads():
    """Context for a full-size oracle call on ORACLE_WORKERS threads: BLAS runs one thread
    per worker, so the workers do not oversubscribe the cores."""
    from threadpoolctl import threadpool_limits

    return threadpool_limits(limits=1)


class LazyExperts:
    """Per-expert NVFP4 weights of a workload, drawn on first use (None = null entry)."""

    def __init__(self, w: wl.Workload, which: str, null=(), keep: bool = True):
        self.w, self.which, self.null, self.keep = w, which, set(null), keep
        self._cache = {}

    def __len__(self):
        return self.w.num_experts

    def get(self, e, keep=None):
        keep = self.keep if keep is None else keep
        if e in self.null or self.w.is_null(e):
            return None
        if e in self._cache:
            return self._cache[e]
        fn = wl.expert_gate_up if self.which == "gate_up" else wl.expert_down
        ex = fn(self.w, e)
        if keep:
            self._cache[e] = ex
        return ex

    def __getitem__(self, e):
        return self.get(e)

    def __iter__(self):
        return (self.get(e) for e in range(len(self)))


def upload_table(hip, experts, scale2, n: int, k: int, only=None):
    """ExpertTable from a sequence of (packed, scales) host pairs or None.

    ``only``: upload just these experts (the rest become null entries)."""
    packed, scales = [], []
    for e in range(len(experts)):
        if only is not None and e not in only:
            ex = None
        else:
            ex = experts.get(e, keep=False) if isinstance(experts, LazyExperts) else experts[e]
        if ex is None:
            packed.append(None)
            scales.append(None)
        else:
            packed.append(dev(ex[0]))
            scales.append(dev(ex[1]))
    return hip.ExpertTable(packed, scales, np.asarray(scale2, np.float32), n, k)


def align_buffers(rows: int, top_k: int, num_experts: int):
    s = rows * top_k
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(sorted_token_ids=torch.full((max(s, 1),), -7, **i32),
                sorted_expert_ids=torch.full((max(s, 1),), -7, **i32),
                expert_offsets=torch.full((num_experts + 1,), -7, **i32),
                token_to_perm=torch.full((max(s, 1),), -7, **i32),
                active_experts=torch.full((num_experts,), -7, **i32),
                counters=torch.full((2,), -7, **i32))


_TABLES = {}


def workload_tables(hip, w: wl.Workload, only=None):
    """(lazy gate_up, lazy down, device gate_up table, device down table) of a workload,
    built once per test session. ``only``: upload just these experts."""
    key = (w.name, None if only is None else tuple(sorted(only)))
    if key not in _TABLES:
        gu, dn = LazyExperts(w, "gate_up", keep=False), LazyExperts(w, "down", keep=False)
        gt = upload_table(hip, gu, wl.scale2_gate_up(w), *wl.gate_up_shape(w), only=only)
        dt = upload_table(hip, dn, wl.scale2_down(w), *wl.down_shape(w), only=only)
        _TABLES[key] = (gu, dn, gt, dt)
    return _TABLES[key]
