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

# Host threads for the oracle's per-expert loop at full size (the GPU machine gives a process
# 16 CPUs; its count of the host's cores may be larger).
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
