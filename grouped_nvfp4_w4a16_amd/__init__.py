"""grouped_nvfp4_w4a16_amd: routed-MoE prefill with a grouped NVFP4 W4A16 GEMM on MI355X.

Thin Python binding of ``libmoe_w4a16.so`` (the HIP kernels behind the C ABI in
``include/moe_w4a16.h``). This module only marshals arguments: torch tensors supply device
memory and the current HIP stream, every step of the computation runs in the library's
kernels. Nothing here falls back to another implementation: if the library is missing,
``load()`` raises.

Calls (same names as the C ABI):
- ``moe_align``: top-k ids -> expert-sorted slot order.
- ``moe_w4a16_grouped_gemm``: one launch over all experts.
- ``swiglu_clamp``, ``moe_combine``.
- ``moe_w4a16_dequant_bf16``: diagnostic, the BF16 weight operand the GEMM decodes.
- ``moe_router_topk``: router logits -> top-k ids and weights.
- ``moe_dense_gate_up_swiglu_bf16``, ``moe_dense_gemm_bf16``: the shared expert's BF16
  GEMMs (gate/up with the SwiGLU in the epilogue, then down).
- ``moe_row_union``, ``moe_w4a16_gemv_union``, ``moe_w4a16_gemv_union_swiglu``: the
  decode / verify path for a few rows (the union of their experts, each swept once).

Helpers: ``ExpertTable`` (device pointer table of per-expert NVFP4 weights),
``Workspace`` (every buffer of one layer call, allocated once), ``SharedExpert`` (the
shared expert's weights and buffers), ``moe_layer`` (the calls of one routed layer in
order), ``DecodeWorkspace`` and ``moe_layer_decode`` (the same layer for a few rows through
the union path).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "load", "MoeError", "moe_align", "moe_w4a16_grouped_gemm", "swiglu_clamp", "moe_combine",
    "moe_w4a16_grouped_gemm_swiglu", "moe_w4a16_dequant_bf16", "moe_router_topk",
    "moe_layer_from_logits", "ExpertTable", "Workspace", "moe_layer", "EXPORTS", "LIB_PATH",
    "moe_dense_gemm_bf16", "moe_dense_gate_up_swiglu_bf16", "moe_dense_workspace_bytes",
    "dense_workspace", "SharedExpert", "moe_zero_rows", "moe_align_zero",
    "moe_row_union", "moe_w4a16_gemv_union", "moe_w4a16_gemv_union_swiglu", "DecodeWorkspace",
    "moe_layer_decode", "UNION_MAX_ROWS", "source_sha256", "moe_hbm_read_probe",
    "moe_dense_gemm_bf16_noalloc", "DENSE_NOALLOC_SCRATCH_BYTES", "moe_dense_splitk_ways",
    "moe_dense_gemm_bf16_partials", "moe_combine_partials", "SharedPartials",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_w4a16.so")

# Every symbol include/moe_w4a16.h declares.
EXPORTS = (
    "moe_w4a16_status_string", "moe_w4a16_last_error", "moe_w4a16_source_sha256", "moe_align",
    "moe_w4a16_grouped_gemm",
    "moe_w4a16_grouped_gemm_swiglu", "swiglu_clamp", "moe_combine", "moe_w4a16_dequant_bf16",
    "moe_router_topk", "moe_dense_gemm_bf16", "moe_dense_gate_up_swiglu_bf16",
    "moe_dense_workspace_bytes", "moe_zero_rows", "moe_row_union", "moe_w4a16_gemv_union",
    "moe_w4a16_gemv_union_swiglu", "moe_hbm_read_probe", "moe_dense_gemm_bf16_noalloc",
    "moe_align_zero", "moe_dense_splitk_ways", "moe_dense_gemm_bf16_partials",
    "moe_combine_partials",
)

UNION_MAX_IDS = 1024  # MOE_UNION_MAX_IDS: rows * top_k of moe_row_union
UNION_MAX_ROWS = 16  # MOE_UNION_MAX_ROWS: rows of moe_w4a16_gemv_union
UNION_GEMV_MAX_IDS = 512  # MOE_UNION_GEMV_MAX_IDS: rows * top_k of moe_w4a16_gemv_union
DENSE_NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_DENSE_NOALLOC_SCRATCH_BYTES

_LIB = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

_SIGNATURES = {
    "moe_w4a16_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_w4a16_last_error": ([], ctypes.c_char_p),
    "moe_w4a16_source_sha256": ([], ctypes.c_char_p),
    "moe_align": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_align_zero": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32,
                        _vp], ctypes.c_int),
    "moe_w4a16_grouped_gemm": (
        [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
         _vp], ctypes.c_int),
    "moe_w4a16_grouped_gemm_swiglu": (
        [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
         _f32, _vp], ctypes.c_int),
    "swiglu_clamp": ([_vp, _vp, _i64, _vp, _i64, _i32, _i32, _f32, _vp], ctypes.c_int),
    "moe_combine_partials": ([_vp, _i64, _i32, _vp, _vp, _vp, _i32, _i64, _vp, _i64, _i32, _i32,
                              _i32, _vp], ctypes.c_int),
    "moe_dense_splitk_ways": ([_i32, _i32], ctypes.c_int32),
    "moe_dense_gemm_bf16_partials": ([_vp, _i64, _vp, _i64, _vp, _i32, _i32, _i32, _i64, _vp],
                                     ctypes.c_int),
    "moe_combine": ([_vp, _i64, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp],
                    ctypes.c_int),
    "moe_w4a16_dequant_bf16": ([_vp, _vp, _f32, _vp, _i32, _i32, _vp], ctypes.c_int),
    "moe_router_topk": ([_vp, _i64, _i32, _i32, _vp, _i32, _f32, _i32, _vp, _vp, _vp],
                        ctypes.c_int),
    "moe_dense_gemm_bf16": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp, _i64,
                             _vp], ctypes.c_int),
    "moe_dense_gate_up_swiglu_bf16": (
        [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _i64, _vp],
        ctypes.c_int),
    "moe_dense_workspace_bytes": ([_i32, _i32, _i32, _i32], _i64),
    "moe_dense_gemm_bf16_noalloc": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp],
                                    ctypes.c_int),
    "moe_hbm_read_probe": ([_vp, _i64, _vp, _i32, _i32, _vp], ctypes.c_int),
    "moe_zero_rows": ([_vp, _i64, _i32, _i32, _vp], ctypes.c_int),
    "moe_row_union": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_w4a16_gemv_union": (
        [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i64, _i32, _i32,
         _vp], ctypes.c_int),
    "moe_w4a16_gemv_union_swiglu": (
        [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i64, _i32, _i32,
         _f32, _vp], ctypes.c_int),
}


class MoeError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, name: str, status: int, message: str):
        super().__init__(f"{name} failed with status {status}: {message}")
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the shared library (once). Raises if it has not been built, or if it was built
    from sources other than the ones on disk (the source hash compiled into it differs)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m grouped_nvfp4_w4a16_amd.build`")
    # torch's HIP runtime first: the library then binds to the one torch uses instead of
    # loading a second runtime into the process.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    from . import build as _build

    built, on_disk = lib.moe_w4a16_source_sha256().decode(), _build.source_sha256()
    if built != on_disk:
        raise RuntimeError(
            f"{path} was built from other sources (library {built[:16]}, sources on disk "
            f"{on_disk[:16]}): rebuild it with `python -m grouped_nvfp4_w4a16_amd.build`")
    _LIB = lib
    return lib


def source_sha256() -> str:
    """The source hash compiled into the loaded library (equal to the sources on disk)."""
    return load().moe_w4a16_source_sha256().decode()


def _check(name: str, status: int) -> None:
    if status != 0:
        lib = load()
        msg = lib.moe_w4a16_last_error().decode() or lib.moe_w4a16_status_string(status).decode()
        raise MoeError(name, status, msg)


def _p(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _want(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")


def _bf16_matrix(t, name):
    """(data tensor, leading dimension in elements) of a row-major 2-D BF16 tensor."""
    import torch

    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected BF16 data, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a row-major 2-D tensor")
    return t, t.stride(0)


# ------------------------------------------------------------------------------- calls

def moe_align(topk_ids, num_experts: int, sorted_token_ids, sorted_expert_ids, expert_offsets,
              token_to_perm, active_experts=None, counters=None, stream=None, zero=None) -> None:
    """Expert-sorted slot order of ``topk_ids`` (int32 ``[rows, top_k]``); see the header.
    With ``zero`` (a BF16 ``[rows * top_k, cols]`` view, e.g. ``expert_out``), the same
    launch also zeroes it: moe_align_zero, the sort and the zero-first step together."""
    import torch

    for t, n in ((topk_ids, "topk_ids"), (sorted_token_ids, "sorted_token_ids"),
                 (sorted_expert_ids, "sorted_expert_ids"), (expert_offsets, "expert_offsets"),
                 (token_to_perm, "token_to_perm"), (active_experts, "active_experts"),
                 (counters, "counters")):
        _want(t, torch.int32, n)
    rows, top_k = topk_ids.shape
    s = rows * top_k
    if not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous")
    for t, need, n in ((sorted_token_ids, s, "sorted_token_ids"),
                       (sorted_expert_ids, s, "sorted_expert_ids"),
                       (token_to_perm, s, "token_to_perm"),
                       (expert_offsets, num_experts + 1, "expert_offsets"),
                       (active_experts, num_experts, "active_experts"), (counters, 2, "counters")):
        if t is not None and (t.numel() < need or not t.is_contiguous()):
            raise ValueError(f"{n}: needs {need} contiguous elements")
    if zero is not None:
        zero, ldz = _bf16_matrix(zero, "zero")
        if zero.shape[0] != s:
            raise ValueError("zero: needs rows * top_k rows")
        _check("moe_align_zero", load().moe_align_zero(
            _p(topk_ids), rows, top_k, num_experts, _p(sorted_token_ids),
            _p(sorted_expert_ids), _p(expert_offsets), _p(token_to_perm), _p(active_experts),
            _p(counters), _p(zero), ldz, zero.shape[1], _stream(stream)))
        return
    _check("moe_align", load().moe_align(
        _p(topk_ids), rows, top_k, num_experts, _p(sorted_token_ids), _p(sorted_expert_ids),
        _p(expert_offsets), _p(token_to_perm), _p(active_experts), _p(counters),
        _stream(stream)))


def _active_list(active_experts, counters, num_experts):
    """moe_align's active-expert list and counters (both or neither)."""
    import torch

    if (active_experts is None) != (counters is None):
        raise ValueError("active_experts and counters go together")
    _want(active_experts, torch.int32, "active_experts")
    _want(counters, torch.int32, "counters")
    if active_experts is not None and (active_experts.numel() < num_experts or
                                       counters.numel() < 2):
        raise ValueError("active_experts needs num_experts elements, counters 2")
    return _p(active_experts), _p(counters)


def moe_w4a16_grouped_gemm(a, table: "ExpertTable", expert_offsets, c, a_gather=None,
                           max_rows: int | None = None, stream=None, active_experts=None,
                           counters=None) -> None:
    """``c[s] = a[g(s)] @ W_e^T`` for every sorted row s of every present expert e. With
    moe_align's ``active_experts`` and ``counters``, a launch with fewer rows than experts
    visits only the experts that have rows (same results)."""
    import torch

    a, lda = _bf16_matrix(a, "a")
    c, ldc = _bf16_matrix(c, "c")
    _want(expert_offsets, torch.int32, "expert_offsets")
    _want(a_gather, torch.int32, "a_gather")
    act_p, cnt_p = _active_list(active_experts, counters, table.num_experts)
    if expert_offsets.numel() < table.num_experts + 1:
        raise ValueError("expert_offsets: needs num_experts + 1 elements")
    rows = c.shape[0] if max_rows is None else max_rows
    if rows > c.shape[0] or (a_gather is not None and a_gather.numel() < rows):
        raise ValueError("max_rows exceeds c or a_gather")
    if a_gather is None and rows > a.shape[0]:
        raise ValueError("without a_gather, a needs max_rows rows")
    if a.shape[1] < table.k or c.shape[1] < table.n:
        raise ValueError("a or c too narrow for the table's k, n")
    _check("moe_w4a16_grouped_gemm", load().moe_w4a16_grouped_gemm(
        _p(a), lda, a.shape[0], _p(a_gather), _p(table.packed_ptrs), _p(table.scale_ptrs),
        _p(table.scale2), _p(expert_offsets), table.num_experts, act_p, cnt_p, _p(c), ldc,
        rows, table.n, table.k, _stream(stream)))


def moe_w4a16_grouped_gemm_swiglu(a, table: "ExpertTable", expert_offsets, act, limit: float,
                                  a_gather=None, max_rows: int | None = None,
                                  stream=None, active_experts=None, counters=None) -> None:
    """``act[s] = swiglu_clamp(gate, up)`` of ``a[g(s)] @ W_e^T`` for a fused gate_up table
    (``table.n = 2 mi``), without storing the gate_up values. ``active_experts`` and
    ``counters`` as for moe_w4a16_grouped_gemm."""
    import torch

    if table.n % 2:
        raise ValueError("the fused gate_up table needs an even n")
    mi = table.n // 2
    a, lda = _bf16_matrix(a, "a")
    act, ld_act = _bf16_matrix(act, "act")
    _want(expert_offsets, torch.int32, "expert_offsets")
    _want(a_gather, torch.int32, "a_gather")
    if expert_offsets.numel() < table.num_experts + 1:
        raise ValueError("expert_offsets: needs num_experts + 1 elements")
    rows = act.shape[0] if max_rows is None else max_rows
    if rows > act.shape[0] or (a_gather is not None and a_gather.numel() < rows):
        raise ValueError("max_rows exceeds act or a_gather")
    if a_gather is None and rows > a.shape[0]:
        raise ValueError("without a_gather, a needs max_rows rows")
    if a.shape[1] < table.k or act.shape[1] < mi:
        raise ValueError("a or act too narrow for the table's k, n / 2")
    act_p, cnt_p = _active_list(active_experts, counters, table.num_experts)
    _check("moe_w4a16_grouped_gemm_swiglu", load().moe_w4a16_grouped_gemm_swiglu(
        _p(a), lda, a.shape[0], _p(a_gather), _p(table.packed_ptrs), _p(table.scale_ptrs),
        _p(table.scale2), _p(expert_offsets), table.num_experts, act_p, cnt_p, _p(act),
        ld_act, rows, mi, table.k, float(limit), _stream(stream)))



def moe_row_union(topk_ids, num_experts: int, u_eid, u_slot, slot_perm=None, counters=None,
                  stream=None, present=None) -> None:
    """The union of the experts the rows of ``topk_ids`` (int32 ``[rows, top_k]``) selected:
    ``u_eid [rows*top_k]``, ``u_slot [rows*top_k, rows]``, optional ``slot_perm`` and
    ``counters``; see the header. ``present`` (an ``ExpertTable``) leaves out the experts
    with null entries in that table: their slots are not covered."""
    import torch

    for t, n in ((topk_ids, "topk_ids"), (u_eid, "u_eid"), (u_slot, "u_slot"),
                 (slot_perm, "slot_perm"), (counters, "counters")):
        _want(t, torch.int32, n)
    rows, top_k = topk_ids.shape
    t_ids = rows * top_k
    if not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous")
    for t, need, n in ((u_eid, t_ids, "u_eid"), (u_slot, t_ids * rows, "u_slot"),
                       (slot_perm, t_ids, "slot_perm"), (counters, 2, "counters")):
        if t is not None and (t.numel() < need or not t.is_contiguous()):
            raise ValueError(f"{n}: needs {need} contiguous elements")
    pres = None
    if present is not None:
        if present.num_experts != num_experts:
            raise ValueError("present: the table has another number of experts")
        pres = _p(present.packed_ptrs)
    _check("moe_row_union", load().moe_row_union(
        _p(topk_ids), rows, top_k, num_experts, pres, _p(u_eid), _p(u_slot), _p(slot_perm),
        _p(counters), _stream(stream)))


def _union_gemv_common(a, table, u_eid, u_slot, c, rows, top_k, a_per_slot):
    import torch

    a, lda = _bf16_matrix(a, "a")
    c, ldc = _bf16_matrix(c, "c")
    _want(u_eid, torch.int32, "u_eid")
    _want(u_slot, torch.int32, "u_slot")
    t_ids = rows * top_k
    if u_eid.numel() < t_ids or u_slot.numel() < t_ids * rows:
        raise ValueError("u_eid / u_slot too small for rows * top_k")
    if not (u_eid.is_contiguous() and u_slot.is_contiguous()):
        raise ValueError("u_eid and u_slot must be contiguous")
    if c.shape[0] < t_ids:
        raise ValueError("c needs rows * top_k rows")
    if a.shape[0] < (t_ids if a_per_slot else rows):
        raise ValueError("a needs rows (or rows * top_k with a_per_slot) rows")
    if a.shape[1] < table.k:
        raise ValueError("a too narrow for the table's k")
    return a, lda, c, ldc


def moe_w4a16_gemv_union(a, table: "ExpertTable", u_eid, u_slot, c, rows: int, top_k: int,
                         a_per_slot: bool = False, stream=None) -> None:
    """``c[r*top_k + j] = a[src] @ W_e^T`` for each union entry's rows (src = r, or the slot
    r*top_k + j with ``a_per_slot``); each union expert's weights are swept once."""
    a, lda, c, ldc = _union_gemv_common(a, table, u_eid, u_slot, c, rows, top_k, a_per_slot)
    if c.shape[1] < table.n:
        raise ValueError("c too narrow for the table's n")
    _check("moe_w4a16_gemv_union", load().moe_w4a16_gemv_union(
        _p(a), lda, a.shape[0], int(bool(a_per_slot)), _p(table.packed_ptrs),
        _p(table.scale_ptrs), _p(table.scale2), _p(u_eid), _p(u_slot), rows, top_k,
        table.num_experts, _p(c), ldc, table.n, table.k, _stream(stream)))


def moe_w4a16_gemv_union_swiglu(a, table: "ExpertTable", u_eid, u_slot, act, limit: float,
                                rows: int, top_k: int, a_per_slot: bool = False,
                                stream=None) -> None:
    """moe_w4a16_gemv_union over a fused gate_up table with the SwiGLU clamp in the
    epilogue: ``act[r*top_k + j] = swiglu_clamp(gate, up)``."""
    if table.n % 2:
        raise ValueError("the fused gate_up table needs an even n")
    mi = table.n // 2
    a, lda, act, ld_act = _union_gemv_common(a, table, u_eid, u_slot, act, rows, top_k,
                                             a_per_slot)
    if act.shape[1] < mi:
        raise ValueError("act too narrow for the table's n / 2")
    _check("moe_w4a16_gemv_union_swiglu", load().moe_w4a16_gemv_union_swiglu(
        _p(a), lda, a.shape[0], int(bool(a_per_slot)), _p(table.packed_ptrs),
        _p(table.scale_ptrs), _p(table.scale2), _p(u_eid), _p(u_slot), rows, top_k,
        table.num_experts, _p(act), ld_act, mi, table.k, float(limit), _stream(stream)))

def moe_router_topk(logits, top_k: int, topk_ids, topk_weights, bias=None,
                    routed_scale: float = 1.0, renormalize: bool = True, stream=None) -> None:
    """Top-k expert ids and weights of each row of FP32 ``logits`` ``[rows, E]`` into
    ``topk_ids`` int32 and ``topk_weights`` float32, both ``[rows, top_k]`` contiguous."""
    import torch

    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda:
        raise TypeError("logits: expected a 2-D float32 device tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits: rows must be contiguous")
    rows, n_exp = logits.shape
    for t, dt, name in ((topk_ids, torch.int32, "topk_ids"), (topk_weights, torch.float32,
                                                                "topk_weights")):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.numel() < rows * top_k:
            raise ValueError(f"{name}: expected a contiguous {dt} device tensor of rows * top_k")
    if bias is not None:
        _want(bias, torch.float32, "bias")
        if bias.numel() < n_exp:
            raise ValueError("bias: needs num_experts entries")
    _check("moe_router_topk", load().moe_router_topk(
        _p(logits), logits.stride(0), rows, n_exp, _p(bias), int(top_k), float(routed_scale),
        1 if renormalize else 0, _p(topk_ids), _p(topk_weights), _stream(stream)))


def swiglu_clamp(gate, up, out, limit: float, stream=None) -> None:
    """``out = silu(min(gate, L)) * clamp(up, -L, L)`` over ``[rows, n]`` views."""
    if gate.shape != up.shape or gate.stride() != up.stride():
        raise ValueError("gate and up must be views of the same shape and strides")
    gate, ld_in = _bf16_matrix(gate, "gate")
    out, ld_out = _bf16_matrix(out, "out")
    rows, n = gate.shape
    if out.shape[0] < rows or out.shape[1] < n:
        raise ValueError("out too small")
    _check("swiglu_clamp", load().swiglu_clamp(
        _p(gate), _p(up), ld_in, _p(out), ld_out, rows, n, float(limit), _stream(stream)))


class SharedPartials:
    """The shared expert's down projection as FP32 split-K partial sums: ``partials`` a
    contiguous float32 ``[ways, rows, hidden]`` device tensor (moe_dense_gemm_bf16_partials).
    Passed as moe_combine's ``shared``, it is reduced inside the combine
    (moe_combine_partials), with the bits of the BF16 output moe_dense_gemm_bf16 writes."""

    def __init__(self, partials):
        import torch

        _want(partials, torch.float32, "partials")
        if partials.dim() != 3 or not partials.is_contiguous() or not partials.is_cuda:
            raise ValueError("partials: expected a contiguous [ways, rows, hidden] device tensor")
        self.partials = partials
        self.ways = partials.shape[0]


def moe_combine(expert_out, token_to_perm, topk_weights, out, shared=None, stream=None) -> None:
    """``out[r] = sum_j w[r, j] * expert_out[token_to_perm[r, j]] (+ shared[r])``. ``shared``
    is a BF16 ``[rows, H]`` view, a ``SharedPartials`` (moe_combine_partials) or None."""
    import torch

    expert_out, ld_e = _bf16_matrix(expert_out, "expert_out")
    out, ld_out = _bf16_matrix(out, "out")
    _want(token_to_perm, torch.int32, "token_to_perm")
    _want(topk_weights, torch.float32, "topk_weights")
    rows, top_k = topk_weights.shape
    if token_to_perm.numel() < rows * top_k or not token_to_perm.is_contiguous():
        raise ValueError("token_to_perm: needs rows * top_k contiguous elements")
    if not topk_weights.is_contiguous():
        raise ValueError("topk_weights must be contiguous")
    hidden = out.shape[1]
    if expert_out.shape[1] < hidden or out.shape[0] < rows:
        raise ValueError("shape mismatch")
    if isinstance(shared, SharedPartials):
        if tuple(shared.partials.shape[1:]) != (rows, hidden):
            raise ValueError(f"shared partials {tuple(shared.partials.shape)} do not match "
                             f"{rows} rows x {hidden}")
        _check("moe_combine_partials", load().moe_combine_partials(
            _p(expert_out), ld_e, expert_out.shape[0], _p(token_to_perm), _p(topk_weights),
            _p(shared.partials), shared.ways, shared.partials.numel() * 4, _p(out), ld_out,
            rows, hidden, top_k, _stream(stream)))
        return
    ld_s = 0
    if shared is not None:
        shared, ld_s = _bf16_matrix(shared, "shared")
    _check("moe_combine", load().moe_combine(
        _p(expert_out), ld_e, expert_out.shape[0], _p(token_to_perm), _p(topk_weights),
        _p(shared), ld_s, _p(out), ld_out, rows, hidden, top_k, _stream(stream)))


def moe_combine_partials(expert_out, token_to_perm, topk_weights, out, partials: SharedPartials,
                         stream=None) -> None:
    """moe_combine with the shared term reduced from split-K partials (same bits as the
    BF16 output of the split-K down projection)."""
    if not isinstance(partials, SharedPartials):
        raise TypeError("partials: expected a SharedPartials")
    moe_combine(expert_out, token_to_perm, topk_weights, out, partials, stream)


def moe_w4a16_dequant_bf16(packed, scales, scale2: float, out, stream=None) -> None:
    """Diagnostic: the BF16 weight operand ``out[n, k]`` the grouped GEMM decodes."""
    import torch

    _want(packed, torch.uint8, "packed")
    _want(scales, torch.uint8, "scales")
    n, half_k = packed.shape
    k = half_k * 2
    if scales.shape != (n, k // 16) or out.shape != (n, k):
        raise ValueError("shape mismatch")
    _check("moe_w4a16_dequant_bf16", load().moe_w4a16_dequant_bf16(
        _p(packed), _p(scales), float(scale2), _p(out), n, k, _stream(stream)))


def moe_hbm_read_probe(buf, sink, blocks: int = 2048, unroll: int = 8, stream=None) -> None:
    """Diagnostic: stream every byte of the contiguous device tensor ``buf`` (a read-only
    HBM ceiling probe, or a cache-evicting stream); ``sink`` is a uint32 device tensor of
    at least ``blocks`` elements that the loads feed."""
    import torch

    if sink.dtype not in (torch.int32, torch.uint32) or not sink.is_cuda:
        raise TypeError("sink: expected an int32 or uint32 device tensor")
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_contiguous():
        raise ValueError("buf and sink must be contiguous device tensors")
    if sink.numel() < blocks:
        raise ValueError("sink needs one element per block")
    nbytes = buf.numel() * buf.element_size()
    _check("moe_hbm_read_probe", load().moe_hbm_read_probe(
        _p(buf), nbytes, _p(sink), int(blocks), int(unroll), _stream(stream)))


def moe_zero_rows(c, stream=None) -> None:
    """Zero a BF16 ``[rows, cols]`` row-major view (the zero-first step on expert_out)."""
    c, ldc = _bf16_matrix(c, "c")
    _check("moe_zero_rows", load().moe_zero_rows(_p(c), ldc, c.shape[0], c.shape[1],
                                                 _stream(stream)))


def moe_dense_workspace_bytes(m: int, n: int, k: int, swiglu: bool = False) -> int:
    """Bytes of the split-K workspace of moe_dense_gemm_bf16 (``n`` = output width) or of
    moe_dense_gate_up_swiglu_bf16 (``swiglu=True``, ``n`` = inter) at these sizes."""
    return int(load().moe_dense_workspace_bytes(int(m), int(n), int(k), 1 if swiglu else 0))


def dense_workspace(m: int, n: int, k: int, swiglu: bool = False, device="cuda"):
    """A uint8 device tensor sized for the split-K form at these sizes."""
    import torch

    return torch.empty(max(moe_dense_workspace_bytes(m, n, k, swiglu), 1), dtype=torch.uint8,
                       device=device)


def _workspace(ws):
    import torch

    if ws is None:
        return None, 0
    _want(ws, torch.uint8, "workspace")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return _p(ws), ws.numel()


def moe_dense_gemm_bf16(a, b, c, stream=None, workspace=None) -> None:
    """``c[m, n] = a[m, :] @ b[n, :]`` (BF16 in and out, FP32 accumulation) over
    ``a [M, K]``, ``b [N, K]`` and ``c [M, N]`` row-major views. With ``workspace`` (see
    ``dense_workspace``) it runs split over K with larger tiles."""
    a, lda = _bf16_matrix(a, "a")
    b, ldb = _bf16_matrix(b, "b")
    c, ldc = _bf16_matrix(c, "c")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(c.shape) != (m, n):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, c {tuple(c.shape)}")
    wp, wb = _workspace(workspace)
    _check("moe_dense_gemm_bf16", load().moe_dense_gemm_bf16(
        _p(a), lda, _p(b), ldb, _p(c), ldc, m, n, k, wp, wb, _stream(stream)))


def moe_dense_splitk_ways(m: int, k: int) -> int:
    """The K split count of the split-K form for m rows at this k."""
    return int(load().moe_dense_splitk_ways(int(m), int(k)))


def moe_dense_gemm_bf16_partials(a, b, partials, stream=None) -> SharedPartials:
    """The split-K form's FP32 partial sums of ``a [M, K] @ b [N, K]^T`` into the front of
    the contiguous float32 device tensor ``partials`` (at least ways x M x N elements,
    ways = moe_dense_splitk_ways(M, K)); returns them as a ``[ways, M, N]``
    ``SharedPartials`` view."""
    import torch

    a, lda = _bf16_matrix(a, "a")
    b, ldb = _bf16_matrix(b, "b")
    _want(partials, torch.float32, "partials")
    if not partials.is_contiguous():
        raise ValueError("partials must be contiguous")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}")
    ways = moe_dense_splitk_ways(m, k)
    _check("moe_dense_gemm_bf16_partials", load().moe_dense_gemm_bf16_partials(
        _p(a), lda, _p(b), ldb, _p(partials), m, n, k, partials.numel() * 4, _stream(stream)))
    return SharedPartials(partials.view(-1)[:ways * m * n].view(ways, m, n))


def moe_dense_gemm_bf16_noalloc(a, b, c, stream=None) -> None:
    """moe_dense_gemm_bf16 in its split-K form with the library's own device scratch (no
    workspace, no allocation by anyone); same bits as ``moe_dense_gemm_bf16`` with a
    workspace. Sizes whose partials exceed ``DENSE_NOALLOC_SCRATCH_BYTES`` raise."""
    a, lda = _bf16_matrix(a, "a")
    b, ldb = _bf16_matrix(b, "b")
    c, ldc = _bf16_matrix(c, "c")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(c.shape) != (m, n):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, c {tuple(c.shape)}")
    _check("moe_dense_gemm_bf16_noalloc", load().moe_dense_gemm_bf16_noalloc(
        _p(a), lda, _p(b), ldb, _p(c), ldc, m, n, k, _stream(stream)))


def moe_dense_gate_up_swiglu_bf16(a, gate_w, up_w, act, limit: float, stream=None,
                                  workspace=None) -> None:
    """``act = swiglu_clamp(bf16(a @ gate_w^T), bf16(a @ up_w^T))`` in one launch over
    ``a [M, K]``, ``gate_w`` and ``up_w [I, K]`` (same strides) and ``act [M, I]``. With
    ``workspace`` it runs split over K with larger tiles."""
    a, lda = _bf16_matrix(a, "a")
    gate_w, ldw = _bf16_matrix(gate_w, "gate_w")
    up_w, ldw_up = _bf16_matrix(up_w, "up_w")
    act, ld_act = _bf16_matrix(act, "act")
    m, k = a.shape
    inter = gate_w.shape[0]
    if tuple(up_w.shape) != tuple(gate_w.shape) or ldw_up != ldw:
        raise ValueError("gate_w and up_w must have the same shape and strides")
    if gate_w.shape[1] != k or tuple(act.shape) != (m, inter):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, gate_w {tuple(gate_w.shape)}, "
                         f"act {tuple(act.shape)}")
    wp, wb = _workspace(workspace)
    _check("moe_dense_gate_up_swiglu_bf16", load().moe_dense_gate_up_swiglu_bf16(
        _p(a), lda, _p(gate_w), _p(up_w), ldw, _p(act), ld_act, m, inter, k, float(limit),
        wp, wb, _stream(stream)))


# ----------------------------------------------------------------------------- helpers

class SharedExpert:
    """The shared expert: BF16 ``gate_w``, ``up_w`` ``[I, H]`` and ``down_w`` ``[H, I]``
    device tensors, plus its activation and output buffers for up to ``max_rows`` rows.
    Calling it runs moe_dense_gate_up_swiglu_bf16 then moe_dense_gemm_bf16 and returns the
    ``[rows, H]`` output view (the combine's ``shared`` term). With ``split_k`` (default)
    both run in their split-K form through one workspace (the two calls are ordered on
    the stream, so they can share it) when a call has at least ``SPLIT_K_MIN_ROWS`` rows;
    with fewer, the single pass is faster (measured at H 6144, width 2048: equal at 64
    rows, 1.5x faster at 8)."""

    SPLIT_K_MIN_ROWS = 128

    def __init__(self, gate_w, up_w, down_w, max_rows: int, split_k: bool = True):
        import torch

        inter, hidden = gate_w.shape
        if tuple(up_w.shape) != (inter, hidden) or tuple(down_w.shape) != (hidden, inter):
            raise ValueError("expected gate_w, up_w [I, H] and down_w [H, I]")
        self.gate_w, self.up_w, self.down_w = gate_w, up_w, down_w
        self.inter, self.hidden = inter, hidden
        self.act = torch.empty(max_rows, inter, dtype=torch.bfloat16, device=gate_w.device)
        self.out = torch.empty(max_rows, hidden, dtype=torch.bfloat16, device=gate_w.device)
        self.workspace = None
        if split_k and max_rows >= self.SPLIT_K_MIN_ROWS:
            # the partial tiles grow with the row tiles: size for every row count up to
            # max_rows (the split count shrinks as the row tiles grow)
            nbytes = max(max(moe_dense_workspace_bytes(m, inter, hidden, True),
                             moe_dense_workspace_bytes(m, hidden, inter, False))
                         for m in range(128, max_rows + 128, 128))
            self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                                         device=gate_w.device)

    def __call__(self, x, limit: float, stream=None):
        rows = x.shape[0]
        if rows > self.act.shape[0]:
            raise ValueError(f"{rows} rows exceed the {self.act.shape[0]} the buffers hold")
        act, out = self.act[:rows], self.out[:rows]
        ws = self.workspace if rows >= self.SPLIT_K_MIN_ROWS else None
        moe_dense_gate_up_swiglu_bf16(x, self.gate_w, self.up_w, act, limit, stream, ws)
        moe_dense_gemm_bf16(act, self.down_w, out, stream, ws)
        return out

    def for_combine(self, x, limit: float, stream=None):
        """The combine's shared term for the rows of ``x``: in the split-K form, the down
        projection's FP32 partial sums (a ``SharedPartials`` in the workspace, which
        moe_combine reduces: the same bits as __call__'s output, one launch fewer); else
        __call__'s BF16 output. The partials stay valid until the next call on this
        shared expert is enqueued."""
        import torch

        rows = x.shape[0]
        if rows > self.act.shape[0]:
            raise ValueError(f"{rows} rows exceed the {self.act.shape[0]} the buffers hold")
        ws = self.workspace if rows >= self.SPLIT_K_MIN_ROWS else None
        if ws is None:
            return self(x, limit, stream)
        act = self.act[:rows]
        moe_dense_gate_up_swiglu_bf16(x, self.gate_w, self.up_w, act, limit, stream, ws)
        # the workspace's partial tiles are read by the gate/up reduction before (stream
        # order) the down projection's partials overwrite them
        return moe_dense_gemm_bf16_partials(act, self.down_w, ws.view(torch.float32), stream)


class ExpertTable:
    """Device pointer table of one NVFP4 projection for all experts.

    ``packed[e]`` is a uint8 ``[n, k/2]`` device tensor and ``scales[e]`` a uint8
    ``[n, k/16]`` one, or ``None`` for an expert that is not present (a null entry: the
    GEMM leaves its rows alone). ``scale2`` holds one float per expert. The table keeps
    the tensors alive.
    """

    def __init__(self, packed, scales, scale2, n: int, k: int, device=None):
        import torch

        if len(packed) != len(scales) or len(packed) != len(scale2):
            raise ValueError("packed, scales and scale2 need one entry per expert")
        self.n, self.k, self.num_experts = int(n), int(k), len(packed)
        pp, sp = [], []
        for e, (p, s) in enumerate(zip(packed, scales)):
            if (p is None) != (s is None):
                raise ValueError(f"expert {e}: packed and scales must both be present or None")
            if p is None:
                pp.append(0)
                sp.append(0)
                continue
            if p.dtype != torch.uint8 or s.dtype != torch.uint8 or not p.is_cuda:
                raise TypeError(f"expert {e}: expected uint8 device tensors")
            if tuple(p.shape) != (n, k // 2) or tuple(s.shape) != (n, k // 16):
                raise ValueError(f"expert {e}: expected [{n}, {k // 2}] and [{n}, {k // 16}]")
            if not (p.is_contiguous() and s.is_contiguous()):
                raise ValueError(f"expert {e}: weights must be contiguous")
            if p.data_ptr() % 16 or s.data_ptr() % 16:
                raise ValueError(f"expert {e}: weights must be 16-byte aligned")
            pp.append(p.data_ptr())
            sp.append(s.data_ptr())
            if device is None:
                device = p.device
        if device is None:  # every entry null
            device = "cuda"
        self._keep = (list(packed), list(scales))
        self.packed_ptrs = torch.tensor(pp, dtype=torch.int64, device=device)
        self.scale_ptrs = torch.tensor(sp, dtype=torch.int64, device=device)
        self.scale2 = torch.as_tensor(scale2, dtype=torch.float32).to(device)
        self.present = [p is not None for p in packed]


class Workspace:
    """Every buffer one routed-layer call needs, allocated once for up to ``max_rows``."""

    def __init__(self, max_rows: int, top_k: int, num_experts: int, hidden: int,
                 moe_intermediate: int, device="cuda"):
        import torch

        s = max_rows * top_k
        i32 = dict(dtype=torch.int32, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        self.max_rows, self.top_k, self.num_experts = max_rows, top_k, num_experts
        self.sorted_token_ids = torch.empty(s, **i32)
        self.sorted_expert_ids = torch.empty(s, **i32)
        self.expert_offsets = torch.empty(num_experts + 1, **i32)
        self.token_to_perm = torch.empty(s, **i32)
        self.active_experts = torch.empty(num_experts, **i32)
        self.counters = torch.empty(2, **i32)
        self.topk_ids = torch.empty(max_rows, top_k, **i32)  # the device router's output
        self.topk_weights = torch.empty(max_rows, top_k, dtype=torch.float32, device=device)
        self.gate_up = torch.empty(s, 2 * moe_intermediate, **bf)
        self.act = torch.empty(s, moe_intermediate, **bf)
        self.expert_out = torch.empty(s, hidden, **bf)


def _same_experts(gate_up: ExpertTable, down: ExpertTable) -> None:
    """A layer's two tables must hold the same experts: a down entry whose gate_up entry is
    null would read activation rows nothing wrote."""
    if gate_up.num_experts != down.num_experts or gate_up.present != down.present:
        raise ValueError("gate_up and down tables must have the same experts present "
                         "(null entries at the same expert ids)")


def moe_layer(x, topk_ids, topk_weights, gate_up: ExpertTable, down: ExpertTable,
              moe_intermediate: int, limit: float, ws: Workspace, out, shared=None,
              stream=None, fused: bool = True) -> None:
    """One routed MoE layer over the rows of ``x``, all on the device, in the order of the
    grouped-prefill arm: align (and zero expert_out) -> grouped GEMM gate_up (rows gathered
    through sorted_token_ids) with the SwiGLU clamp fused into its epilogue -> grouped GEMM
    down -> indexed combine. ``fused=False`` runs the gate_up GEMM and swiglu_clamp as two
    calls (same bits).
    ``ws.expert_out`` is zeroed first, in the sort's launch (moe_align_zero), so experts
    that are not present add zero. When every down-projection entry is present the down
    GEMM writes every row the combine reads (each valid slot's row lies in its expert's
    segment), so the zeroing is skipped.
    ``shared`` is the combine's shared term: a ``[rows, H]`` BF16 tensor, a
    ``SharedPartials``, or a ``SharedExpert``, which is then run over ``x`` after the routed
    experts (its down projection's split-K reduction inside the combine when it runs in
    the split-K form: same bits)."""
    _same_experts(gate_up, down)
    rows, top_k = topk_ids.shape
    s = rows * top_k
    # absent down experts: their expert_out rows are zeroed in the sort's launch
    moe_align(topk_ids, gate_up.num_experts, ws.sorted_token_ids, ws.sorted_expert_ids,
              ws.expert_offsets, ws.token_to_perm, ws.active_experts, ws.counters, stream,
              zero=None if all(down.present) else ws.expert_out[:s])
    mi = moe_intermediate
    active = dict(active_experts=ws.active_experts, counters=ws.counters)
    if fused:
        moe_w4a16_grouped_gemm_swiglu(x, gate_up, ws.expert_offsets, ws.act, limit,
                                      ws.sorted_token_ids, max_rows=s, stream=stream, **active)
    else:
        moe_w4a16_grouped_gemm(x, gate_up, ws.expert_offsets, ws.gate_up, ws.sorted_token_ids,
                               max_rows=s, stream=stream, **active)
        swiglu_clamp(ws.gate_up[:s, :mi], ws.gate_up[:s, mi:2 * mi], ws.act[:s], limit, stream)
    moe_w4a16_grouped_gemm(ws.act, down, ws.expert_offsets, ws.expert_out, None, max_rows=s,
                           stream=stream, **active)
    if isinstance(shared, SharedExpert):
        shared = shared.for_combine(x, limit, stream)
    moe_combine(ws.expert_out[:s], ws.token_to_perm, topk_weights, out, shared, stream)


def moe_layer_from_logits(x, logits, top_k: int, gate_up: ExpertTable, down: ExpertTable,
                          moe_intermediate: int, limit: float, ws: Workspace, out, bias=None,
                          routed_scale: float = 1.0, renormalize: bool = True, shared=None,
                          stream=None, fused: bool = True) -> None:
    """The layer from FP32 router logits ``[rows, E]``: moe_router_topk into
    ``ws.topk_ids`` / ``ws.topk_weights``, then moe_layer."""
    rows = logits.shape[0]
    ids, wts = ws.topk_ids[:rows], ws.topk_weights[:rows]
    if ids.shape[1] != top_k:
        raise ValueError("the workspace was made for another top_k")
    moe_router_topk(logits, top_k, ids, wts, bias, routed_scale, renormalize, stream)
    moe_layer(x, ids, wts, gate_up, down, moe_intermediate, limit, ws, out, shared, stream,
              fused)


class DecodeWorkspace:
    """Every buffer one decode-path layer call needs, for up to ``max_rows`` (<= 16) rows."""

    def __init__(self, max_rows: int, top_k: int, hidden: int, moe_intermediate: int,
                 device="cuda"):
        import torch

        if not 1 <= max_rows <= UNION_MAX_ROWS or max_rows * top_k > UNION_GEMV_MAX_IDS:
            raise ValueError("the decode path takes 1..16 rows and rows * top_k <= 512")
        t = max_rows * top_k
        i32 = dict(dtype=torch.int32, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        self.max_rows, self.top_k = max_rows, top_k
        self.u_eid = torch.empty(t, **i32)
        self.u_slot = torch.empty(t * max_rows, **i32)
        self.slot_perm = torch.empty(t, **i32)
        self.counters = torch.empty(2, **i32)
        self.gate_up = torch.empty(t, 2 * moe_intermediate, **bf)
        self.act = torch.empty(t, moe_intermediate, **bf)
        self.expert_out = torch.empty(t, hidden, **bf)


def moe_layer_decode(x, topk_ids, topk_weights, gate_up: ExpertTable, down: ExpertTable,
                     moe_intermediate: int, limit: float, ws: DecodeWorkspace, out,
                     shared=None, stream=None, fused: bool = True) -> None:
    """The routed layer for a few rows (<= 16) through the union of their experts:
    moe_row_union -> union GEMV gate_up (each row's input) with the SwiGLU clamp fused ->
    union GEMV down (each slot's activation) -> combine through ``slot_perm``. Outputs are
    laid out by (row, slot), so no sort and no expert-sorted permutation are needed.
    ``fused=False`` runs the gate_up GEMV and swiglu_clamp as two calls (same bits).
    Slots of experts absent from the down table are left out of the union (the combine
    skips them), so unlike the sorted path no zero-first step is needed. On MI355X the
    sorted path (``moe_layer``) is faster from about 4 rows on; this path wins below."""
    _same_experts(gate_up, down)
    rows, top_k = topk_ids.shape
    t = rows * top_k
    if rows > ws.max_rows or top_k != ws.top_k:
        raise ValueError("the workspace was made for fewer rows or another top_k")
    u_slot = ws.u_slot[:t * rows]
    # Slots of experts absent from the down table are left out of the union: the combine
    # skips them, so no row needs the zero-first step.
    moe_row_union(topk_ids, gate_up.num_experts, ws.u_eid, u_slot, ws.slot_perm, ws.counters,
                  stream, present=None if all(down.present) else down)
    mi = moe_intermediate
    if fused:
        moe_w4a16_gemv_union_swiglu(x, gate_up, ws.u_eid, u_slot, ws.act, limit, rows, top_k,
                                    stream=stream)
    else:
        moe_w4a16_gemv_union(x, gate_up, ws.u_eid, u_slot, ws.gate_up, rows, top_k,
                             stream=stream)
        swiglu_clamp(ws.gate_up[:t, :mi], ws.gate_up[:t, mi:2 * mi], ws.act[:t], limit, stream)
    moe_w4a16_gemv_union(ws.act, down, ws.u_eid, u_slot, ws.expert_out, rows, top_k,
                         a_per_slot=True, stream=stream)
    if isinstance(shared, SharedExpert):
        shared = shared.for_combine(x, limit, stream)
    moe_combine(ws.expert_out[:t], ws.slot_perm[:t], topk_weights, out, shared, stream)
