"""Oracle for the routed-MoE prefill path (test infrastructure only).

Plain definitions, FP64 unless the pages fix a precision. Grouping and sorting only
change the order in which the same per-slot products are formed, so the grouped GEMM
is written here as its plain definition: one dense product per expert segment.

Sources (the pages' own sections):
- Weight layout and dequant: forward_prefill_gemm module docs, "Layout compatibility"
  table (rows "packed byte for logical k", "nibble", "codebook", "block scale",
  "per-tensor scale", "remote expert (EP)", "table index"), and "What is NOT
  bit-identical", item 2 (the BF16-rounded dequant product).
- Routing buffers: glm5next_mlp forward.rs (2026-09-25), field docs of
  Glm5NextMlpWorkspace for sorted_token_ids, sorted_expert_ids, expert_offsets and
  token_to_perm.
- SwiGLU with clamp: the doc comment of swiglu / swiglu_rows in both forward.rs pages.
- Combine: forward_moe (2026-09-25), the glm5next_moe_combine_indexed launch and the
  comment that the routed rows are expert-sorted and read back through token_to_perm;
  "Zero FIRST" comment of the older forward_moe for the skipped-slot zeros.
- Router top-k: forward_moe (both pages), the router launch: FP32 logits [rows, E], an
  optional per-expert bias, top_k, n_group = 1 (the only value accepted), routed_scale
  and a renormalize flag; -1 marks an unfilled slot. The pages do not print the
  kernel's arithmetic; router_topk takes the plainest reading (its docstring).
- Shared expert: forward_dense (both glm5next_mlp forward.rs pages), a BF16 SwiGLU MLP
  run once over all rows, and the gemm helper above it (C[M, N] = A[M, K] B[N, K]^T,
  BF16 in and out); forward_moe passes its output to the combine unscaled.
- Decode / verify (a few rows): forward.rs (2026-09-25), the workspace fields u_eid
  ("union expert ids, -1 = entry unused") and u_slot ("slot per union entry per row, -1 =
  row absent"), the doc of the row-batched GEMV (C[rows, top_k, N], the union of the rows'
  selected experts, each expert swept once, the same per-(row, slot) result as one GEMV per
  row) and the doc of moe_row_groups (which rows share a sweep never changes what a row
  adds). row_union, union_gemv and moe_layer_decode follow those statements.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_from_f32, bf16_bits_to_f64, e2m1_decode, e4m3fn_decode, round_bf16

GROUP_SIZE = 16  # k values per E4M3 block scale ("block scale" row: GROUP_SIZE 16)

E2M1_VALUES = e2m1_decode(np.arange(16))  # value of each 4-bit code
E4M3_VALUES = e4m3fn_decode(np.arange(256))  # value of each 8-bit scale code


# ---------------------------------------------------------------------------------------
# Dequant
# ---------------------------------------------------------------------------------------

def nibbles_of(packed: np.ndarray, k_total: int) -> np.ndarray:
    """Unpack an N-major ``[N, K/2]`` byte matrix to ``[N, K]`` nibbles.

    The byte for logical k of row n is ``packed[n, k // 2]``; even k takes the low
    nibble, odd k the high nibble ("packed byte" and "nibble" rows of the layout table).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    n_rows = packed.shape[0]
    assert packed.shape == (n_rows, k_total // 2)
    k = np.arange(k_total)
    byte = packed[:, k // 2]
    return np.where(k % 2 == 0, byte & 0xF, byte >> 4).astype(np.uint8)


def dequant_f32(packed: np.ndarray, scales: np.ndarray, scale2: float) -> np.ndarray:
    """FP32 dequantised weights ``[N, K]`` (returned as float64 holding FP32 values).

    ``w = fl32(fl32(E2M1[q] * E4M3[s]) * scale2)``: the codebook value times the block
    scale of ``scales[n, k // 16]``, then times the expert's FP32 scale2, each product
    rounded to FP32 in that order (the grouped GEMM's order, scale2 "multiplied into the
    dequant"). The first product is exact in FP32.
    """
    scales = np.asarray(scales, dtype=np.uint8)
    n_rows, n_groups = scales.shape
    k_total = n_groups * GROUP_SIZE
    q = nibbles_of(packed, k_total)
    # Each code is decoded by the format definition once; elements then index the result.
    v = E2M1_VALUES.astype(np.float32)[q]
    d = E4M3_VALUES.astype(np.float32)[scales]  # E4M3 values are exact in FP32
    d_per_k = np.repeat(d, GROUP_SIZE, axis=1)
    s2 = np.float32(scale2)
    with np.errstate(invalid="ignore", over="ignore"):
        w32 = (v * d_per_k).astype(np.float32) * s2
    return w32.astype(np.float32).astype(np.float64)


def dequant(packed: np.ndarray, scales: np.ndarray, scale2: float, mode: str) -> np.ndarray:
    """Dequantised weights as float64 ``[N, K]``.

    ``mode="exact"``: the FP32 product itself. ``mode="bf16w"``: that FP32 product rounded
    to BF16 (round-to-nearest-even), the operand the grouped GEMM feeds its BF16 MMA.
    """
    w32 = dequant_f32(packed, scales, scale2)
    if mode == "exact":
        return w32
    if mode == "bf16w":
        return bf16_bits_to_f64(bf16_bits_from_f32(w32.astype(np.float32)))
    raise ValueError(mode)


def dequant_bf16_bits(packed: np.ndarray, scales: np.ndarray, scale2: float) -> np.ndarray:
    """BF16 bit patterns (uint16 ``[N, K]``) of the BF16-rounded dequantised weights."""
    return bf16_bits_from_f32(dequant_f32(packed, scales, scale2).astype(np.float32))


# ---------------------------------------------------------------------------------------
# Align: counting sort of the routed slots by expert
# ---------------------------------------------------------------------------------------

def align(topk_ids: np.ndarray, num_experts: int) -> dict:
    """Sort the routed slots by expert (stable in the flat slot index).

    Flat slot ``t = r * top_k + j`` of ``topk_ids[r, j]`` is valid when its id is in
    ``[0, E)``; -1 is the router's "unfilled" sentinel and every out-of-range id is
    excluded and counted. Returns:

    - ``expert_offsets[E+1]``: exclusive prefix sum of per-expert slot counts.
    - ``sorted_token_ids[S]``: for sorted row p, the token row ``t // top_k`` it came
      from ("sorted row to original token").
    - ``sorted_expert_ids[S]``: the expert of sorted row p.
    - ``token_to_perm[T, top_k]``: slot t's row in the expert-sorted order, -1 if invalid.
    - ``n_invalid``: number of excluded slots.

    Rows ``[expert_offsets[E], S)`` of the two sorted arrays hold -1.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    rows, top_k = ids.shape
    flat = ids.reshape(-1)
    n_slots = flat.size
    valid = (flat >= 0) & (flat < num_experts)

    counts = np.zeros(num_experts, dtype=np.int64)
    for t in range(n_slots):
        if valid[t]:
            counts[flat[t]] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    for e in range(num_experts):
        offsets[e + 1] = offsets[e] + counts[e]

    seen = np.zeros(num_experts, dtype=np.int64)  # slots of each expert placed so far
    sorted_token_ids = np.full(n_slots, -1, dtype=np.int64)
    sorted_expert_ids = np.full(n_slots, -1, dtype=np.int64)
    token_to_perm = np.full(n_slots, -1, dtype=np.int64)
    for t in range(n_slots):
        if not valid[t]:
            continue
        e = flat[t]
        pos = offsets[e] + seen[e]
        seen[e] += 1
        sorted_token_ids[pos] = t // top_k
        sorted_expert_ids[pos] = e
        token_to_perm[t] = pos
    return {
        "expert_offsets": offsets.astype(np.int32),
        "sorted_token_ids": sorted_token_ids.astype(np.int32),
        "sorted_expert_ids": sorted_expert_ids.astype(np.int32),
        "token_to_perm": token_to_perm.reshape(rows, top_k).astype(np.int32),
        "n_invalid": int((~valid).sum()),
    }


# ---------------------------------------------------------------------------------------
# Router top-k
# ---------------------------------------------------------------------------------------

def router_topk(logits, top_k: int, bias=None, routed_scale: float = 1.0,
                renormalize: bool = True):
    """Top-k expert selection of each row of FP32 router logits ``[T, E]``.

    Reading of the pages' router launch (forward_moe): scores are the softmax of the row's
    logits; the selection key of expert e is its score plus ``bias[e]`` when a bias is
    given, else the logit itself (softmax is increasing, so this is the same selection
    without the ties that rounding the scores could create); the top_k largest keys are
    taken in descending order, equal keys to the lower expert id. The weight of a
    selected expert is its score, divided by the selected scores' sum when
    ``renormalize``, times ``routed_scale``. If top_k exceeds E the extra slots are -1
    with weight 0. Returns ``(ids int32 [T, top_k], weights float64 [T, top_k])``.
    """
    lg = np.asarray(logits, dtype=np.float64)
    rows, n_exp = lg.shape
    ids = np.full((rows, top_k), -1, dtype=np.int32)
    wts = np.zeros((rows, top_k), dtype=np.float64)
    for r in range(rows):
        z = np.exp(lg[r] - lg[r].max())
        scores = z / z.sum()
        key = scores + np.asarray(bias, dtype=np.float64) if bias is not None else lg[r]
        # descending key, equal keys in ascending id: a stable sort of -key
        order = sorted(range(n_exp), key=lambda e: (-key[e], e))
        sel = order[:min(top_k, n_exp)]
        w = scores[sel]
        if renormalize:
            w = w / w.sum()
        ids[r, :len(sel)] = sel
        wts[r, :len(sel)] = w * routed_scale
    return ids, wts


# ---------------------------------------------------------------------------------------
# Grouped GEMM
# ---------------------------------------------------------------------------------------

def grouped_gemm(a, a_gather, experts, scale2, expert_offsets, out, mode: str,
                 expert_subset=None, workers: int = 1):
    """Grouped W4A16 product over the expert-sorted rows, written into ``out`` (float64).

    For every expert e whose table entry is not null (``experts[e]`` is a
    ``(packed [N, K/2], scales [N, K/16])`` pair; ``None`` is a null pointer, a remote
    expert), and every sorted row s in ``[expert_offsets[e], expert_offsets[e+1])``::

        out[s, n] = sum_k a[g(s), k] * w_e[n, k],   g(s) = a_gather[s] if a_gather else s

    in FP64, with ``w_e`` from :func:`dequant` in ``mode``. Rows of null experts are left
    as they are: the caller's zeros stand. ``expert_subset`` limits the work to some
    experts (used for sampled checks at large sizes).

    Each expert writes only its own segment of rows, so the experts are independent;
    ``workers > 1`` runs them on that many threads (for full-size checks), with the same
    result.
    """
    a = np.asarray(a, dtype=np.float64)
    offsets = np.asarray(expert_offsets, dtype=np.int64)
    num_experts = offsets.size - 1
    todo = range(num_experts) if expert_subset is None else expert_subset

    def one_expert(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            return
        ex = experts[e]
        if ex is None:
            return
        packed, scales = ex
        w = dequant(packed, scales, float(scale2[e]), mode)
        rows = np.arange(lo, hi)
        src = rows if a_gather is None else np.asarray(a_gather, dtype=np.int64)[rows]
        out[lo:hi, :] = a[src, :] @ w.T

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(one_expert, todo))  # list() re-raises a worker's exception
    else:
        for e in todo:
            one_expert(e)
    return out


# ---------------------------------------------------------------------------------------
# SwiGLU with clamp, combine, layer
# ---------------------------------------------------------------------------------------

def swiglu_clamp(gate, up, limit: float):
    """``silu(min(gate, L)) * clamp(up, -L, L)`` elementwise in FP64, silu(x) = x / (1 + e^-x).

    The gate is clamped from above only; the up value on both sides.
    """
    g = np.minimum(np.asarray(gate, dtype=np.float64), limit)
    u = np.minimum(np.maximum(np.asarray(up, dtype=np.float64), -limit), limit)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return silu * u


def combine(expert_out, token_to_perm, topk_weights, shared=None):
    """``out[r, h] = sum_j w[r, j] * expert_out[token_to_perm[r, j], h] (+ shared[r, h])``.

    Slots with ``token_to_perm < 0`` are skipped. FP64, slots summed in j order.
    """
    e_out = np.asarray(expert_out, dtype=np.float64)
    ttp = np.asarray(token_to_perm, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float64)
    rows, top_k = ttp.shape
    out = np.zeros((rows, e_out.shape[1]), dtype=np.float64)
    for j in range(top_k):
        p = ttp[:, j]
        ok = p >= 0
        out[ok] += wts[ok, j][:, None] * e_out[p[ok]]
    if shared is not None:
        out += np.asarray(shared, dtype=np.float64)
    return out


def moe_layer(x, topk_ids, topk_weights, gate_up, down, scale2_gate_up, scale2_down,
              moe_intermediate: int, limit: float, mode: str, shared=None, workers: int = 1):
    """One routed MoE layer over the rows of ``x`` (float64 ``[T, H]``).

    Steps, in the order of the grouped-prefill arm of forward_moe (2026-09-25):
    align -> zero expert_out -> grouped GEMM gate_up (A gathered through
    sorted_token_ids) -> SwiGLU clamp -> grouped GEMM down (A = activated rows in sorted
    order) -> indexed combine. ``gate_up[e]`` holds the fused ``[2*mi, H]`` projection,
    gate rows ``[0, mi)`` then up rows ``[mi, 2*mi)``; ``down[e]`` is ``[H, mi]``.

    In ``mode="bf16w"`` the three buffers the kernels keep in BF16 (gate_up output,
    activation, expert_out) are rounded to BF16; the returned output is left unrounded.
    ``workers`` is passed to both grouped GEMMs. Returns ``(out, intermediates)``.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, hidden = x.shape
    num_experts = len(gate_up)
    al = align(topk_ids, num_experts)
    n_slots = al["sorted_token_ids"].size
    rnd = round_bf16 if mode == "bf16w" else (lambda v: v)

    c = np.full((n_slots, 2 * moe_intermediate), np.nan)  # null-expert rows stay undefined
    grouped_gemm(x, al["sorted_token_ids"], gate_up, scale2_gate_up, al["expert_offsets"], c, mode,
                 workers=workers)
    c = rnd(c)
    act = rnd(swiglu_clamp(c[:, :moe_intermediate], c[:, moe_intermediate:], limit))
    expert_out = np.zeros((n_slots, hidden))  # zero first: skipped slots add exactly 0
    grouped_gemm(act, None, down, scale2_down, al["expert_offsets"], expert_out, mode,
                 workers=workers)
    expert_out = rnd(expert_out)
    out = combine(expert_out, al["token_to_perm"], topk_weights, shared)
    return out, {"align": al, "c": c, "act": act, "expert_out": expert_out}


# ---------------------------------------------------------------------------------------
# Shared expert
# ---------------------------------------------------------------------------------------

def dense_mlp(x, gate_w, up_w, down_w, limit: float, mode: str):
    """The shared expert: ``down(swiglu_clamp(gate(x), up(x)))`` over the rows of ``x``.

    ``x`` is ``[T, H]``; ``gate_w`` and ``up_w`` are ``[I, H]`` and ``down_w`` is ``[H, I]``,
    each stored the way the pages' gemm takes its B operand (``C = A @ B^T``, B ``[N, K]``).
    Products in FP64 of the given values::

        gate = x @ gate_w^T,  up = x @ up_w^T,  act = swiglu_clamp(gate, up, limit)
        out  = act @ down_w^T

    In ``mode="bf16w"`` the buffers the pages keep in BF16 (gate, up, act, and the output
    itself) are rounded to BF16; ``mode="exact"`` rounds nothing.
    Returns ``(out, {"gate", "up", "act"})``.
    """
    if mode not in ("exact", "bf16w"):
        raise ValueError(mode)
    rnd = round_bf16 if mode == "bf16w" else (lambda v: v)
    x = np.asarray(x, dtype=np.float64)
    gate = rnd(x @ np.asarray(gate_w, dtype=np.float64).T)
    up = rnd(x @ np.asarray(up_w, dtype=np.float64).T)
    act = rnd(swiglu_clamp(gate, up, limit))
    out = rnd(act @ np.asarray(down_w, dtype=np.float64).T)
    return out, {"gate": gate, "up": up, "act": act}



# ---------------------------------------------------------------------------------------
# Decode / verify: the union of a few rows' experts, each swept once
# ---------------------------------------------------------------------------------------

def row_union(topk_ids: np.ndarray, num_experts: int, present=None) -> dict:
    """The union of the experts the rows selected, with each row's slot per union entry.

    Flat slot ``t = r * top_k + j``. A slot is covered when its id is in ``[0, E)``, the
    expert is present (``present[e]`` true, when a mask is given: an expert absent from
    this GPU's table is treated like an invalid id) and no lower slot of the same row holds
    the same id (a proper top-k never repeats an expert in a row; a repeat is treated like
    an invalid id). Returns:

    - ``u_eid[rows * top_k]``: the distinct ids of the covered slots in order of first
      appearance in the flat order, then -1.
    - ``u_slot[rows * top_k, rows]``: ``u_slot[p, r] = j`` when row r's slot j is covered
      and selects ``u_eid[p]``, else -1.
    - ``slot_perm[rows, top_k]``: ``t`` for a covered slot, -1 otherwise (the combine's
      ``token_to_perm`` over outputs laid out as ``[rows * top_k, N]``).
    - ``n_union``, ``n_uncovered``.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    rows, top_k = ids.shape
    n_ids = rows * top_k
    u_eid = np.full(n_ids, -1, dtype=np.int64)
    u_slot = np.full((n_ids, rows), -1, dtype=np.int64)
    slot_perm = np.full((rows, top_k), -1, dtype=np.int64)
    entry_of = {}  # expert id -> union entry
    for r in range(rows):
        for j in range(top_k):
            e = int(ids[r, j])
            if not 0 <= e < num_experts:
                continue
            if present is not None and not present[e]:
                continue  # absent expert: like an invalid id
            if any(int(ids[r, jj]) == e for jj in range(j)):
                continue  # repeated in this row
            if e not in entry_of:
                entry_of[e] = len(entry_of)
                u_eid[entry_of[e]] = e
            u_slot[entry_of[e], r] = j
            slot_perm[r, j] = r * top_k + j
    return {
        "u_eid": u_eid.astype(np.int32),
        "u_slot": u_slot.astype(np.int32),
        "slot_perm": slot_perm.astype(np.int32),
        "n_union": len(entry_of),
        "n_uncovered": int((slot_perm < 0).sum()),
    }


def union_gemv(a, a_per_slot: bool, experts, scale2, u_eid, u_slot, top_k: int, out,
               mode: str):
    """W4A16 product over the union entries, written into ``out`` (float64 ``[rows*top_k, N]``).

    For every entry p with ``e = u_eid[p] >= 0`` and a non-null table entry, and every row r
    with ``j = u_slot[p, r] >= 0``::

        out[r * top_k + j, n] = sum_k a[src, k] * w_e[n, k]

    in FP64, ``src = r * top_k + j`` when ``a_per_slot`` (the down projection reads each
    slot's own activation) else ``r`` (gate_up reads the row's input). Other rows of
    ``out`` are left as they are.
    """
    a = np.asarray(a, dtype=np.float64)
    u_eid = np.asarray(u_eid, dtype=np.int64)
    u_slot = np.asarray(u_slot, dtype=np.int64)
    for p in range(u_eid.size):
        e = int(u_eid[p])
        if e < 0 or experts[e] is None:
            continue
        rs = [r for r in range(u_slot.shape[1]) if u_slot[p, r] >= 0]
        if not rs:
            continue
        packed, scales = experts[e]
        w = dequant(packed, scales, float(scale2[e]), mode)
        dst = np.array([r * top_k + int(u_slot[p, r]) for r in rs])
        src = dst if a_per_slot else np.array(rs)
        out[dst, :] = a[src, :] @ w.T
    return out


def moe_layer_decode(x, topk_ids, topk_weights, gate_up, down, scale2_gate_up, scale2_down,
                     moe_intermediate: int, limit: float, mode: str, shared=None):
    """The routed layer for a few rows through the union of their experts.

    row_union -> union_gemv gate_up (input: the row) -> SwiGLU clamp -> union_gemv down
    (input: the slot's activation) -> combine through ``slot_perm``. Buffers and rounding
    as :func:`moe_layer` (``mode="bf16w"`` rounds the gate_up output, the activation and the
    down output to BF16); outputs are laid out ``[rows * top_k, N]`` by (row, slot) instead
    of by expert. Returns ``(out, intermediates)``.
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    rows, top_k = ids.shape
    hidden = x.shape[1]
    un = row_union(ids, len(gate_up))
    rnd = round_bf16 if mode == "bf16w" else (lambda v: v)
    c = np.full((rows * top_k, 2 * moe_intermediate), np.nan)  # uncovered rows undefined
    union_gemv(x, False, gate_up, scale2_gate_up, un["u_eid"], un["u_slot"], top_k, c, mode)
    c = rnd(c)
    act = rnd(swiglu_clamp(c[:, :moe_intermediate], c[:, moe_intermediate:], limit))
    expert_out = np.zeros((rows * top_k, hidden))  # remote experts add exactly 0
    union_gemv(act, True, down, scale2_down, un["u_eid"], un["u_slot"], top_k, expert_out,
               mode)
    expert_out = rnd(expert_out)
    out = combine(expert_out, un["slot_perm"], topk_weights, shared)
    return out, {"union": un, "c": c, "act": act, "expert_out": expert_out}
