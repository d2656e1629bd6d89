"""Benchmark of the routed-MoE prefill hot path on one MI355X.

One step = one pass of the whole path over one 256-row batch of the prefill sub-chunk
workload (256 experts, top_k 8, hidden 6144, moe_intermediate 2048, NVFP4 weights):
moe_align -> grouped GEMM gate_up with the SwiGLU clamp fused into its epilogue
(``--unfused``: the GEMM and swiglu_clamp as two calls) -> grouped GEMM down ->
moe_combine, all enqueued on one HIP stream with every input already in HBM. When the down
table has null entries, expert_out is zeroed first, in the sort's launch (moe_align_zero);
otherwise every row the combine reads is written by the down GEMM.

After the W warm-up steps, untimed steps continue until 0.15 s of warm-up has passed (the
GPU's clock ramps over the first tens of milliseconds of load); their number is reported as
``settle_steps``. Then exactly K steps are timed.

Prints ONE JSON line. ``value`` is HBM GB/s on the unique expert-weight bytes the step
reads (experts touched by the batch, both projections) divided by the step time;
``tflops`` is the useful FLOP rate. ``roofline`` covers the dominant kernel (the gate_up
grouped GEMM), timed with HIP events on the stream it runs on. ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload.

``shared_expert`` times the shared expert (a BF16 SwiGLU MLP of width moe_intermediate
over the same rows: moe_dense_gate_up_swiglu_bf16 then moe_dense_gemm_bf16) after the
timed steps, outside ``value``, and the down projection's split-K partials alone (the
layer's form, their reduction inside the combine); ``--with-shared`` runs it inside each
step instead and feeds it to the combine (as split-K partials when it runs split).

``decode`` times the decode / verify path on the small-M workload (8 rows, 256 experts,
half of them absent) after the timed steps, outside ``value``: the union path
(moe_row_union -> union GEMVs -> combine; the union leaves out experts absent from the
table, so this path needs no zeroing) and the sorted path on the same rows.
``--decode`` runs the main step itself through the union path (rows <= 16).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--copy-probe] [--unfused] [--device-router]
                       [--with-shared] [--no-shared] [--decode] [--no-decode] [--no-long]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E datasheet peak
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak
SETTLE_S = 0.15  # untimed warm-up time before the timed steps (clock ramp)
# Counter-measured HBM traffic of the gate_up GEMM on a workload, valid only for the kernel
# source it was measured on (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated with a copy
# kernel).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_gate_up_swiglu_{}_hbm_traffic.md")
KERNEL_SOURCES = ("grouped_nvfp4_w4a16_amd/csrc/grouped_gemm.hip",
                  "grouped_nvfp4_w4a16_amd/csrc/nvfp4_decode.h",
                  "grouped_nvfp4_w4a16_amd/csrc/w4a16_mma.h",
                  "grouped_nvfp4_w4a16_amd/csrc/swiglu.h",
                  "grouped_nvfp4_w4a16_amd/csrc/buffer_io.h")
METRIC = "grouped MoE W4A16 GEMM: HBM GB/s on unique weights + TFLOP/s, 256-row prefill"


def proj_bytes(n: int, k: int) -> int:
    """HBM bytes of one expert's NVFP4 projection: packed nibbles, E4M3 scales, scale2."""
    return n * k // 2 + n * k // 16 + 4


def kernel_source_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per gate_up launch from the committed counter summary of the workload, or
    None when the summary is missing, covers another kernel or was taken on a different
    kernel source."""
    try:
        text = open(TRAFFIC_FILE.format(workload)).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith("- `"):
            key, _, val = line.strip()[3:].partition("`:")
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_sha256() or fields.get("kernel") != kernel:
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


FLUSH_BYTES = 2 << 30  # 8x the 256 MB last-level cache (MALL)


class HbmProbe:
    """The library's pure-read probe over a 2 GiB buffer: the measured HBM read ceiling
    (best of a few launch shapes), and a cache-evicting stream between timed iterations
    of workloads that would otherwise stay cache-resident."""

    SHAPES = ((1024, 8), (2048, 8), (4096, 8), (2048, 16), (4096, 16))

    def __init__(self, hip, torch):
        self.hip, self.torch = hip, torch
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.buf.fill_(1)
        self.sink = torch.empty(max(b for b, _ in self.SHAPES), dtype=torch.int32,
                                device="cuda")

    def flush(self):
        self.hip.moe_hbm_read_probe(self.buf, self.sink, 2048, 8)

    def ceiling(self, reps: int = 10) -> dict:
        torch = self.torch
        stream = torch.cuda.current_stream()
        best = None
        for blocks, unroll in self.SHAPES:
            for _ in range(2):
                self.hip.moe_hbm_read_probe(self.buf, self.sink, blocks, unroll)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                self.hip.moe_hbm_read_probe(self.buf, self.sink, blocks, unroll)
            e1.record(stream)
            torch.cuda.synchronize()
            gbs = FLUSH_BYTES * reps / (e0.elapsed_time(e1) / 1000.0) / 1e9
            if best is None or gbs > best["GBps"]:
                best = {"GBps": round(gbs, 1), "blocks": blocks, "unroll": unroll}
        return {"kernel": "moe_hbm_read_probe", "bytes": FLUSH_BYTES, **best}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_subchunk")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the gate_up GEMM and swiglu_clamp as two calls")
    ap.add_argument("--device-router", action="store_true",
                    help="start each step from FP32 router logits (moe_router_topk on the "
                         "device) instead of precomputed top-k ids and weights")
    ap.add_argument("--with-shared", action="store_true",
                    help="run the shared expert inside each step (its output joins the "
                         "combine)")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the separate shared-expert measurement")
    ap.add_argument("--decode", action="store_true",
                    help="run the step through the decode path (union of the rows' experts, "
                         "each swept once; rows <= 16)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the separate decode-path measurement")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the skewed-routing long-prefill leg")
    return ap.parse_args()


def upload_workload(hip, w, torch):
    """Device copies of every input of the workload (weights drawn per expert)."""
    import workloads as wl

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    gp, gs, dp, ds = [], [], [], []
    for e in range(w.num_experts):
        if w.is_null(e):
            for lst in (gp, gs, dp, ds):
                lst.append(None)
            continue
        p, s = wl.expert_gate_up(w, e)
        gp.append(dev(p))
        gs.append(dev(s))
        if w.gemm_n:  # a single grouped GEMM: no down projection
            continue
        p, s = wl.expert_down(w, e)
        dp.append(dev(p))
        ds.append(dev(s))
    n_gu, k_gu = wl.gate_up_shape(w)
    n_dn, k_dn = wl.down_shape(w)
    gt = hip.ExpertTable(gp, gs, wl.scale2_gate_up(w), n_gu, k_gu)
    dt = None if w.gemm_n else hip.ExpertTable(dp, ds, wl.scale2_down(w), n_dn, k_dn)
    ids, wts = wl.routing(w)
    x = dev(wl.activations(w).view(np.int16)).view(torch.bfloat16)
    return gt, dt, dev(ids), dev(wts), x, ids


def cpu_baseline(w, ids_chunk, seconds_budget=15.0):
    """The oracle (BF16-weight mode) on a bounded sample: whole experts of the batch, both
    projections, in expert order, until about ``seconds_budget`` of host time is spent."""
    import workloads as wl
    from oracle import codecs, moe

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    al = moe.align(ids_chunk, w.num_experts)
    offsets = al["expert_offsets"]
    x = codecs.bf16_bits_to_f64(wl.activations(w)[:ids_chunk.shape[0]])
    s2gu, s2dn = wl.scale2_gate_up(w), wl.scale2_down(w)
    n_gu, k_gu = wl.gate_up_shape(w)
    n_dn, k_dn = wl.down_shape(w)
    mi = w.moe_intermediate
    single = bool(w.gemm_n)  # one grouped GEMM: no SwiGLU and no down projection
    done_bytes, flops, experts = 0, 0.0, 0
    c = np.zeros((int(offsets[-1]), n_gu))
    act = np.zeros((int(offsets[-1]), mi))
    out = np.zeros((int(offsets[-1]), n_dn))
    spent = 0.0
    for e in range(w.num_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo or w.is_null(e):
            continue
        gu = [None] * w.num_experts
        dn = [None] * w.num_experts
        gu[e] = wl.expert_gate_up(w, e)  # input generation: not timed
        if not single:
            dn[e] = wl.expert_down(w, e)
        t0 = time.perf_counter()
        moe.grouped_gemm(x, al["sorted_token_ids"], gu, s2gu, offsets, c, "bf16w",
                         expert_subset=[e])
        if not single:
            cr = codecs.round_bf16(c[lo:hi])
            act[lo:hi] = codecs.round_bf16(moe.swiglu_clamp(cr[:, :mi], cr[:, mi:], w.limit))
            moe.grouped_gemm(act, None, dn, s2dn, offsets, out, "bf16w", expert_subset=[e])
        spent += time.perf_counter() - t0
        done_bytes += proj_bytes(n_gu, k_gu) + (0 if single else proj_bytes(n_dn, k_dn))
        flops += 2.0 * (hi - lo) * (n_gu * k_gu + (0 if single else n_dn * k_dn))
        experts += 1
        if spent > seconds_budget:
            break
    dt = spent
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"{experts} experts of the {w.name} batch "
                       f"({'the grouped GEMM' if single else 'gate_up + SwiGLU + down'}, "
                       f"all their routed rows, BF16-weight mode, generation excluded), "
                       f"{dt:.1f} s"),
            "tflops": round(flops / dt / 1e12, 6)}


def time_shared_expert(se, x, w, steps, torch, stream, probe):
    """The shared expert over one batch of rows: the gate/up GEMM with the SwiGLU, then the
    down GEMM. Its working set (~84 MB) fits in the last-level cache, so each timed launch
    follows a cache-evicting stream (``probe.flush``) and has its own pair of HIP events
    (median reported); the MALL-warm rate (``steps`` launches back to back between two
    events, queued while the GPU is busy so that host launch time is not counted) is
    reported beside it. Each kernel's roofline bound is the larger of its HBM
    time (weights + input rows + output rows, once) and its matrix-core time (dense BF16
    peak)."""
    import grouped_nvfp4_w4a16_amd as hip

    rows, hidden, inter = x.shape[0], w.hidden, w.moe_intermediate
    act, outb = se.act[:rows], se.out[:rows]

    def timed(ws):
        launches = (lambda: hip.moe_dense_gate_up_swiglu_bf16(x, se.gate_w, se.up_w, act,
                                                              w.limit, workspace=ws),
                    lambda: hip.moe_dense_gemm_bf16(act, se.down_w, outb, workspace=ws))
        for _ in range(3):
            for fn in launches:
                fn()
        torch.cuda.synchronize()
        cold, warm = [], []
        for fn in launches:
            pairs = []
            for _ in range(steps):
                probe.flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                pairs.append((e0, e1))
            # Back to back: a call takes the host longer than the GPU, so the launches are
            # queued behind a few cache-evicting reads (each ~0.3 ms of GPU time, enough
            # for about eight calls) and the GPU never waits for the host between them.
            for _ in range(2 + steps // 8):
                probe.flush()
            fn()  # untimed: brings the operands back into the caches
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(float(np.median([a.elapsed_time(b) for a, b in pairs])) / 1000.0)
            warm.append(e0.elapsed_time(e1) / 1000.0 / steps)
        return cold, warm

    # the split-K form (the shared expert's own, through its workspace), then the
    # single-pass form for comparison
    (gu, dn), (gu_w, dn_w) = timed(se.workspace)
    (gu1, dn1), _ = timed(None)
    # the down projection as the layer runs it: its split-K partials alone, their
    # reduction done by the combine (moe_combine_partials)
    part = se.workspace.view(torch.float32)
    pairs = []
    for _ in range(steps):
        probe.flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        hip.moe_dense_gemm_bf16_partials(act, se.down_w, part)
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    dn_part = float(np.median([a.elapsed_time(b) for a, b in pairs])) / 1000.0

    def roof(name, secs, wbytes, in_bytes, out_bytes, flops):
        nbytes = wbytes + in_bytes + out_bytes
        t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
        if t_hbm >= t_mfma:
            ach, peak, unit, bound = nbytes / secs / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
        else:
            ach, peak, unit, bound = flops / secs / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        return {"kernel": name, "us": round(secs * 1e6, 2), "bound": bound,
                "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "alg_bytes_per_launch": int(nbytes),
                "TFLOPs": round(flops / secs / 1e12, 2)}

    return {"rows": rows, "inter": inter, "hidden": hidden,
            "gate_up_swiglu": roof("moe_dense_gate_up_swiglu_bf16", gu, 2 * inter * hidden * 2,
                                   rows * hidden * 2, rows * inter * 2,
                                   2.0 * rows * 2 * inter * hidden),
            "down": roof("moe_dense_gemm_bf16", dn, hidden * inter * 2, rows * inter * 2,
                         rows * hidden * 2, 2.0 * rows * hidden * inter),
            "down_partials_us": round(dn_part * 1e6, 2),
            "down_partials_note": ("moe_dense_gemm_bf16_partials alone: the layer's form, whose "
                                   "split-K reduction runs inside the combine "
                                   "(moe_combine_partials), which then reads "
                                   f"{4 * hip.moe_dense_splitk_ways(rows, inter)} bytes of "
                                   "partials per shared-term element instead of 2"),
            "total_us": round((gu + dn) * 1e6, 2), "form": "split-K (workspace)",
            "timing": "each launch after a 2 GiB cache-evicting read, median",
            "mall_warm_us": {"gate_up_swiglu": round(gu_w * 1e6, 2),
                             "down": round(dn_w * 1e6, 2)},
            "single_pass_us": {"gate_up_swiglu": round(gu1 * 1e6, 2),
                               "down": round(dn1 * 1e6, 2)}}


def time_decode_leg(hip, torch, steps, probe):
    """The decode / verify path on the small-M workload (8 rows over 256 experts, experts
    [128, 256) absent), timed per stage with HIP events: the union path (moe_row_union ->
    union GEMV gate_up with the SwiGLU -> union GEMV down -> combine) and the sorted path
    (moe_align_zero -> grouped GEMMs -> combine) on the same rows. Its weights (0.68 GB)
    would partly stay in the 256 MB last-level cache from one step to the next, so every
    timed step follows a cache-evicting stream outside its events; times are medians over
    the steps. GB/s is unique weight bytes (live experts, both projections) per step."""
    import workloads as wl

    w = wl.WORKLOADS["small_m"]
    gt, dt, ids, wts, x, ids_host = upload_workload(hip, w, torch)
    rows, mi, hidden, top_k = w.rows, w.moe_intermediate, w.hidden, w.top_k
    s = rows * top_k
    ws = hip.Workspace(rows, top_k, w.num_experts, hidden, mi)
    dws = hip.DecodeWorkspace(rows, top_k, hidden, mi)
    out = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    u_slot = dws.u_slot[:s * rows]
    active = dict(active_experts=ws.active_experts, counters=ws.counters)
    n_gu, k_gu = wl.gate_up_shape(w)
    n_dn, k_dn = wl.down_shape(w)
    live = sorted({int(e) for e in ids_host.reshape(-1) if not w.is_null(int(e))})
    wbytes = len(live) * (proj_bytes(n_gu, k_gu) + proj_bytes(n_dn, k_dn))
    gu_alg = (len(live) * proj_bytes(n_gu, k_gu) + rows * hidden * 2
              + int(sum(1 for e in ids_host.reshape(-1) if not w.is_null(int(e)))) * mi * 2)
    paths = {
        "union": [
            # experts absent from the down table are left out of the union (the combine
            # skips their slots): no zero-first step on this path
            ("moe_row_union", lambda: hip.moe_row_union(ids, w.num_experts, dws.u_eid, u_slot,
                                                        dws.slot_perm, dws.counters,
                                                        present=dt)),
            ("gemv_union_gate_up_swiglu", lambda: hip.moe_w4a16_gemv_union_swiglu(
                x, gt, dws.u_eid, u_slot, dws.act, w.limit, rows, top_k)),
            ("gemv_union_down", lambda: hip.moe_w4a16_gemv_union(
                dws.act, dt, dws.u_eid, u_slot, dws.expert_out, rows, top_k, a_per_slot=True)),
            ("moe_combine", lambda: hip.moe_combine(dws.expert_out[:s], dws.slot_perm[:s], wts,
                                                    out))],
        "sorted": [
            ("moe_align_zero", lambda: hip.moe_align(ids, w.num_experts, ws.sorted_token_ids,
                                                     ws.sorted_expert_ids, ws.expert_offsets,
                                                     ws.token_to_perm, ws.active_experts,
                                                     ws.counters, zero=ws.expert_out[:s])),
            ("grouped_gemm_gate_up_swiglu", lambda: hip.moe_w4a16_grouped_gemm_swiglu(
                x, gt, ws.expert_offsets, ws.act, w.limit, ws.sorted_token_ids, max_rows=s,
                **active)),
            ("grouped_gemm_down", lambda: hip.moe_w4a16_grouped_gemm(
                ws.act, dt, ws.expert_offsets, ws.expert_out, None, max_rows=s, **active)),
            ("moe_combine", lambda: hip.moe_combine(ws.expert_out[:s], ws.token_to_perm, wts,
                                                    out))],
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, stages in paths.items():
        for _ in range(3):
            for _, fn in stages:
                fn()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(steps)]
        for i in range(steps):
            probe.flush()
            for j, (_, fn) in enumerate(stages):
                ev[i][j].record(stream)
                fn()
            ev[i][len(stages)].record(stream)
        torch.cuda.synchronize()
        # medians: a host stall while the queue is empty (between a stage's start event
        # and its launch) lands in one step's times and would move a mean
        step_us = float(np.median([ev[i][0].elapsed_time(ev[i][len(stages)]) * 1000.0
                                   for i in range(steps)]))
        kus = {n: round(float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) * 1000.0
                                         for i in range(steps)])), 2)
               for j, (n, _) in enumerate(stages)}
        res[name] = {"step_us": round(step_us, 2), "GBps": round(wbytes / step_us / 1e3, 1),
                     "kernel_us": kus}
    def roof(kernel, us):
        achieved = gu_alg / us / 1e3
        return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "alg_bytes_per_launch": int(gu_alg), "avg_launch_us": us}

    # The union GEMV is what moe_layer_decode runs; the sorted path's grouped GEMM on the
    # same rows is reported beside it.
    return {"workload": w.name, "rows": rows, "live_experts": len(live),
            "unique_weight_bytes": int(wbytes),
            "timing": "each step after a 2 GiB cache-evicting read; medians over the steps",
            **res,
            "faster_path": min(res, key=lambda k: res[k]["step_us"]),
            "roofline": roof("moe_w4a16_gemv_union_swiglu (gate_up + SwiGLU)",
                             res["union"]["kernel_us"]["gemv_union_gate_up_swiglu"]),
            "roofline_sorted": roof("moe_w4a16_grouped_gemm_swiglu (gate_up + SwiGLU)",
                                    res["sorted"]["kernel_us"]["grouped_gemm_gate_up_swiglu"])}


def measure_workload(hip, torch, w, args, probe, steps: int, warmup: int):
    """Runs the step on workload ``w``: ``warmup`` untimed steps, untimed steps until the
    clock has settled, then exactly ``steps`` timed steps (one sub-chunk each, cycling
    through the workload's sub-chunks). Workloads whose unique weight bytes per step are
    under 1 GiB would stay partly in the 256 MB last-level cache between steps, so for
    them each timed step follows a cache-evicting stream outside the step's events and
    the step time is the mean of the per-step event times. Returns the measured fields,
    the stream, the first sub-chunk's rows and host routing (for the side legs)."""
    import workloads as wl

    t_gen = time.perf_counter()
    gt, dt, ids_all, wts_all, x_all, ids_host = upload_workload(hip, w, torch)
    print(f"bench: uploaded {w.name} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    rows = w.chunk
    mi, hidden = w.moe_intermediate, w.hidden
    ws = hip.Workspace(rows, w.top_k, w.num_experts, hidden, mi)
    out = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    n_chunks = w.n_chunks

    # Per-step work (for a multi-chunk workload each step runs one sub-chunk, cycling
    # through them).
    n_gu, k_gu = wl.gate_up_shape(w)
    n_dn, k_dn = wl.down_shape(w)
    single = bool(w.gemm_n)  # one grouped GEMM (no SwiGLU, down or combine)
    step_bytes, step_flops, gu_bytes_alg, dn_bytes_alg = [], [], [], []
    gu_w, dn_w, gu_fl, dn_fl = [], [], [], []
    for c in range(n_chunks):
        ids_c = ids_host[c * rows:(c + 1) * rows]
        cnt = np.bincount(ids_c.reshape(-1), minlength=w.num_experts)
        live = [e for e in range(w.num_experts) if cnt[e] > 0 and not w.is_null(e)]
        slots_live = int(sum(cnt[e] for e in live))
        dn_proj = proj_bytes(n_dn, k_dn) if not single else 0
        wb = len(live) * (proj_bytes(n_gu, k_gu) + dn_proj)
        step_bytes.append(wb)
        step_flops.append(2.0 * slots_live * (n_gu * k_gu + (0 if single else n_dn * k_dn)))
        gu_w.append(len(live) * proj_bytes(n_gu, k_gu))
        dn_w.append(len(live) * dn_proj)
        gu_fl.append(2.0 * slots_live * n_gu * k_gu)
        dn_fl.append(0.0 if single else 2.0 * slots_live * n_dn * k_dn)
        # gate_up launch, algorithmic bytes: touched weights + the activation rows read
        # once + the output rows written once (the SwiGLU output when fused, else the
        # gate_up values) + routing metadata
        out_cols = n_gu if (args.unfused or single) else mi
        gu_bytes_alg.append(len(live) * proj_bytes(n_gu, k_gu) + rows * hidden * 2
                            + slots_live * out_cols * 2 + (w.num_experts + 1) * 4
                            + rows * w.top_k * 4)
        # down launch: touched weights + the activation rows in + expert_out rows out
        dn_bytes_alg.append(len(live) * dn_proj + slots_live * (mi + hidden) * 2
                            + (w.num_experts + 1) * 4)

    stream = torch.cuda.current_stream()
    need_zero = dt is not None and not all(dt.present)
    se = None
    if (args.with_shared or not args.no_shared) and w.moe_intermediate > 0:
        sg, su, sd = (torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
                      for b in wl.shared_expert(w))
        se = hip.SharedExpert(sg, su, sd, rows)
    shared_out = [None]
    cur_chunk = [0]
    logits_all = (torch.from_numpy(wl.router_logits(w)).cuda() if args.device_router else None)
    s = rows * w.top_k

    # The stages of one step, in order; each is timed with HIP events on the stream.
    def st_router(x, ids, wts):
        c = cur_chunk[0]
        hip.moe_router_topk(logits_all[c * rows:(c + 1) * rows], w.top_k, ws.topk_ids,
                            ws.topk_weights)

    def st_align(x, ids, wts):
        # null down entries: their rows must read as zero in the combine, zeroed in the
        # sort's launch (moe_align_zero)
        hip.moe_align(ids, w.num_experts, ws.sorted_token_ids, ws.sorted_expert_ids,
                      ws.expert_offsets, ws.token_to_perm, ws.active_experts, ws.counters,
                      zero=ws.expert_out[:s] if need_zero else None)

    c_single = (torch.empty((max(s, 1), n_gu), dtype=torch.bfloat16, device="cuda")
                if single else None)

    active = dict(active_experts=ws.active_experts, counters=ws.counters)

    def st_single(x, ids, wts):
        hip.moe_w4a16_grouped_gemm(x, gt, ws.expert_offsets, c_single, ws.sorted_token_ids,
                                   max_rows=s, **active)

    def st_gate_up(x, ids, wts):
        hip.moe_w4a16_grouped_gemm(x, gt, ws.expert_offsets, ws.gate_up, ws.sorted_token_ids,
                                   max_rows=s, **active)

    def st_swiglu(x, ids, wts):
        hip.swiglu_clamp(ws.gate_up[:s, :mi], ws.gate_up[:s, mi:2 * mi], ws.act[:s], w.limit)

    def st_gate_up_swiglu(x, ids, wts):
        hip.moe_w4a16_grouped_gemm_swiglu(x, gt, ws.expert_offsets, ws.act, w.limit,
                                          ws.sorted_token_ids, max_rows=s, **active)

    def st_down(x, ids, wts):
        hip.moe_w4a16_grouped_gemm(ws.act, dt, ws.expert_offsets, ws.expert_out, None,
                                   max_rows=s, **active)

    def st_shared(x, ids, wts):  # split-K: the down reduction runs in the combine
        shared_out[0] = se.for_combine(x, w.limit)

    def st_combine(x, ids, wts):
        hip.moe_combine(ws.expert_out[:s], ws.token_to_perm, wts, out, shared_out[0])

    # The decode path: the union of the rows' experts, outputs by (row, slot).
    dws = hip.DecodeWorkspace(rows, w.top_k, hidden, mi) if args.decode else None

    def st_union(x, ids, wts):  # absent experts' slots left out: no zero-first step
        hip.moe_row_union(ids, w.num_experts, dws.u_eid, dws.u_slot[:s * rows], dws.slot_perm,
                          dws.counters, present=dt if need_zero else None)

    def st_union_gate_up(x, ids, wts):
        hip.moe_w4a16_gemv_union_swiglu(x, gt, dws.u_eid, dws.u_slot[:s * rows], dws.act,
                                        w.limit, rows, w.top_k)

    def st_union_down(x, ids, wts):
        hip.moe_w4a16_gemv_union(dws.act, dt, dws.u_eid, dws.u_slot[:s * rows],
                                 dws.expert_out, rows, w.top_k, a_per_slot=True)

    def st_union_combine(x, ids, wts):
        hip.moe_combine(dws.expert_out[:s], dws.slot_perm[:s], wts, out, shared_out[0])

    stages = [("moe_router_topk", st_router)] if args.device_router else []
    if args.decode:
        stages.append(("moe_row_union", st_union))
        stages += [("gemv_union_gate_up_swiglu", st_union_gate_up),
                   ("gemv_union_down", st_union_down)]
        gu_name, dn_name = "gemv_union_gate_up_swiglu", "gemv_union_down"
    elif single:
        stages += [("moe_align", st_align), ("grouped_gemm", st_single)]
        gu_name, dn_name = "grouped_gemm", None
    else:
        stages.append(("moe_align_zero" if need_zero else "moe_align", st_align))
        if args.unfused:
            stages += [("grouped_gemm_gate_up", st_gate_up), ("swiglu_clamp", st_swiglu)]
            gu_name = "grouped_gemm_gate_up"
        else:
            stages.append(("grouped_gemm_gate_up_swiglu", st_gate_up_swiglu))
            gu_name = "grouped_gemm_gate_up_swiglu"
        stages.append(("grouped_gemm_down", st_down))
        dn_name = "grouped_gemm_down"
    if args.with_shared:
        stages.append(("shared_expert", st_shared))
        # its BF16 weights are unique weight bytes of the step too
        for c in range(n_chunks):
            step_bytes[c] += 3 * mi * hidden * 2
            step_flops[c] += 2.0 * rows * 3 * mi * hidden
    if not single:
        stages.append(("moe_combine", st_union_combine if args.decode else st_combine))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    flush = max(step_bytes) < (1 << 30)

    def step(i, events=None):
        c = i % n_chunks
        cur_chunk[0] = c
        sl = slice(c * rows, (c + 1) * rows)
        ids, wts, x = ids_all[sl], wts_all[sl], x_all[sl]
        if args.device_router:  # the router writes the workspace's ids and weights
            ids, wts = ws.topk_ids, ws.topk_weights
        for j, (_, fn) in enumerate(stages):
            if events:
                events[j].record(stream)
            fn(x, ids, wts)
        if events:
            events[len(stages)].record(stream)

    t_warm = time.perf_counter()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Clock settle: the GPU needs some tens of milliseconds of load to reach its steady
    # clock (measured: the first ~25 steps of 1 ms run 1.30 -> 1.02 ms). After the W
    # warm-up steps, further untimed steps run until at least SETTLE_S of warm-up has
    # passed, so the timed steps measure the steady state. Their count is reported.
    settle = 0
    t_w = time.perf_counter() - t_warm
    while t_w < SETTLE_S and settle < 1000:
        for _ in range(5):
            step(warmup + settle)
            settle += 1
        torch.cuda.synchronize()
        t_w = time.perf_counter() - t_warm
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        if flush:
            probe.flush()
        step(i, ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = [n for n, _ in stages]
    per = {n: [] for n in names}
    step_ms = []
    for i in range(steps):
        for j, n in enumerate(names):
            per[n].append(ev[i][j].elapsed_time(ev[i][j + 1]))
        step_ms.append(ev[i][0].elapsed_time(ev[i][len(stages)]))
    kern_us = {n: round(1000.0 * float(np.mean(v)), 2) for n, v in per.items()}
    gpu_ms = float(np.sum(step_ms)) if flush else start.elapsed_time(end)
    ms_per_step = gpu_ms / steps

    chunk_of = [i % n_chunks for i in range(steps)]
    total_bytes = sum(step_bytes[c] for c in chunk_of)
    total_flops = sum(step_flops[c] for c in chunk_of)
    value = total_bytes / (gpu_ms / 1000.0) / 1e9
    tflops = total_flops / (gpu_ms / 1000.0) / 1e12

    gu_s = np.array(per[gu_name]) / 1000.0
    dn_s = np.array(per[dn_name]) / 1000.0 if dn_name else None
    gu_alg = np.array([gu_bytes_alg[c] for c in chunk_of])
    achieved = float(np.mean(gu_alg) / np.mean(gu_s) / 1e9)

    def gemm_line(wb, fl, secs, alg=None):
        t = float(np.mean(secs))
        d = {"us": round(t * 1e6, 2),
             "weight_GBps": round(float(np.mean([wb[c] for c in chunk_of])) / t / 1e9, 1),
             "TFLOPs": round(float(np.mean([fl[c] for c in chunk_of])) / t / 1e12, 2)}
        if alg is not None:
            d["alg_GBps"] = round(float(np.mean([alg[c] for c in chunk_of])) / t / 1e9, 1)
        return d

    per_gemm = {"gate_up": gemm_line(gu_w, gu_fl, gu_s, gu_bytes_alg)}
    if dn_name:
        per_gemm["down"] = gemm_line(dn_w, dn_fl, dn_s, dn_bytes_alg)
    kernel_label = ("moe_w4a16_gemv_union_swiglu (gate_up + SwiGLU)" if args.decode
                    else "moe_w4a16_grouped_gemm (single GEMM)" if single
                    else "moe_w4a16_grouped_gemm (gate_up)" if args.unfused
                    else "moe_w4a16_grouped_gemm_swiglu (gate_up + SwiGLU)")
    roofline = {"kernel": kernel_label, "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kernel_label, w.name),
                "avg_launch_us": round(float(np.mean(gu_s)) * 1e6, 2),
                "alg_bytes_per_launch": int(np.mean(gu_alg))}
    fields = {
        "value": round(value, 2), "ms_per_step": round(ms_per_step, 4), "settle_steps": settle,
        "tflops": round(tflops, 2),
        "step_ms_p10_p90": [round(float(np.percentile(step_ms, 10)), 4),
                            round(float(np.percentile(step_ms, 90)), 4)],
        "gemms": per_gemm, "kernel_us": kern_us, "roofline": roofline,
        "unique_weight_bytes_per_step": int(np.mean([step_bytes[c] for c in chunk_of])),
        "wall_s": round(wall, 4),
        "cache_flush_between_steps": bool(flush),
    }
    return fields, {"stream": stream, "se": se, "x_rows": x_all[:rows], "ids_host": ids_host}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the routed-MoE path runs on one GPU only (asked for --gpus {args.gpus}); "
              "splitting the experts across GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import grouped_nvfp4_w4a16_amd as hip
    import workloads as wl

    if not os.path.exists(hip.LIB_PATH):
        from grouped_nvfp4_w4a16_amd import build as builder
        builder.build()
    hip.load()
    torch.cuda.set_device(0)
    w = wl.WORKLOADS[args.workload]
    if args.with_shared and w.moe_intermediate == 0:
        print(f"bench.py: {w.name} is a single GEMM; it has no shared expert", file=sys.stderr)
        sys.exit(2)
    if args.decode and (w.chunk > hip.UNION_MAX_ROWS or w.moe_intermediate == 0):
        print(f"bench.py: the decode path takes layer workloads of at most "
              f"{hip.UNION_MAX_ROWS} rows per step ({w.name} has {w.chunk})", file=sys.stderr)
        sys.exit(2)
    if w.gemm_n and (args.decode or args.unfused or args.device_router):
        print(f"bench.py: {w.name} is a single grouped GEMM step (align + GEMM)",
              file=sys.stderr)
        sys.exit(2)

    probe = HbmProbe(hip, torch)
    ceiling = probe.ceiling()
    print(f"bench: HBM read ceiling {ceiling['GBps']} GB/s", file=sys.stderr, flush=True)

    fields, side = measure_workload(hip, torch, w, args, probe, args.steps, args.warmup)
    fields["roofline"]["ceiling_GBps"] = ceiling["GBps"]
    fields["roofline"]["frac_of_ceiling"] = round(fields["roofline"]["achieved"] /
                                                  ceiling["GBps"], 4)

    shared = None
    if side["se"] is not None and not args.with_shared:
        shared = time_shared_expert(side["se"], side["x_rows"], w, args.steps, torch,
                                    side["stream"], probe)

    decode = None
    if w.name == "prefill_subchunk" and not args.no_decode and not args.decode:
        decode = time_decode_leg(hip, torch, args.steps, probe)

    long_leg = None
    if w.name == "prefill_subchunk" and not args.no_long and not args.decode:
        # skewed routing: the 16 sub-chunks of the long prefill, each a step, two passes
        wl_long = wl.WORKLOADS["long_prefill"]
        side = None
        long_args = argparse.Namespace(**{**vars(args), "with_shared": False, "no_shared": True,
                                          "device_router": False})
        lf, _ = measure_workload(hip, torch, wl_long, long_args, probe,
                                 2 * wl_long.n_chunks, args.warmup)
        lf["roofline"]["ceiling_GBps"] = ceiling["GBps"]
        lf["roofline"]["frac_of_ceiling"] = round(lf["roofline"]["achieved"] / ceiling["GBps"], 4)
        long_leg = {"workload": wl_long.name, "rows_per_step": wl_long.chunk,
                    "sub_chunks": wl_long.n_chunks, "routing": wl_long.routing,
                    "steps": 2 * wl_long.n_chunks, "unit": "GB/s",
                    "frac_of_peak": round(lf["value"] / HBM_PEAK_GBS, 4), **lf}

    if args.copy_probe:  # a plain copy of known size, for scaling HBM counters
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        ids_host = wl.routing(w)[0]
        cpu = cpu_baseline(w, ids_host[:w.chunk])

    mi, hidden = w.moe_intermediate, w.hidden
    line = {
        "metric": METRIC, "value": fields["value"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": fields["settle_steps"],
        "ms_per_step": fields["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded NVFP4 weights and BF16 N(0,1) activations, random init)",
        "config": {"workload": w.name, "rows_per_step": w.chunk, "experts": w.num_experts,
                   "top_k": w.top_k, "hidden": hidden, "moe_intermediate": mi,
                   "routing": w.routing, "weight_format": "NVFP4 (E2M1 + E4M3/16 + FP32)",
                   "parallelism": "single GPU"},
        "tflops": fields["tflops"],
        "step_ms_p10_p90": fields["step_ms_p10_p90"],
        "frac_of_peak": round(fields["value"] / HBM_PEAK_GBS, 4),
        "frac_of_ceiling": round(fields["value"] / ceiling["GBps"], 4),
        "hbm_ceiling": ceiling,
        "gemms": fields["gemms"],
        "gate_up_fused_swiglu": not args.unfused,
        "device_router": bool(args.device_router),
        "shared_expert_in_step": bool(args.with_shared),
        "shared_expert": shared,
        "decode_path": bool(args.decode),
        "decode": decode,
        "long_prefill": long_leg,
        "unique_weight_bytes_per_step": fields["unique_weight_bytes_per_step"],
        "cache_flush_between_steps": fields["cache_flush_between_steps"],
        "wall_s": fields["wall_s"],
        "kernel_us": fields["kernel_us"],
        "roofline": fields["roofline"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
