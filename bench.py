#!/usr/bin/env python3
"""Benchmark of the layer-boundary path on one MI355X.

A step is one fused boundary at the prefill fused-batch cap: publish P = 8
bf16 partials [2048, 4096] and fold them into the residual with the RMSNorm
read (bnd_fold_norm). Inputs and outputs rotate over sets that together exceed
1 GiB, so the 256 MB Infinity Cache cannot serve a step from a previous one.
`value` is tokens/s over the K timed steps (wall clock between device
synchronisations); the roofline block reports the kernel's algorithmic bytes
over its average duration from HIP events recorded on the launch stream.

Secondary measurements (the quantised read, the MoE finalize over all rows
and over the reduce-scatter share, complete_only, snapshot and add_to_output,
the unfused fallback beside the fused fold, a variable-size share, the decode
chain eager and as a HIP graph next to an empty kernel's launch cost, and a
streaming kernel with the fold's 9:2 read:write mix and no arithmetic as an
achievable-bandwidth context figure) and the oracle's CPU baseline go into the
same JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused fold+RMSNorm tokens/s and achieved HBM GB/s (% of peak), T=2048 H=4096"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
ROTATE_BYTES = 1 << 30          # >= 4x the 256 MB Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["kernels.h", "launch.h", "k_partials.hip", "k_moe.hip", "k_read.hip",
                  "k_complete.hip", "k_wave.hip", "k_wave_complete.hip", "host.cpp"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# C++ comments, string and character literals, in source order: the literals are matched so that
# a "//" inside one is not taken for a comment
_CXX_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_text(src: str) -> str:
    """The source with comments removed and whitespace runs collapsed: what the compiler sees."""
    src = _CXX_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    """sha256 of the kernel and launch sources' code (comments and layout excluded)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "reduce_residual_rmsnorm_bnd_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from the committed counter summary, if it matches these kernels."""
    path = os.path.join(PROFILES, "traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^\| {re.escape(workload)} \|[^\n]*\| ([0-9.]+) \|$", text, flags=re.M)
    return float(m.group(1)) if m else None


# --------------------------------------------------------------------------
# timing harness
# --------------------------------------------------------------------------

class HipEvents:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def elapsed_s(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e-3

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def nearest_rank(sorted_values, q: float) -> float:
    """The q-quantile of an ascending list by the nearest-rank rule."""
    n = len(sorted_values)
    return sorted_values[min(n - 1, max(0, math.ceil(q * n) - 1))]


def sampling_plan(steps: int):
    """The timed launches that record their own start/stop events: every `every`-th one from the
    first, and the last, with `every` = steps - 1 clamped to 1..32, so that a run of any length
    has both ends of its timed region on the device clock, a short run (up to 33 steps) samples
    only those two, and a long one one launch in 32 (the event packets add a few microseconds to
    each sampled launch). Returns (every, the sampled step indices, ascending)."""
    if steps < 1:
        raise ValueError(f"need at least one timed step, not {steps}")
    every = max(1, min(32, steps - 1))
    sampled = list(range(0, steps, every))
    if sampled[-1] != steps - 1:
        sampled.append(steps - 1)
    return every, sampled


class Timed:
    """Runs step(i, start, stop) K times after W warmup steps. The launches that
    `sampling_plan` names (the first, the last and every `every`-th) record
    start/stop events from their own dispatch (bnd_time_next_launch ->
    hipExtLaunchKernel) on the stream they run on; the event packets add a
    few microseconds of queue gap each, so sampling a fraction of the launches
    keeps the timed region close to an unobserved run.

    Per-launch figures from those events:
      span      the first launch's start to the last launch's stop over K: the
                device time per launch of the whole timed region, gaps and
                event packets included; it reads high when the host's issue
                rate, not the kernel, sets the pace (short kernels);
      dispatch  a sampled launch's own start-to-stop: its start is taken while
                the previous kernel's last waves still drain, so it reads high
                when launches run back to back;
      interval  start to start of consecutive sampled launches over the
                launches between them (reported only).
    The kernel time is the smaller of the span and dispatch means (the dispatch
    mean alone for a single step).

    `sync` waits for the device; `events(n)` makes n event handles (`.ev[i]`,
    `.elapsed_s(a, b)`, `.close()`)."""

    def __init__(self, sync, events=None):
        self.sync = sync
        self.events = events if events is not None else HipEvents

    def run(self, step, n_sets: int, warmup: int, steps: int):
        every, sampled = sampling_plan(steps)
        for i in range(warmup):
            step(i % n_sets, None, None)
        ev = self.events(2 * len(sampled))
        try:
            slot = {i: n for n, i in enumerate(sampled)}
            self.sync()
            t0 = time.perf_counter()
            for i in range(steps):
                n = slot.get(i)
                if n is None:
                    step((warmup + i) % n_sets, None, None)
                else:
                    step((warmup + i) % n_sets, ev.ev[2 * n], ev.ev[2 * n + 1])
            self.sync()
            wall = time.perf_counter() - t0
            durs = sorted(ev.elapsed_s(2 * n, 2 * n + 1) for n in range(len(sampled)))
            gaps = sorted(ev.elapsed_s(2 * n, 2 * n + 2) / (sampled[n + 1] - sampled[n])
                          for n in range(len(sampled) - 1))
            span = ev.elapsed_s(0, 2 * len(sampled) - 1) / steps
        finally:
            ev.close()
        dispatch = sum(durs) / len(durs)
        interval = sum(gaps) / len(gaps) if gaps else None
        quant = lambda v, q: nearest_rank(v, q) if v else None
        return {
            "wall_s": wall,
            "kernel_s": min(dispatch, span) if steps > 1 else dispatch,
            "span_s": span,
            "dispatch_event_mean_s": dispatch,
            "dispatch_event_median_s": durs[len(durs) // 2],
            "dispatch_event_p10_s": nearest_rank(durs, 0.10),
            "dispatch_event_p90_s": nearest_rank(durs, 0.90),
            "interval_median_s": gaps[len(gaps) // 2] if gaps else None,
            "interval_p10_s": quant(gaps, 0.10),
            "interval_p90_s": quant(gaps, 0.90),
            "dispatch_events": len(durs),
            "interval_mean_s": interval,
            "intervals": len(gaps),
            "sample_every": every,
        }


def launch_desc(bnd) -> dict:
    """The shape of this thread's last launch through the library, as the bench reports it."""
    rows, threads, vpt, one_wave = bnd.last_launch_shape()
    return {"workgroups": rows, "threads": threads, "vectors_per_thread": vpt,
            "rows_per_workgroup": 1, "one_wavefront_per_row": one_wave,
            "ring_depth": bnd.last_launch_ring_depth()}


def us(seconds):
    """Seconds to microseconds, None passing through."""
    return None if seconds is None else seconds * 1e6


def kernel_fields(t, bnd) -> dict:
    """Per-launch figures of a timed run, with the launch shape it used."""
    return {"launch": launch_desc(bnd), "kernel_us": us(t["kernel_s"]),
            "span_us_per_launch": us(t["span_s"]),
            "dispatch_event_mean_us": us(t["dispatch_event_mean_s"]),
            "interval_us_per_launch": us(t["interval_mean_s"]),
            **spread_fields(t)}


def spread_fields(t) -> dict:
    """Median, p10 and p90 of a timed run's sampled launches (start to stop) and of its per-launch
    intervals, in microseconds."""
    return {f"{k}_{q}_us": us(t[f"{k}_{q}_s"])
            for k in ("dispatch_event", "interval") for q in ("median", "p10", "p90")}


def fold_case(torch, bnd, d, n_sets, fp8=False, row_begin=0, rows=None):
    """Device sets for a partials fold; returns (step function, algorithmic bytes per launch)."""
    T, H, P = d["T"], d["H"], d["P"]
    rows = T - row_begin if rows is None else rows
    dev = torch.device("cuda:0")
    L = bnd.lib()
    base_parts = [c.to(dev) for c in d["partials"]]
    base_res = d["residual"][row_begin:row_begin + rows].to(dev)
    w = d["weight"].to(dev)
    sets = []
    for s_i in range(n_sets):
        parts = base_parts if s_i == 0 else [c.clone() for c in base_parts]
        res = base_res.clone()
        st = bnd.bnd_stream_create(T, H, res, row_begin, rows)
        bnd.bnd_written(st, res)
        if fp8:
            out = (torch.empty(rows, H, dtype=torch.uint8, device=dev),
                   torch.empty(rows, dtype=torch.float32, device=dev))
        else:
            out = (torch.empty(rows, H, dtype=torch.bfloat16, device=dev),)
        arr = (ctypes.c_void_p * P)(*[c.data_ptr() for c in parts])
        sets.append((st, parts, res, out, arr))
    owed = ctypes.c_uint64()
    eps = ctypes.c_float(d["eps"])
    wptr = ctypes.c_void_p(w.data_ptr())
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(i, ev0, ev1):
        st, parts, res, out, arr = sets[i]
        rc = L.bnd_publish_partials(st.handle, arr, P, H, ctypes.byref(owed))
        if ev0 is not None:
            rc |= L.bnd_time_next_launch(ev0, ev1)
        if fp8:
            rc |= L.bnd_fold_norm_quant_fp8(st.handle, owed.value, wptr, eps,
                                            ctypes.c_void_p(out[0].data_ptr()), H,
                                            ctypes.c_void_p(out[1].data_ptr()), hs)
        else:
            rc |= L.bnd_fold_norm(st.handle, owed.value, wptr, eps,
                                  ctypes.c_void_p(out[0].data_ptr()), H, hs)
        if rc:
            raise RuntimeError(L.bnd_last_error().decode())

    el = rows * H
    read = (P * el + el) * 2 + H * 4
    write = el * 2 + (el + rows * 4 if fp8 else el * 2)
    keep = (sets, base_parts, w)
    return step, read + write, keep


def moe_case(torch, bnd, d, n_sets, row_begin=0, rows=None, terminal_gemma=False):
    """MoE finalize sets; with terminal_gemma the streams use the Gemma weight form and each
    step releases the stream after the finalize (the final norm of a stack), then marks the
    residual written again for the next step (host-only calls)."""
    T, H, k = d["T"], d["H"], d["k"]
    rows = T - row_begin if rows is None else rows
    dev = torch.device("cuda:0")
    L = bnd.lib()
    E0 = d["expert_rows"].to(dev)
    idx0 = d["idx"].to(dev)
    gate0 = d["gate"].to(dev)
    res0 = d["residual"][row_begin:row_begin + rows].to(dev)
    w = d["weight"].to(dev)
    sets = []
    for s_i in range(n_sets):
        E = E0 if s_i == 0 else E0.clone()
        res = res0.clone()
        st = bnd.bnd_stream_create(T, H, res, row_begin, rows)
        if terminal_gemma:
            bnd.bnd_stream_set_norm_form(st, bnd.BND_NORM_GEMMA)
        bnd.bnd_written(st, res)
        y = torch.empty(rows, H, dtype=torch.bfloat16, device=dev)
        sets.append((st, E, res, y))
    owed = ctypes.c_uint64()
    eps = ctypes.c_float(d["eps"])
    wptr = ctypes.c_void_p(w.data_ptr())
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    iptr, gptr = ctypes.c_void_p(idx0.data_ptr()), ctypes.c_void_p(gate0.data_ptr())

    def step(i, ev0, ev1):
        st, E, res, y = sets[i]
        rc = L.bnd_publish_moe(st.handle, ctypes.c_void_p(E.data_ptr()), E.shape[0], H, iptr, gptr, k,
                               ctypes.byref(owed))
        if ev0 is not None:
            rc |= L.bnd_time_next_launch(ev0, ev1)
        rc |= L.bnd_moe_finalize_fold_norm(st.handle, owed.value, wptr, eps,
                                           ctypes.c_void_p(y.data_ptr()), H, hs)
        if terminal_gemma:
            rc |= L.bnd_take_output(st.handle)
            rc |= L.bnd_written(st.handle, ctypes.c_void_p(res.data_ptr()), H)
        if rc:
            raise RuntimeError(L.bnd_last_error().decode())

    el = rows * H
    read = rows * k * H * 2 + el * 2 + H * 4 + rows * k * 8
    write = el * 4
    return step, read + write, (sets, idx0, gate0, w)


def aux_case(torch, bnd, d, n_sets, kind):
    """snapshot, add_to_output or complete_only over the prefill workload: each step publishes
    the partials, runs the call into a separate output, then marks the residual written again
    (host-only) so the next step can publish. kind "unfused" is the fallback of a refused fused
    fold, two launches per step: complete_only into a bf16 buffer, then a one-source fold_norm of
    that buffer (the stream ends Written)."""
    T, H, P = d["T"], d["H"], d["P"]
    dev = torch.device("cuda:0")
    L = bnd.lib()
    base_parts = [c.to(dev) for c in d["partials"]]
    base_res = d["residual"].to(dev)
    extra0 = d["residual"].to(dev)  # any [T, H] bf16 tensor serves as the extra contribution
    w = d["weight"].to(dev)
    sets = []
    for s_i in range(n_sets):
        parts = base_parts if s_i == 0 else [c.clone() for c in base_parts]
        res = base_res.clone()
        extra = extra0.clone() if kind == "add_to_output" else None
        st = bnd.bnd_stream_create(T, H, res)
        bnd.bnd_written(st, res)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        y = torch.empty(T, H, dtype=torch.bfloat16, device=dev) if kind == "unfused" else None
        arr = (ctypes.c_void_p * P)(*[c.data_ptr() for c in parts])
        sets.append((st, parts, res, extra, out, y, arr))
    owed = ctypes.c_uint64()
    new = ctypes.c_uint64()
    eps = ctypes.c_float(d["eps"])
    wptr = ctypes.c_void_p(w.data_ptr())
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(i, ev0, ev1):
        st, parts, res, extra, out, y, arr = sets[i]
        rc = L.bnd_publish_partials(st.handle, arr, P, H, ctypes.byref(owed))
        if ev0 is not None:
            rc |= L.bnd_time_next_launch(ev0, ev1)
        if kind == "snapshot":
            rc |= L.bnd_snapshot(st.handle, owed.value, ctypes.c_void_p(out.data_ptr()), H, hs)
        elif kind == "add_to_output":
            rc |= L.bnd_add_to_output(st.handle, owed.value, ctypes.c_void_p(extra.data_ptr()), H,
                                      ctypes.c_void_p(out.data_ptr()), H, ctypes.byref(new), hs)
        else:  # complete_only, or the first launch of the unfused fallback
            rc |= L.bnd_complete_only(st.handle, owed.value, ctypes.c_void_p(out.data_ptr()), H,
                                      ctypes.byref(new), hs)
        if kind == "unfused":
            rc |= L.bnd_fold_norm(st.handle, new.value, wptr, eps, ctypes.c_void_p(y.data_ptr()), H, hs)
        else:
            rc |= L.bnd_written(st.handle, ctypes.c_void_p(res.data_ptr()), H)
        if rc:
            raise RuntimeError(L.bnd_last_error().decode())

    el = T * H
    reads = {"snapshot": P + 1, "add_to_output": P + 1, "complete_only": P}
    # the unfused pair moves the fused fold's bytes plus one bf16 [T, H] write and its re-read
    nbytes = ((P + 1) * el * 2 + 2 * el * 2 + H * 4 + 2 * el * 2 if kind == "unfused"
              else reads[kind] * el * 2 + el * 2)
    return step, nbytes, (sets, base_parts, w)


def decode_chain(torch, bnd, workloads, T, reps_eager, reps_graph, H=4096, P=4, n_b=96):
    """1 enter + 96 folds with fresh partials per boundary: eager and HIP-graph us/boundary."""
    dev = torch.device("cuda:0")
    start = workloads.decode_start(T, H)
    x_in = start["x_in"].to(dev)
    w0 = start["weight"].to(dev)
    bounds = []
    for b in range(n_b):
        d = workloads.decode_boundary(T, b, P, H)
        bounds.append(([c.to(dev) for c in d["partials"]], d["weight"].to(dev)))
    res = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    L = bnd.lib()
    arrs = [(ctypes.c_void_p * P)(*[c.data_ptr() for c in parts]) for parts, _ in bounds]
    wptrs = [ctypes.c_void_p(w.data_ptr()) for _, w in bounds]
    eps = ctypes.c_float(1e-6)
    owed = ctypes.c_uint64()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def chain(st):
        hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = L.bnd_take_output(st.handle)
        rc |= L.bnd_enter_norm(st.handle, ptr(x_in), H, ptr(w0), eps, ptr(y), H, hs)
        for b in range(n_b):
            rc |= L.bnd_publish_partials(st.handle, arrs[b], P, H, ctypes.byref(owed))
            rc |= L.bnd_fold_norm(st.handle, owed.value, wptrs[b], eps, ptr(y), H, hs)
        if rc:
            raise RuntimeError(L.bnd_last_error().decode())

    st = bnd.bnd_stream_create(T, H, res)
    for _ in range(3):
        chain(st)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps_eager):
        chain(st)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / (reps_eager * (n_b + 1))

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain(st)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        chain(st)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps_graph):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / (reps_graph * (n_b + 1))
    bytes_b = T * (P + 3) * H * 2 + H * 4
    return {"T": T, "us_per_boundary_eager": eager * 1e6, "us_per_boundary_graph": graph * 1e6,
            "tokens_per_s_graph": T / graph, "algorithmic_bytes_per_boundary": bytes_b,
            "GBps_graph": bytes_b / graph / 1e9}


def launch_floor(torch, n_launches=97, reps_eager=20, reps_graph=50, workgroups=1, threads=512, with_args=False):
    """An empty kernel (libboundary_ceiling.so) launched back to back as many times as the decode
    chain launches, eager and replayed from a HIP graph: the per-launch cost with no work, the
    floor under the decode boundary's time per launch. One 512-thread workgroup is the launch
    shape of a one-row fold at H = 4096. With `with_args` the empty kernel takes the boundary
    kernels' argument block and reads one field of it."""
    from reduce_residual_rmsnorm_bnd_amd import _build

    L = ctypes.CDLL(_build.CEILING_LIB_PATH)
    fn = L.bnd_ceiling_empty_args if with_args else L.bnd_ceiling_empty
    fn.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int

    def chain():
        hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(n_launches):
            if fn(workgroups, threads, hs):
                raise RuntimeError("empty kernel launch failed")

    for _ in range(3):
        chain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps_eager):
        chain()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / (reps_eager * n_launches)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        chain()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps_graph):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / (reps_graph * n_launches)
    out = {"launches": n_launches, "workgroups": workgroups, "threads": threads,
           "us_per_launch_eager": eager * 1e6, "us_per_launch_graph": graph * 1e6}
    if with_args:
        L.bnd_ceiling_args_bytes.restype = ctypes.c_int
        out["argument_bytes"] = L.bnd_ceiling_args_bytes()
    return out


def copy_ceiling(torch, n_bytes=1 << 30, reps=20):
    """A plain device copy of a 1 GiB buffer (torch's copy kernel), for context."""
    a = torch.empty(n_bytes // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    return {"bytes": 2 * n_bytes, "GBps": 2 * n_bytes / t / 1e9}


def back_to_back_us(torch, launch, n_sets: int, reps: int = 300, warmup: int = 20) -> float:
    """Mean time per launch of `reps` back-to-back launches, no per-launch events: events on
    torch's current stream (where the launches go) around the whole run."""
    for i in range(warmup):
        launch(i % n_sets)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        launch((warmup + i) % n_sets)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def stream_ceiling(torch, T: int, H: int, n_src: int, n_out: int, kernel_us: dict, byte_second: bool = False):
    """The arithmetic-free streaming kernel (libboundary_ceiling.so: n_src row reads and n_out row
    writes per row, the boundary kernels' rows, resources and cache policy) over rotating sets of
    [T, H] rows, for four launch shapes; beside it the boundary calls with the same mix, timed the
    same way (back-to-back launches) in the same process (`kernel_us`: name -> us). With
    `byte_second` the second output has one byte per element, as the fp8 read's codes."""
    from reduce_residual_rmsnorm_bnd_amd import _build

    L = ctypes.CDLL(_build.CEILING_LIB_PATH)
    vp = ctypes.c_void_p
    args = [ctypes.POINTER(vp), ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int, vp]
    L.bnd_ceiling_mix.argtypes = args
    L.bnd_ceiling_mix_byte_out1.argtypes = args
    mix = L.bnd_ceiling_mix_byte_out1 if byte_second else L.bnd_ceiling_mix
    if byte_second and n_out != 2:
        raise ValueError("a byte-wide second output needs two outputs")
    nbytes = (n_src + n_out) * T * H * 2 - (T * H if byte_second else 0)
    n_sets = max(2, -(-ROTATE_BYTES // nbytes))
    sets = []
    for _ in range(n_sets):
        bufs = [torch.zeros(T, H, dtype=torch.bfloat16, device="cuda:0") for _ in range(n_src + 1)]
        if n_out == 2:
            bufs.append(torch.zeros(T, H, dtype=torch.uint8 if byte_second else torch.bfloat16, device="cuda:0"))
        sets.append((bufs, (vp * n_src)(*[b.data_ptr() for b in bufs[:n_src]]), vp(bufs[n_src].data_ptr()),
                     vp(bufs[n_src + 1].data_ptr()) if n_out == 2 else vp()))
    stream = vp(torch.cuda.current_stream().cuda_stream)
    shapes = {}
    # every shape of one row per workgroup whose threads x vectors cover the row once (not twice)
    cover = [(t, v) for t in (64, 128, 256, 512, 1024) for v in (1, 2, 4, 8) if H <= t * v * 8 < 2 * H]
    if not cover:
        raise ValueError(f"no one-row-per-workgroup shape of the streaming kernel covers H = {H}")
    for threads, vpt in cover:
        def launch(i, threads=threads, vpt=vpt):
            _, src, o0, o1 = sets[i]
            rc = mix(src, n_src, o0, o1, T, H, H, threads, vpt, stream)
            if rc:
                raise RuntimeError(f"ceiling launch failed: {rc}")
        shapes[f"{threads}x{vpt}"] = back_to_back_us(torch, launch, n_sets)
    best = min(shapes, key=shapes.get)
    del sets
    torch.cuda.empty_cache()
    out = {"reads_writes": f"{n_src}:{n_out - 0.5 if byte_second else n_out}", "bytes": nbytes,
           "us_per_launch_by_shape": shapes,
           "best_shape": best, "GBps": nbytes / shapes[best] / 1e3,
           "frac": nbytes / shapes[best] / 1e3 / PEAK_HBM_GBPS}
    for name, us in kernel_us.items():
        out[f"{name}_back_to_back_us"] = us
        out[f"{name}_time_over_ceiling_time"] = us / shapes[best] if us else None
    return out


def gather_ceiling(torch, dm, moe_us, rows=None, others=None):
    """The gathering 9:2 stream (libboundary_ceiling.so: eight rows read through the MoE
    workload's own index, the ninth by row, two rows written, no arithmetic) over rotating copies
    of the expert rows, beside the MoE finalize timed the same way. `rows` = (row_begin, count)
    restricts it to a share of the token rows, as the reduce-scatter share reads them."""
    from reduce_residual_rmsnorm_bnd_amd import _build

    L = ctypes.CDLL(_build.CEILING_LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.bnd_ceiling_gather_9r2w.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int,
                                          ctypes.c_int, vp]
    T, H, k = dm["T"], dm["H"], dm["k"]
    if k != 8:
        raise ValueError("the gathering stream reads eight rows")
    rb, R = (0, T) if rows is None else rows
    if rb < 0 or R < 1 or rb + R > T:
        raise ValueError(f"rows {rb}..{rb + R - 1} outside the batch of {T}")
    E0 = dm["expert_rows"].to("cuda:0")
    idx = dm["idx"].to("cuda:0")
    idx_ptr = idx.data_ptr() + rb * k * 4  # int32 [T, k]: the share's first row
    nbytes = 11 * R * H * 2
    # rotate over at least 1 GiB of the bytes a launch moves (its gathered rows lie anywhere in the
    # expert buffer, so each set gets its own copy of that buffer), as the MoE finalize's timing does
    n_sets = max(2, -(-ROTATE_BYTES // nbytes))
    sets = []
    for s_i in range(n_sets):
        E = E0 if s_i == 0 else E0.clone()
        bufs = [torch.zeros(R, H, dtype=torch.bfloat16, device="cuda:0") for _ in range(3)]
        sets.append((E, bufs))
    stream = vp(torch.cuda.current_stream().cuda_stream)
    shapes = {}
    for threads, vpt in ((64, 8), (256, 2), (512, 1)):
        def launch(i, threads=threads, vpt=vpt):
            E, (s8, o0, o1) = sets[i]
            rc = L.bnd_ceiling_gather_9r2w(vp(E.data_ptr()), E.shape[0], vp(idx_ptr), vp(s8.data_ptr()),
                                           vp(o0.data_ptr()), vp(o1.data_ptr()), R, H, H, threads, vpt, stream)
            if rc:
                raise RuntimeError(f"gather ceiling launch failed: {rc}")
        shapes[f"{threads}x{vpt}"] = back_to_back_us(torch, launch, n_sets)
    best = min(shapes, key=shapes.get)
    del sets, E0
    torch.cuda.empty_cache()
    return {"rows": [rb, rb + R - 1], "bytes": nbytes, "rotation_sets": n_sets, "us_per_launch_by_shape": shapes,
            "best_shape": best, "GBps": nbytes / shapes[best] / 1e3,
            "frac": nbytes / shapes[best] / 1e3 / PEAK_HBM_GBPS,
            "moe_back_to_back_us": moe_us,
            "moe_time_over_ceiling_time": moe_us / shapes[best] if moe_us else None,
            **{f"{name}_back_to_back_us": us for name, us in (others or {}).items()},
            **{f"{name}_time_over_ceiling_time": us / shapes[best] if us else None
               for name, us in (others or {}).items()}}


def device_memory_info():
    """Memory clock and bus width as the HIP runtime reports them, and the peak they imply."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    dev = ctypes.c_int()
    if hip.hipGetDevice(ctypes.byref(dev)) != 0:
        return None
    vals = {}
    # hipDeviceAttributeMemoryClockRate = 60, MemoryBusWidth = 59, MultiprocessorCount = 63
    for name, attr in (("memory_clock_khz", 60), ("memory_bus_width_bits", 59),
                       ("compute_units", 63)):
        v = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) == 0:
            vals[name] = v.value
    return vals


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cgroup_cpu_quota():
    """CPUs the process's cgroup may use (cpu.max quota / period), or None when unlimited or
    unreadable."""
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        return None if quota == "max" else int(quota) / int(period)
    except (OSError, ValueError):
        return None


def host_cpu_info() -> dict:
    """The host's cores as the process sees them: the machine's count, the affinity set, the
    cgroup quota, OMP_NUM_THREADS, the CPU model; and `share`, the cores the all-core oracle
    run uses: the affinity set, bounded by the quota and by OMP_NUM_THREADS where they are set."""
    affinity = len(os.sched_getaffinity(0))
    quota = cgroup_cpu_quota()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    share = affinity
    if quota:
        share = min(share, max(1, int(quota)))
    if omp.isdigit() and int(omp) > 0:
        share = min(share, int(omp))
    return {"host_cores": os.cpu_count(), "affinity_cores": affinity, "cgroup_cpu_quota": quota,
            "omp_num_threads": int(omp) if omp.isdigit() else None, "share": share, "cpu": cpu_model()}


def oracle_inputs(workloads, d):
    import oracle

    return (oracle.Oracle(), [workloads.bf16_bits(c) for c in d["partials"]],
            workloads.bf16_bits(d["residual"]), d["weight"].numpy())


def cpu_threads_rate(workloads, d, budget_s: float, threads: int):
    """The same oracle function over row chunks, one chunk per host thread (ctypes releases
    the GIL); only the harness partitions the rows. Whole prefill passes for about `budget_s`."""
    import concurrent.futures as cf

    o, parts, res, w = oracle_inputs(workloads, d)
    T = d["T"]
    bounds = [(T * i // threads, T * (i + 1) // threads) for i in range(threads)]

    def chunk(b):
        lo, hi = b
        o.fold_norm(parts, res[lo:hi].copy(), w, d["eps"], row_begin=lo, rows=hi - lo)

    passes = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        while True:
            list(ex.map(chunk, bounds))
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return passes, el


def cpu_single_rate(workloads, d, budget_s: float):
    """The oracle on one thread pinned to one host core, whole prefill passes for about
    `budget_s` (at least three); returns (pass times, total seconds, the core)."""
    o, parts, res, w = oracle_inputs(workloads, d)
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})  # the calling thread, which runs the oracle
    try:
        times = []
        t0 = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            o.fold_norm(parts, res, w, d["eps"])
            times.append(time.perf_counter() - t1)
            el = time.perf_counter() - t0
            if el >= budget_s and len(times) >= 3:
                break
    finally:
        os.sched_setaffinity(0, allowed)
    return times, el, core


def cpu_baseline(workloads, d, budget_s: float) -> dict:
    """The fp64 oracle (plain C, single-threaded per call) over the whole prefill workload on the
    host: one thread per core of the process's share of the host (headline value), and one
    thread pinned to one core (`single_core`). Rates count whole passes of the 2048-row boundary;
    GB/s uses the kernel's algorithmic bytes."""
    info = host_cpu_info()
    T, H, P = d["T"], d["H"], d["P"]
    nbytes = (P + 3) * T * H * 2 + H * 4
    threads = info["share"]
    log(f"CPU baseline: the oracle on {threads} threads for ~{budget_s / 2:.0f} s")
    passes, el = cpu_threads_rate(workloads, d, budget_s / 2, threads)
    log(f"CPU baseline: the oracle on one pinned core for ~{budget_s:.0f} s")
    times, el1, core = cpu_single_rate(workloads, d, budget_s)
    med = sorted(times)[len(times) // 2]
    return {"value": passes * T / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "GBps": passes * nbytes / el / 1e9,
            "sample": f"{passes} passes of the full prefill boundary (2048 rows x 4096, P=8), each split "
                      f"into {threads} row chunks run on {threads} threads, in {el:.1f} s, fp64",
            **info,
            "single_core": {"value": T / med, "unit": "tokens/s", "cores": 1, "GBps": nbytes / med / 1e9,
                            "sample": f"{len(times)} passes of the same boundary in {el1:.1f} s on one "
                                      f"thread pinned to core {core}; rate of the median pass"}}


def leg(sec: dict, name: str, fn, torch=None):
    """Runs one secondary measurement; an exception is recorded under its name instead of ending
    the run, so the headline line is still printed."""
    try:
        out = fn()
        if out is not None:
            sec[name] = out
    except Exception as e:  # noqa: BLE001 - any failure of a secondary figure is reported, not fatal
        import traceback

        traceback.print_exc(file=sys.stderr)
        sec[name] = {"error": f"{type(e).__name__}: {e}"}
    if torch is not None:
        torch.cuda.empty_cache()


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true", help="only the prefill step")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--with-copy", action="store_true",
                    help="also run the 1 GiB reference copy (a known byte count for counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    return args


def headline(torch, bnd, d, timer, steps: int, warmup: int):
    """The prefill fold timed over `steps` launches: the result line without its secondary part,
    the step function (for later back-to-back timing) and the buffers it keeps alive."""
    props = torch.cuda.get_device_properties(0)
    per_set = (d["P"] + 3) * d["T"] * d["H"] * 2
    n_sets = max(2, -(-ROTATE_BYTES // per_set))
    step, nbytes, keep = fold_case(torch, bnd, d, n_sets)
    log(f"timing {steps} steps over {n_sets} rotating sets")
    t = timer.run(step, n_sets, warmup, steps)
    shape = launch_desc(bnd)
    achieved = nbytes / t["kernel_s"] / 1e9
    traffic = traffic_from_profiles("prefill T=2048 H=4096 P=8")
    result = {
        "metric": METRIC,
        "value": steps * d["T"] / t["wall_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": t["wall_s"] / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill boundary fold+RMSNorm, T=2048 H=4096 P=8, bf16 in/out",
                   "T": 2048, "H": 4096, "P": 8, "rotation_sets": n_sets,
                   "device": getattr(props, "gcnArchName", props.name),
                   "storage": "bf16 partials, residual and y; fp32 weight", "accumulate": "fp32",
                   "device_memory": device_memory_info()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": ("bnd_fold_norm's kernel, "
                                + (f"wave_read_kernel<Partials, {shape['vectors_per_thread']} vectors per lane, "
                                   "bf16 out> (one wavefront per row)" if shape["one_wavefront_per_row"] else
                                   f"read_kernel<Partials, P=8, {shape['vectors_per_thread']} vectors per thread, "
                                   f"bf16 out> ({shape['threads']} threads per row)")),
                     "launch": shape,
                     "algorithmic_bytes": nbytes,
                     "kernel_mean_us": us(t["kernel_s"]),
                     "kernel_timing": "HIP events recorded by the launches' own dispatch over the timed "
                                      "region: the smaller of the first launch's start to the last "
                                      "launch's stop / K, and the mean start-to-stop of the sampled launches",
                     "span_us_per_launch": us(t["span_s"]),
                     "dispatch_event_mean_us": us(t["dispatch_event_mean_s"]),
                     **spread_fields(t),
                     "dispatch_events": t["dispatch_events"],
                     "interval_us_per_launch": us(t["interval_mean_s"]),
                     "intervals": t["intervals"],
                     "sample_every": t["sample_every"],
                     "steady_state_us_per_launch": t["wall_s"] / steps * 1e6},
    }
    return result, step, n_sets, keep


def secondary(torch, bnd, workloads, d, timer, fold_step, n_sets) -> dict:
    """Every other figure of the JSON line, each leg isolated (`leg`)."""
    sec = {}
    b2b = {}
    leg(b2b, "fold", lambda: back_to_back_us(torch, lambda i: fold_step(i, None, None), n_sets))
    fold_us = b2b["fold"] if isinstance(b2b["fold"], float) else None

    log("9:2 streaming ceiling (the fold's loads and stores without arithmetic)")
    leg(sec, "stream_ceiling_9r2w_T2048_H4096",
        lambda: stream_ceiling(torch, d["T"], d["H"], 9, 2, {"fold": fold_us}), torch)

    fp8_us = {}

    def fp8():
        log("quantised read (T=2048 H=7168 P=8, fp8 out)")
        dq = workloads.quantised()
        n_q = max(2, -(-ROTATE_BYTES // ((dq["P"] + 2) * dq["T"] * dq["H"] * 2 + dq["T"] * dq["H"])))
        step, nb, keep = fold_case(torch, bnd, dq, n_q, fp8=True)
        tq = timer.run(step, n_q, 20, 256)
        fp8_us["fp8"] = back_to_back_us(torch, lambda i: step(i, None, None), n_q)
        return {"tokens_per_s_kernel": 2048 / tq["kernel_s"], **kernel_fields(tq, bnd),
                "GBps": nb / tq["kernel_s"] / 1e9, "frac": nb / tq["kernel_s"] / 1e9 / PEAK_HBM_GBPS,
                "algorithmic_bytes": nb, "back_to_back_us": fp8_us["fp8"]}

    leg(sec, "fp8_T2048_H7168_P8", fp8, torch)
    # the fp8 read writes a bf16 residual row and a row of one-byte codes: between the 9:1 and 9:2
    # streams at its width
    log("9:1, 9:2 and 9:1.5 streaming ceilings at H = 7168 (the quantised read's width)")
    leg(sec, "stream_ceiling_9r1w_T2048_H7168",
        lambda: stream_ceiling(torch, 2048, 7168, 9, 1, {"fp8": fp8_us.get("fp8")}), torch)
    leg(sec, "stream_ceiling_9r2w_T2048_H7168",
        lambda: stream_ceiling(torch, 2048, 7168, 9, 2, {"fp8": fp8_us.get("fp8")}), torch)
    # the fp8 read's own mix: nine reads, a bf16 row and a row of one-byte codes written
    leg(sec, "stream_ceiling_9r1h_T2048_H7168",
        lambda: stream_ceiling(torch, 2048, 7168, 9, 2, {"fp8": fp8_us.get("fp8")}, byte_second=True), torch)

    log("MoE finalize (T=2048 H=4096 k=8), full rows and rows 768..1023")
    dm = workloads.moe()
    moe_us = {}

    def moe(rb, rows, tg):
        # rotate over at least 1 GiB of the bytes a launch moves: a share reads only its rows' picks
        n_m = max(2, -(-ROTATE_BYTES // (rows * (dm["k"] + 3) * dm["H"] * 2)))
        step, nb, keep = moe_case(torch, bnd, dm, n_m, rb, rows, terminal_gemma=tg)
        tm = timer.run(step, n_m, 20, 256)
        out = {"tokens_per_s_kernel": rows / tm["kernel_s"], **kernel_fields(tm, bnd),
               "GBps": nb / tm["kernel_s"] / 1e9, "frac": nb / tm["kernel_s"] / 1e9 / PEAK_HBM_GBPS,
               "algorithmic_bytes": nb}
        moe_us[(rows, tg)] = back_to_back_us(torch, lambda i: step(i, None, None), n_m)
        out["back_to_back_us"] = moe_us[(rows, tg)]
        return out

    # the full-row calls first, then the share with its 47 rotation sets
    leg(sec, "moe_full_T2048_H4096_k8", lambda: moe(0, 2048, False), torch)
    leg(sec, "moe_terminal_gemma_T2048_H4096_k8", lambda: moe(0, 2048, True), torch)
    leg(sec, "moe_slice_rows768_1023", lambda: moe(*workloads.MOE_SLICE, False), torch)
    log("gathering 9:2 streaming ceilings (the MoE finalize's loads and stores without arithmetic)")
    leg(sec, "gather_ceiling_9r2w_T2048_H4096_k8",
        lambda: gather_ceiling(torch, dm, moe_us.get((2048, False)),
                               others={"moe_terminal_gemma": moe_us.get((2048, True))}), torch)
    leg(sec, "gather_ceiling_9r2w_rows768_1023_H4096_k8",
        lambda: gather_ceiling(torch, dm, moe_us.get((workloads.MOE_SLICE[1], False)), rows=workloads.MOE_SLICE), torch)
    del dm

    log("complete_only, snapshot and add_to_output (prefill sizes), the unfused fallback, "
        "the largest RSv share of 2047 rows")
    aux_us = {}

    def aux(kind):
        step, nb, keep = aux_case(torch, bnd, d, n_sets, kind)
        ta = timer.run(step, n_sets, 20, 256)
        aux_us[kind] = back_to_back_us(torch, lambda i: step(i, None, None), n_sets)
        return {**kernel_fields(ta, bnd), "GBps": nb / ta["kernel_s"] / 1e9,
                "frac": nb / ta["kernel_s"] / 1e9 / PEAK_HBM_GBPS, "algorithmic_bytes": nb}

    for kind in ("complete_only", "snapshot", "add_to_output"):
        leg(sec, f"{kind}_T2048_H4096_P8", lambda kind=kind: aux(kind), torch)
    log("8:1 and 9:1 streaming ceilings (complete_only; snapshot and add_to_output)")
    leg(sec, "stream_ceiling_8r1w_T2048_H4096", lambda: stream_ceiling(
        torch, d["T"], d["H"], 8, 1, {"complete_only": aux_us.get("complete_only")}), torch)
    leg(sec, "stream_ceiling_9r1w_T2048_H4096", lambda: stream_ceiling(
        torch, d["T"], d["H"], 9, 1, {"snapshot": aux_us.get("snapshot"),
                                      "add_to_output": aux_us.get("add_to_output")}), torch)

    def unfused():
        step, nb, keep = aux_case(torch, bnd, d, n_sets, "unfused")
        unfused_us = back_to_back_us(torch, lambda i: step(i, None, None), n_sets)
        return {"launches_per_step": 2, "us_per_step_back_to_back": unfused_us,
                "fused_fold_us_back_to_back": fold_us,
                "unfused_over_fused": unfused_us / fold_us if fold_us else None,
                "algorithmic_bytes": nb, "GBps": nb / unfused_us / 1e3}

    leg(sec, "unfused_fallback_T2048_H4096_P8", unfused, torch)

    rsv_share = {}

    def rsv():
        counts = [300, 0, 511, 256, 257, 1, 400, 322]
        rb, rows, Tr = bnd.bnd_rsv_share(counts, 2)
        dr = workloads.fold_inputs(6, Tr, 4096, 8)
        n_r = max(2, -(-ROTATE_BYTES // (rows * 11 * 4096 * 2)))
        step, nb, keep = fold_case(torch, bnd, dr, n_r, row_begin=rb, rows=rows)
        tr = timer.run(step, n_r, 20, 256)
        fields = kernel_fields(tr, bnd)
        rsv_share.update(rows=rows, us=back_to_back_us(torch, lambda i: step(i, None, None), n_r))
        return {"row_begin": rb, "rows": rows, **fields, "GBps": nb / tr["kernel_s"] / 1e9,
                "frac": nb / tr["kernel_s"] / 1e9 / PEAK_HBM_GBPS, "algorithmic_bytes": nb,
                "back_to_back_us": rsv_share["us"]}

    leg(sec, "rsv_share_511_of_2047_H4096_P8", rsv, torch)
    # the same 9:2 stream over as many rows as the share: two rows per CU, one launch's ramp and drain
    leg(sec, "stream_ceiling_9r2w_T511_H4096",
        lambda: stream_ceiling(torch, rsv_share.get("rows", 511), 4096, 9, 2, {"rsv_share": rsv_share.get("us")}),
        torch)
    def tiny():
        dt = workloads.tiny()
        step, nb, keep = fold_case(torch, bnd, dt, 2)
        tt = timer.run(step, 2, 20, 256)
        return {"T": dt["T"], "H": dt["H"], "P": dt["P"], **kernel_fields(tt, bnd), "algorithmic_bytes": nb,
                "us_per_call_back_to_back": back_to_back_us(torch, lambda i: step(i, None, None), 2),
                "note": "launch-latency bound: 41,984 bytes per call"}

    log("tiny fold (T=16 H=256 P=2)")
    leg(sec, "tiny_T16_H256_P2", tiny, torch)
    log("decode chain (1 enter + 96 folds), eager and graph")
    leg(sec, "decode", lambda: [decode_chain(torch, bnd, workloads, T, 20, 50) for T in (1, 8, 32, 128)], torch)
    leg(sec, "launch_floor_empty_kernel", lambda: launch_floor(torch), torch)
    leg(sec, "launch_floor_empty_kernel_boundary_args", lambda: launch_floor(torch, with_args=True), torch)
    leg(sec, "copy_ceiling_1GiB", lambda: copy_ceiling(torch), torch)
    return sec


def main(argv=None):
    args = parse_args(argv)

    import torch

    import workloads
    import reduce_residual_rmsnorm_bnd_amd as bnd
    from reduce_residual_rmsnorm_bnd_amd import _build

    if not os.path.exists(_build.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    timer = Timed(torch.cuda.synchronize)

    log("generating the prefill workload (T=2048 H=4096 P=8)")
    d = workloads.prefill()
    result, step, n_sets, keep = headline(torch, bnd, d, timer, args.steps, args.warmup)
    if not args.no_secondary:
        result["secondary"] = secondary(torch, bnd, workloads, d, timer, step, n_sets)
    del keep, step
    torch.cuda.empty_cache()
    if args.no_secondary and args.with_copy:
        result["copy_reference_1GiB"] = copy_ceiling(torch)
    try:
        result["cpu_baseline"] = cpu_baseline(workloads, d, args.cpu_seconds)
    except Exception as e:  # noqa: BLE001 - reported in the line, the GPU figures still print
        import traceback

        traceback.print_exc(file=sys.stderr)
        result["cpu_baseline"] = {"error": f"{type(e).__name__}: {e}", "kind": "oracle"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
