#!/usr/bin/env python3
"""Benchmark of the rotated W4A16 linear on one MI355X.

Headline workload: the seven linears of one 8B-class decoder layer (q, k, v, o:
4096 -> 4096/1024/1024/4096; gate, up: 4096 -> 14336; down: 14336 -> 4096), each
with its own transform of K = 8 Givens stages and channel scaling, INT4 group 128.
One decode step = the seven rotated linears at M = 64 tokens as one
paro_linear_batch call. Every step reads its weights, scales, zeros and transform
descriptors cold from HBM: each step takes the next copies from a pool larger than
1 GiB (four times the 256 MB Infinity Cache). Steps are replayed as HIP graphs
captured from the library's own launches, so Python call overhead stays out of
the timed region, and the timed replays continue the pool rotation where the
warm-up replays stopped.

Prints ONE JSON line: decode HBM GB/s of the whole step (algorithmic bytes /
time) with the roofline of its linear kernel, the prefill step of the same layer
(M = 4096) in TFLOP/s with its own roofline, the rotation overhead of both
against the plain INT4 linear on the same packed weights, the CPU oracle's
throughput on bounded samples of each workload, and extras (the Qwen2.5-1.5B-
shaped attention decode step, gate+up decode and prefill, down_proj prefill,
overhead against the stage count, the whole-stack decode and build, chunked
prefill overlap).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rotated W4A16 linear: decode HBM GB/s, prefill TFLOP/s, rotation overhead %"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
POOL_BYTES = int(1.1 * (1 << 30))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-extras", action="store_true", help="skip the extras")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time of the headline's oracle sample")
    p.add_argument("--only", choices=("decode", "prefill"),
                   help="for rocprofv3 runs: only the 8B-class layer's decode (M=64) or prefill (M=4096) step, "
                        "rotated then plain, timed as in the full run; prints one JSON line")
    p.add_argument("--traffic", choices=("decode", "prefill"),
                   help="for rocprofv3 --pmc runs: a 256 MiB float16 negation (the counter calibration copy), "
                        "then --steps plain linear steps of the 8B-class layer (the step's linear kernel alone), "
                        "eagerly, each on its own pool copy; prints one JSON line")
    return p.parse_args()


# --------------------------------------------------------------------------- #
# building blocks
# --------------------------------------------------------------------------- #

class Linear:
    """One linear's prepared transform and packed weights, plus pool copies for cold reads."""

    def __init__(self, rl, torch, L):
        self.L = L
        self.D, self.N, self.K = L.spec.D, L.spec.N, L.spec.K
        self.rot = rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)
        self.w = rl.paro_pack_weights(self.rot, torch.from_numpy(L.W).cuda())
        self.copies = []

    def set_bytes(self):
        return sum(t.numel() * t.element_size() for t in self.w) + self.rot.desc.numel()

    def make_copies(self, rl, n):
        self.copies = []
        for _ in range(n):
            desc = self.rot.desc.clone()
            rot = rl.Rotation(self.K, self.D, desc, rl.paro_rotation(self.K, self.D, desc.data_ptr()))
            self.copies.append((rot, tuple(t.clone() for t in self.w)))


def workload_bytes(M, D, N, K, rotated=True):
    import workloads as W
    return W.algorithmic_bytes(M, D, N, K) if rotated else W.plain_bytes(M, D, N)


class Step:
    """A list of (linear, M) calls; ``slot`` picks the pool copy used by the call."""

    def __init__(self, rl, torch, linears, Ms):
        self.rl, self.torch = rl, torch
        self.linears, self.Ms = linears, Ms
        self.calls = [(li, M) for M in Ms for li in range(len(linears))]
        self.x = {}
        self.y = {}
        self.ws = {}
        for li, M in self.calls:
            lin = linears[li]
            self.x[(li, M)] = torch.from_numpy(lin.L.x[:M]).cuda()
            self.y[(li, M)] = torch.empty((M, lin.N), dtype=torch.float16, device="cuda")
            need = rl.paro_workspace_bytes(M, lin.D, lin.N)
            self.ws[(li, M)] = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        # every call's workspace at once is enough for any batch of these calls
        self.batch_ws = torch.empty(max(sum(t.numel() for t in self.ws.values()), 256), dtype=torch.uint8,
                                    device="cuda")

    def bytes(self, rotated=True):
        return sum(workload_bytes(M, self.linears[li].D, self.linears[li].N, self.linears[li].K, rotated)
                   for li, M in self.calls)

    def flops(self):
        return sum(2.0 * M * self.linears[li].D * self.linears[li].N for li, M in self.calls)

    def _weights(self, li, M, slot):
        lin = self.linears[li]
        if lin.copies:
            return lin.copies[(slot * len(self.Ms) + self.Ms.index(M)) % len(lin.copies)]
        return lin.rot, lin.w

    def enqueue(self, slot, rotated=True, only=None, batched=False):
        """Enqueue the step's calls on the current stream: one library call each, or all of them
        as one paro_linear_batch call (batched)."""
        rl = self.rl
        if batched:
            calls, outs = [], []
            for ci, (li, M) in enumerate(self.calls):
                if only is not None and ci not in only:
                    continue
                rot, w = self._weights(li, M, slot)
                calls.append((rot if rotated else None, self.x[(li, M)], *w))
                outs.append(self.y[(li, M)])
            rl.paro_linear_batch(calls, outs=outs, ws=self.batch_ws)
            return
        for ci, (li, M) in enumerate(self.calls):
            if only is not None and ci not in only:
                continue
            rot, w = self._weights(li, M, slot)
            if rotated:
                rl.paro_rotated_linear(rot, self.x[(li, M)], *w, out=self.y[(li, M)], ws=self.ws[(li, M)])
            else:
                rl.paro_w4a16_linear(self.x[(li, M)], *w, out=self.y[(li, M)], ws=self.ws[(li, M)])


def capture(torch, fn, n_graphs):
    """Capture fn(slot) for slot in range(n_graphs) as separate HIP graphs."""
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # warm the kernels' one-time attributes outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for slot in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(slot)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def read_sclk_mhz():
    """The shader clock the driver reports for the first GPU right now (the starred level of
    sysfs pp_dpm_sclk) and the highest level it lists, in MHz; None where sysfs does not say."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                lines = f.read().splitlines()
        except OSError:
            continue
        levels = [(int(m.group(1)), ln.rstrip().endswith("*"))
                  for ln in lines for m in [re.search(r"(\d+)\s*mhz", ln, re.I)] if m]
        if levels:
            cur = [v for v, star in levels if star]
            return {"now": cur[0] if cur else None, "max_level": max(v for v, _ in levels)}
    return None


SCLK_SAMPLES = []  # (label, read_sclk_mhz()) taken while timed GPU work runs


def time_graphs(torch, graphs, steps, warmup, min_warm_s=0.0, sclk_label=None):
    """Replay graphs round-robin: `warmup` untimed replays (continued until at least `min_warm_s`
    seconds have passed: an idle GPU lowers its clocks, a few ms of work bring them back), then
    `steps` timed ones bracketed by HIP events on the replay stream. The timed replays continue the
    rotation where the warm-up stopped, so the first timed graph is not one the warm-up has just
    run (its copies could still sit in the Infinity Cache). Returns ms per replay."""
    t0 = time.perf_counter()
    t = 0
    while t < warmup or time.perf_counter() - t0 < min_warm_s:
        graphs[t % len(graphs)].replay()
        t += 1
        if t % len(graphs) == 0 and t >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for u in range(steps):
        graphs[(t + u) % len(graphs)].replay()
    end.record()
    if sclk_label is not None:  # the replays are still running: read the clock under load
        SCLK_SAMPLES.append((sclk_label, read_sclk_mhz()))
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_slots(torch, fn, n_slots, per, steps, warmup, min_warm_s=0.05, sclk_label=None):
    """fn(slot) for slot < n_slots, captured as graphs of `per` consecutive slots (so one replay
    carries several steps and host launch cost stays out of the per-step time); returns ms per
    step over `steps` steps (rounded up to whole graphs) after `warmup` untimed ones (and at least
    `min_warm_s` seconds of them)."""
    n_graphs = max(1, n_slots // per)
    gs = capture(torch, lambda g: [fn(g * per + r) for r in range(per)], n_graphs)
    ms = time_graphs(torch, gs, max(1, -(-steps // per)), -(-warmup // per), min_warm_s, sclk_label) / per
    del gs
    return ms


# --------------------------------------------------------------------------- #
# CPU oracle baselines
# --------------------------------------------------------------------------- #

def _blas_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info
                                 if i.get("user_api") == "blas"})) or "unknown"
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores, blas = os.cpu_count() or 1, "unknown"
    return int(cores), blas


def cpu_baseline(step, seconds, rows=None):
    """The oracle's per-call path (float64 transform + x' . deq^T, deq precomputed) on the calls of
    a GPU step, repeated for about ``seconds`` of wall time. ``rows``: compute only that many
    output columns of each call (the weight rows are independent), counting bytes for those."""
    import numpy as np

    import oracle as O

    import workloads as W

    deq = {}
    for li, lin in enumerate(step.linears):
        qw, sc, z = (t.cpu().numpy() for t in lin.w)
        qw = W.qweight_from_blocked(qw)  # the library's blocked order -> the oracle's row-major one
        n = lin.N if rows is None else min(rows, lin.N)
        deq[li] = O.dequantize(qw[:n], sc[:n], z[:n])
    xs = {k: v.cpu().numpy() for k, v in step.x.items()}
    n_steps, t0 = 0, time.perf_counter()
    while True:
        for li, M in step.calls:
            L = step.linears[li].L
            a = O.transform_activations(xs[(li, M)], L.pairs, L.theta, L.scale)
            _ = a @ deq[li].T
        n_steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores, blas = _blas_threads()
    nbytes = sum(workload_bytes(M, step.linears[li].D, deq[li].shape[0], step.linears[li].K) for li, M in step.calls)
    gbs = nbytes * n_steps / el / 1e9
    cols = "" if rows is None else f", the first {rows} output columns of each"
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_steps} oracle passes over the step's {len(step.calls)} calls{cols} "
                      f"(float64 transform + x'.deq^T, deq precomputed) in {el:.1f} s, single pass each; "
                      f"host {os.cpu_count()} logical CPUs, BLAS threads {cores} ({blas})"}


def cpu_pack_baseline(lins, rows, seconds):
    """The oracle's build-time path (float64 fold, quantize, pack) on the first ``rows`` weight rows
    of each linear, repeated for about ``seconds``; weights per second."""
    import oracle as O

    n, t0 = 0, time.perf_counter()
    while True:
        for lin in lins:
            L = lin.L
            O.pack_weights(L.W[:rows], L.pairs, L.theta, L.scale)
            n += rows * lin.D
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores, blas = _blas_threads()
    return {"value": round(n / el / 1e6, 3), "unit": "Mweights/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 fold + quantize + pack of {rows} weight rows of each of {len(lins)} linears, "
                      f"{n} weights in {el:.1f} s"}


def attainable(torch):
    """What this box attains outside the library: a cold streaming copy (1 GiB each way, far past
    the Infinity Cache), a large float16 GEMM from the vendor library (torch.matmul, 8192^3), and
    the floor of one launch (a one-element fill) replayed from a HIP graph."""
    out = {}
    a = torch.empty(1 << 29, dtype=torch.float16, device="cuda")  # 1 GiB
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    out["hbm_copy_GBps"] = round(2 * a.numel() * 2 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    n = 8192
    x = torch.randn(n, n, device="cuda").half()
    w = torch.randn(n, n, device="cuda").half()
    for _ in range(2):
        torch.matmul(x, w)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.matmul(x, w)
    e1.record()
    for i in range(4):  # the 10 products take about 10 ms: four samples 2 ms apart
        SCLK_SAMPLES.append(("vendor fp16 GEMM #%d" % i, read_sclk_mhz()))
        time.sleep(0.002)
    torch.cuda.synchronize()
    out["fp16_gemm_TFLOPs"] = round(2.0 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    del x, w
    t = torch.zeros(1, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        t.fill_(0.0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(100):
            t.fill_(1.0)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    out["graph_launch_floor_us"] = round(e0.elapsed_time(e1) * 1e3 / 500, 2)
    return out


# --------------------------------------------------------------------------- #
# main
# --------------------------------------------------------------------------- #

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import rotated_linear_amd as rl
    import workloads as W

    torch.cuda.init()
    if args.traffic:
        traffic_run(rl, torch, W, args.traffic, args.steps)
        return
    layer = Layer8B(rl, torch, W)
    if args.only:
        res = layer.decode(args) if args.only == "decode" else layer.prefill(args)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return

    dec = layer.decode(args, sclk_label="8B-class layer decode step")
    pre = layer.prefill(args)
    att = attainable(torch)
    for r in (dec["roofline"], pre["roofline"]):
        base = att["hbm_copy_GBps"] if r["unit"] == "GB/s" else att["fp16_gemm_TFLOPs"]
        r["frac_of_attainable"] = round(r["achieved"] / base, 4)
    out = {
        "metric": METRIC, "value": dec["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "8B-class decoder layer, decode: q, k, v, o, gate, up, down "
                               "(4096->4096/1024/1024/4096/14336/14336, 14336->4096), each with its own transform",
                   "M": 64, "K_stages": 8, "group": 128, "calls_per_step": 7,
                   "launch": dec["launch"], "algorithmic_bytes_per_step": dec["algorithmic_bytes"],
                   "cold_pool_bytes": dec["cold_pool_bytes"]},
        "roofline": dec["roofline"],
        "rotation_overhead_pct": dec["overhead_pct"],
        "plain_w4a16": dec["plain"],
        "prefill": {k: v for k, v in pre.items() if k != "roofline"},
        "roofline_prefill": pre["roofline"],
        "attainable": att,
    }
    if not args.no_extras:
        out["extras"] = extras(rl, torch, W, args)
        for e in out["extras"].values():  # the same results against what the box attains
            if "TFLOP/s" in e:
                e["frac_of_attainable_gemm"] = round(e["TFLOP/s"] / att["fp16_gemm_TFLOPs"], 4)
            if "GB/s" in e:
                e["frac_of_attainable_hbm"] = round(e["GB/s"] / att["hbm_copy_GBps"], 4)
    out["sclk_mhz_under_load"] = {label: v for label, v in SCLK_SAMPLES}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layer.decode_step, args.cpu_seconds, rows=2048)
        out["cpu_baseline_by_workload"] = cpu_by_workload(rl, torch, W, layer)
    print(json.dumps(out), flush=True)


CALIB_BYTES = 256 << 20  # bytes read (and written) by the calibration copy
# counter summaries of the headline steps' linear kernel, each valid only for the kernel sources it
# was taken on
TRAFFIC_FILES = {"decode": os.path.join(ROOT, "profiles", "traffic_layer8b_decode_M64.md"),
                 "prefill": os.path.join(ROOT, "profiles", "traffic_layer8b_prefill_M4096.md")}
KERNEL_SOURCES = {"decode": ["rotated_linear_amd/csrc/skinny.hip", "rotated_linear_amd/csrc/gemm.hip",
                             "rotated_linear_amd/csrc/paro_internal.h"],
                  "prefill": ["rotated_linear_amd/csrc/gemm.hip", "rotated_linear_amd/csrc/paro_internal.h"]}


def kernel_source_hash(which):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(which):
    """HBM bytes per launch of the step's linear kernel from the committed counter summary, or None
    when that summary was taken on other kernel sources than the ones built here."""
    try:
        kv = {}
        with open(TRAFFIC_FILES[which]) as fh:
            for line in fh:
                if " = " in line:
                    k, v = line.split(" = ", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256_16") != kernel_source_hash(which):
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def attention_step(rl, torch, W):
    """The default step: q, k, v, o (D=1536) at M = 1, 4, 16, with a cold pool of weight copies."""
    wl = W.WORKLOADS[2]
    linears = [Linear(rl, torch, W.make_linear(2, i)) for i in range(len(wl.linears))]
    Ms = list(wl.Ms)
    set_bytes = sum(l.set_bytes() for l in linears)
    n_sets = max(4, math.ceil(POOL_BYTES / set_bytes))
    for l in linears:
        l.make_copies(rl, n_sets)
    step = Step(rl, torch, linears, Ms)
    step.n_slots = max(1, n_sets // len(Ms))
    torch.cuda.synchronize()
    return step, set_bytes * n_sets


def traffic_run(rl, torch, W, which, reps):
    """Calibration copy, then `reps` plain linear steps of the 8B-class layer (decode M = 64 or
    prefill M = 4096), eagerly, each on its own pool copy (cold reads)."""
    a = torch.ones(CALIB_BYTES // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    layer = Layer8B(rl, torch, W)
    st = layer.decode_step if which == "decode" else layer.prefill_step()
    for r in range(reps):
        st.enqueue(r, rotated=False, batched=True)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": {"step": which, "steps": reps, "calib_bytes": CALIB_BYTES}}), flush=True)


def _divisor_at_most(k, cap):
    """The largest divisor of k that is at most cap (>= 1)."""
    for p in range(max(1, min(cap, k)), 0, -1):
        if k % p == 0:
            return p
    return 1


class Layer8B:
    """The 8B-class decoder layer's seven linears (q, k, v, o, gate, up, down), each with its own
    transform, packed once on the GPU, with a pool of copies (weights, scales, zeros and
    descriptors) larger than 1 GiB so that every step reads cold from HBM."""

    DECODE_M, PREFILL_M = 64, 4096

    def __init__(self, rl, torch, W):
        self.rl, self.torch = rl, torch
        self.lins = [Linear(rl, torch, W.make_linear(5, i)) for i in range(len(W.WORKLOADS[5].linears))]
        self.set_bytes = sum(l.set_bytes() for l in self.lins)
        self.n_sets = max(4, math.ceil(POOL_BYTES / self.set_bytes))
        for l in self.lins:
            l.make_copies(rl, self.n_sets)
        self.decode_step = Step(rl, torch, self.lins, [self.DECODE_M])
        self._prefill = None
        torch.cuda.synchronize()

    def prefill_step(self):
        if self._prefill is None:
            self._prefill = Step(self.rl, self.torch, self.lins, [self.PREFILL_M])
        return self._prefill

    def _time(self, st, rotated, steps, warmup, per, sclk_label=None):
        n_graphs = max(2, self.n_sets // per)
        return time_slots(self.torch, lambda s: st.enqueue(s, rotated=rotated, batched=True), n_graphs * per, per,
                          steps, warmup, min_warm_s=0.0, sclk_label=sclk_label)

    def decode(self, args, sclk_label=None):
        """The decode step: the seven rotated linears at M = 64 as one paro_linear_batch call, timed
        over exactly --steps steps after --warmup untimed ones; beside it the plain linears on the
        same packed weights (the step's linear kernel alone)."""
        st = self.decode_step
        per = _divisor_at_most(args.steps, min(8, self.n_sets // 2))
        ms_rot = self._time(st, True, args.steps, args.warmup, per, sclk_label)
        ms_plain = self._time(st, False, args.steps, args.warmup, per)
        bytes_rot, bytes_plain = st.bytes(True), st.bytes(False)
        gbs = bytes_rot / (ms_rot * 1e-3) / 1e9
        lin_gbs = bytes_plain / (ms_plain * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(lin_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(lin_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode"),
                    "kernel": "the step's INT4 linear launch (paro_linear_batch of the seven plain linears "
                              "on the same packed weights; event-timed graph replays of that launch alone)",
                    "avg_launch_us": round(ms_plain * 1e3, 3), "algorithmic_bytes_per_launch": bytes_plain}
        return {"GB/s": round(gbs, 3), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "ms_per_step": round(ms_rot, 6),
                "us": round(ms_rot * 1e3, 3), "algorithmic_bytes": bytes_rot,
                "overhead_pct": round((ms_rot - ms_plain) / ms_plain * 100.0, 2),
                "plain": {"us": round(ms_plain * 1e3, 3), "GB/s": round(lin_gbs, 3)},
                "launch": "one paro_linear_batch call per step, HIP graphs of %d steps" % per,
                "cold_pool_bytes": self.set_bytes * self.n_sets, "roofline": roofline}

    def prefill(self, args):
        """The prefill step: the seven rotated linears at M = 4096 as one paro_linear_batch call
        (weights from the cold pool), and the plain linears beside it."""
        st = self.prefill_step()
        steps = max(4, args.steps // 2)
        per = _divisor_at_most(steps, min(4, self.n_sets // 2))
        ms_rot = self._time(st, True, steps, max(2, args.warmup // 2), per)
        ms_plain = self._time(st, False, steps, max(2, args.warmup // 2), per)
        fl = st.flops()
        tf = fl / (ms_rot * 1e-3) / 1e12
        lin_tf = fl / (ms_plain * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(lin_tf, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(lin_tf / MFMA_F16_PEAK_TFLOPS, 4), "traffic": measured_traffic("prefill"),
                    "kernel": "the step's INT4 GEMM launches (paro_linear_batch of the seven plain linears "
                              "on the same packed weights)",
                    "avg_launch_us": round(ms_plain * 1e3, 3), "algorithmic_flop_per_launch": fl}
        return {"TFLOP/s": round(tf, 2), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "M": self.PREFILL_M,
                "steps": steps, "us": round(ms_rot * 1e3, 2), "flop": fl,
                "overhead_pct": round((ms_rot - ms_plain) / ms_plain * 100.0, 2),
                "plain": {"us": round(ms_plain * 1e3, 2), "TFLOP/s": round(lin_tf, 2)}, "roofline": roofline}


def cpu_by_workload(rl, torch, W, layer):
    """The oracle's per-call path on bounded samples of the other workloads, and its build-time
    path (fold, quantize, pack) on the 8B-class layer's weights."""
    res = {}
    att = [Linear(rl, torch, W.make_linear(2, i)) for i in range(4)]
    res["attention_decode_step_M1_4_16"] = cpu_baseline(Step(rl, torch, att, [1, 4, 16]), 3.0)
    gu = Linear(rl, torch, W.make_linear(3, 0))
    res["gate_up_M1_16_256"] = cpu_baseline(Step(rl, torch, [gu], [1, 16, 256]), 3.0, rows=2048)
    dn = Linear(rl, torch, W.make_linear(4, 0))
    res["down_prefill_M2048"] = cpu_baseline(Step(rl, torch, [dn], [2048]), 3.0, rows=256)
    res["pack_layer8b"] = cpu_pack_baseline(layer.lins, 32, 4.0)
    return res


def extras(rl, torch, W, args):
    """The Qwen2.5-1.5B-shaped workloads, rotated vs plain: the attention projections' decode step,
    gate+up decode (HBM) and prefill at M = 256 (MFMA), down_proj prefill (MFMA); the overhead
    against the stage count; the whole-stack decode and build; chunked prefill overlap."""
    res = {}
    res.update(attention_decode(rl, torch, W, args))
    L3 = Linear(rl, torch, W.make_linear(3, 0))
    n3 = max(4, math.ceil(POOL_BYTES / L3.set_bytes()))
    L3.make_copies(rl, n3)
    for M in (1, 16):
        st = Step(rl, torch, [L3], [M])
        ms_r = time_slots(torch, lambda s: st.enqueue(s), n3, 8, 2 * n3, 16)
        ms_p = time_slots(torch, lambda s: st.enqueue(s, rotated=False), n3, 8, 2 * n3, 16)
        res[f"gate_up_decode_M{M}"] = {"GB/s": round(st.bytes() / (ms_r * 1e-3) / 1e9, 2),
                                       "frac_hbm": round(st.bytes() / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "us": round(ms_r * 1e3, 3), "plain_us": round(ms_p * 1e3, 3),
                                       "overhead_pct": round((ms_r - ms_p) / ms_p * 100, 2)}
    st = Step(rl, torch, [L3], [256])  # gate+up at M = 256: MFMA-bound (weights from the cold pool)
    ms_r = time_slots(torch, lambda s: st.enqueue(s), n3, 4, 20, 4)
    ms_p = time_slots(torch, lambda s: st.enqueue(s, rotated=False), n3, 4, 20, 4)
    tf = st.flops() / (ms_r * 1e-3) / 1e12
    res["gate_up_prefill_M256"] = {"TFLOP/s": round(tf, 2), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                   "us": round(ms_r * 1e3, 2),
                                   "plain_TFLOP/s": round(st.flops() / (ms_p * 1e-3) / 1e12, 2),
                                   "overhead_pct": round((ms_r - ms_p) / ms_p * 100, 2)}
    del st, L3
    L4 = Linear(rl, torch, W.make_linear(4, 0))
    n4 = max(4, math.ceil(POOL_BYTES / 2 / L4.set_bytes()))
    L4.make_copies(rl, n4)
    st = Step(rl, torch, [L4], [2048])
    ms_r = time_slots(torch, lambda s: st.enqueue(s), n4, 4, 20, 4)
    ms_p = time_slots(torch, lambda s: st.enqueue(s, rotated=False), n4, 4, 20, 4)
    tf = st.flops() / (ms_r * 1e-3) / 1e12
    res["down_prefill_M2048"] = {"TFLOP/s": round(tf, 2), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                 "us": round(ms_r * 1e3, 2),
                                 "plain_TFLOP/s": round(st.flops() / (ms_p * 1e-3) / 1e12, 2),
                                 "overhead_pct": round((ms_r - ms_p) / ms_p * 100, 2)}
    del st, L4
    res.update(overhead_vs_k(rl, torch, W, args))
    res.update(model_stack(rl, torch, W, args))
    res.update(prefill_overlap(rl, torch, W, args))
    return res


def attention_decode(rl, torch, W, args):
    """The Qwen2.5-1.5B-shaped attention projections q, k, v, o (D = 1536) at M = 1, 4, 16: the 12
    rotated calls as one paro_linear_batch call per step, and as 12 library calls, over a cold pool."""
    step, pool_bytes = attention_step(rl, torch, W)
    per = 8
    n = max(1, step.n_slots // per) * per

    def timed(rotated, batched):
        return time_slots(torch, lambda s: step.enqueue(s, rotated=rotated, batched=batched), n, per, 200, 200,
                          min_warm_s=0.05)
    ms_rot, ms_plain = timed(True, True), timed(False, True)
    ms_calls_rot, ms_calls_plain = timed(True, False), timed(False, False)
    b = step.bytes(True)
    return {"attention_decode_step": {
        "GB/s": round(b / (ms_rot * 1e-3) / 1e9, 2), "frac_hbm": round(b / (ms_rot * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "us": round(ms_rot * 1e3, 3), "algorithmic_bytes": b, "plain_us": round(ms_plain * 1e3, 3),
        "overhead_pct": round((ms_rot - ms_plain) / ms_plain * 100, 2), "cold_pool_bytes": pool_bytes,
        "separate_calls": {"us": round(ms_calls_rot * 1e3, 3), "plain_us": round(ms_calls_plain * 1e3, 3),
                           "overhead_pct": round((ms_calls_rot - ms_calls_plain) / ms_calls_plain * 100, 2)},
        "launch": "one paro_linear_batch call of the 12 projections per step"}}


def prefill_overlap(rl, torch, W, args):
    """The down_proj prefill (M = 2048) with its rows in C chunks: chunk c + 1 is transformed on a
    second stream while the plain INT4 linear runs on chunk c (paro_rotate, then
    paro_w4a16_linear on the transformed rows; events order each chunk's two steps). Beside it,
    the same chunks one after the other on one stream, and the unchunked fused call. Each variant
    is one HIP graph per step."""
    L4 = Linear(rl, torch, W.make_linear(4, 0))
    M, D, N = 2048, L4.D, L4.N
    x = torch.from_numpy(L4.L.x[:M]).cuda()
    xr = torch.empty_like(x)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    flops = 2.0 * M * D * N
    entry = {}
    st = Step(rl, torch, [L4], [M])
    ms_f = time_slots(torch, lambda s: st.enqueue(s), 4, 4, 20, 4)
    entry["fused_call_us"] = round(ms_f * 1e3, 2)
    side = torch.cuda.Stream()
    for C in (1, 2, 4, 8):
        rows = M // C
        ws = [torch.empty(max(rl.paro_workspace_bytes(rows, D, N), 256), dtype=torch.uint8, device="cuda")
              for _ in range(2)]

        def chunk(c, gemm_ws):
            r = slice(c * rows, (c + 1) * rows)
            rl.paro_w4a16_linear(xr[r], *L4.w, out=y[r], ws=gemm_ws)

        def serial(s):
            for c in range(C):
                r = slice(c * rows, (c + 1) * rows)
                rl.paro_rotate(L4.rot, x[r], out=xr[r])
                chunk(c, ws[0])

        def overlapped(s):
            main = torch.cuda.current_stream()
            side.wait_stream(main)
            done = []
            for c in range(C):  # transforms on the side stream, each chunk's linear on the main one
                r = slice(c * rows, (c + 1) * rows)
                with torch.cuda.stream(side):
                    rl.paro_rotate(L4.rot, x[r], out=xr[r])
                    ev = torch.cuda.Event()
                    ev.record(side)
                done.append(ev)
            for c in range(C):
                main.wait_event(done[c])
                chunk(c, ws[c % 2] if C > 1 else ws[0])
            main.wait_stream(side)

        ms_s = time_slots(torch, serial, 4, 4, 20, 4)
        ms_o = time_slots(torch, overlapped, 4, 4, 20, 4) if C > 1 else ms_s
        entry[f"C{C}"] = {"serial_us": round(ms_s * 1e3, 2), "overlapped_us": round(ms_o * 1e3, 2),
                          "overlapped_TFLOP/s": round(flops / (ms_o * 1e-3) / 1e12, 2)}
    ms_p = time_slots(torch, lambda s: st.enqueue(s, rotated=False), 4, 4, 20, 4)
    entry["plain_us"] = round(ms_p * 1e3, 2)
    best = min(v["overlapped_us"] for k, v in entry.items() if k.startswith("C"))
    entry["best_overhead_pct"] = round((best - ms_p * 1e3) / (ms_p * 1e3) * 100, 2)
    return {"prefill_overlap_down_M2048": entry}


def _with_stages(L, K):
    """The same linear with only the first K of its transform's stages."""
    import dataclasses
    return dataclasses.replace(L, spec=dataclasses.replace(L.spec, K=K), pairs=L.pairs[:K], theta=L.theta[:K])


def overhead_vs_k(rl, torch, W, args):
    """Rotation overhead against the stage count (K = 0, 2, 4, 8) at the gate+up decode shape (M = 1,
    cold pool) and the down_proj prefill shape (M = 2048), next to the dense alternative the pairwise
    stages replace: a D x D float16 rotation applied to x by the vendor GEMM (torch.matmul), then the
    plain INT4 linear."""
    res = {}
    for name, wid, M, per in (("gate_up_decode_M1", 3, 1, 8), ("down_prefill_M2048", 4, 2048, 4)):
        base = W.make_linear(wid, 0)
        entry = {}
        for K in (0, 2, 4, 8):
            lin = Linear(rl, torch, _with_stages(base, K))
            n = max(4, math.ceil(POOL_BYTES / lin.set_bytes())) if M == 1 else 4
            if M == 1:
                lin.make_copies(rl, n)
            st = Step(rl, torch, [lin], [M])
            if K == 0:
                ms_p = time_slots(torch, lambda s: st.enqueue(s, rotated=False), n, per, 2 * n, per)
                entry["plain_us"] = round(ms_p * 1e3, 2)
            ms_r = time_slots(torch, lambda s: st.enqueue(s), n, per, 2 * n, per)
            entry[f"K{K}"] = {"us": round(ms_r * 1e3, 2), "overhead_pct": round((ms_r - ms_p) / ms_p * 100, 2)}
            if K == 8:  # the dense contrast, on the same packed weights and pool
                D = lin.D
                g = torch.Generator(device="cuda").manual_seed(K)
                R = [torch.randn(D, D, device="cuda", generator=g).half() for _ in range(n if M == 1 else 1)]
                x = st.x[(0, M)]
                xr = torch.empty_like(x)

                def dense(s):
                    torch.matmul(x, R[s % len(R)], out=xr)
                    rot, w = st._weights(0, M, s)
                    rl.paro_w4a16_linear(xr, *w, out=st.y[(0, M)], ws=st.ws[(0, M)])
                ms_d = time_slots(torch, dense, n, per, 2 * n, per)
                entry["dense_fp16_rotation"] = {"us": round(ms_d * 1e3, 2),
                                                "overhead_pct": round((ms_d - ms_p) / ms_p * 100, 2),
                                                "rotation_bytes": D * D * 2, "rotation_flop": 2.0 * M * D * D}
                del R
            del st, lin
        res[f"overhead_vs_K_{name}"] = entry
    return res


def model_stack(rl, torch, W, args):
    """The 1.5B-shaped decoder stack (28 layers x q, k, v, o, gate, up, down; every linear with its
    own transform): build throughput (folding, quantizing and packing all 196 weight matrices) and
    the decode step at M = 1 over the whole stack, as one batched call (grouped launches) and as the
    4 dependent launches per layer a decode step makes (q/k/v, o, gate/up, down). The packed stack
    (about 0.8 GB) is three times the Infinity Cache, so each step reads it cold."""
    res = {}
    nl, specs = W.MODEL_LAYERS, W.MODEL_LINEARS
    Ws = [torch.from_numpy(W.make_model_linear(0, i).W).cuda() for i in range(len(specs))]  # shared by layers
    rots, xs = {}, {}
    for l in range(nl):
        for i in range(len(specs)):
            Li = W.make_model_linear(l, i, with_weights=False)
            rots[(l, i)] = rl.paro_rotation_prepare(Li.pairs, Li.theta, Li.scale)
            xs[(l, i)] = torch.from_numpy(Li.x).cuda()
    packed = {k: (torch.empty((specs[k[1]].N, specs[k[1]].D // 2), dtype=torch.uint8, device="cuda"),
                  torch.empty((specs[k[1]].N, specs[k[1]].D // 128), dtype=torch.float16, device="cuda"),
                  torch.empty((specs[k[1]].N, specs[k[1]].D // 128), dtype=torch.float16, device="cuda"))
              for k in rots}
    for i in range(len(specs)):  # warm the pack kernel on every shape
        rl.paro_pack_weights(rots[(0, i)], Ws[i], out=packed[(0, i)])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for (l, i), rot in rots.items():
        rl.paro_pack_weights(rot, Ws[i], out=packed[(l, i)])
    e1.record()
    torch.cuda.synchronize()
    ms_pack = e0.elapsed_time(e1)
    n_w = nl * sum(sp.N * sp.D for sp in specs)
    res["model_build_pack"] = {"linears": len(rots), "weights": n_w, "ms": round(ms_pack, 2),
                               "Gweights/s": round(n_w / (ms_pack * 1e-3) / 1e9, 3),
                               "fp16_in_GB/s": round(2 * n_w / (ms_pack * 1e-3) / 1e9, 2),
                               "packed_bytes": sum(sum(t.numel() * t.element_size() for t in w) for w in packed.values())}
    del Ws
    ys = {k: torch.empty((1, specs[k[1]].N), dtype=torch.float16, device="cuda") for k in rots}
    keys = list(rots)
    bytes_r = sum(workload_bytes(1, specs[i].D, specs[i].N, specs[i].K) for (l, i) in keys)
    bytes_p = sum(workload_bytes(1, specs[i].D, specs[i].N, specs[i].K, rotated=False) for (l, i) in keys)

    def calls(ks, rotated):
        return [(rots[k] if rotated else None, xs[k], *packed[k]) for k in ks]

    grouped = {r: calls(keys, r) for r in (True, False)}
    phases = {r: [calls([(l, i) for i in ph], r) for l in range(nl) for ph in W.MODEL_PHASES] for r in (True, False)}
    ys_all = [ys[k] for k in keys]
    ys_ph = [[ys[(l, i)] for i in ph] for l in range(nl) for ph in W.MODEL_PHASES]

    def run_grouped(rotated):
        rl.paro_linear_batch(grouped[rotated], outs=ys_all)

    def run_layered(rotated):
        for c, o in zip(phases[rotated], ys_ph):
            rl.paro_linear_batch(c, outs=o)

    # The layered order is the decode step a model makes (each layer's linears wait for the
    # previous phase); the grouped one treats all 196 linears as independent calls, which no
    # real decode step can do: it bounds what batching the launches would give.
    for name, fn in (("layered", run_layered), ("grouped", run_grouped)):
        ms_r = time_slots(torch, lambda s: fn(True), 2, 1, 10, 2)
        ms_p = time_slots(torch, lambda s: fn(False), 2, 1, 10, 2)
        gbs = bytes_r / (ms_r * 1e-3) / 1e9
        res[f"model_decode_M1_{name}"] = {
            "GB/s": round(gbs, 2), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "us": round(ms_r * 1e3, 2),
            "algorithmic_bytes": bytes_r, "plain_us": round(ms_p * 1e3, 2),
            "plain_GB/s": round(bytes_p / (ms_p * 1e-3) / 1e9, 2),
            "overhead_pct": round((ms_r - ms_p) / ms_p * 100, 2),
            "realizable_decode_step": name == "layered",
            "launch": "4 dependent paro_linear_batch calls per layer (q/k/v, o, gate/up, down), 112 per step: "
                      "the order of a real decode step" if name == "layered" else
                      "one paro_linear_batch call for all 196 linears as independent calls (not a realizable "
                      "decode step: the layers depend on each other)"}
    return res


if __name__ == "__main__":
    main()
