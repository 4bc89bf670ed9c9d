#!/usr/bin/env python3
"""Throughput of sliced r-bit qgemm on one MI355X.

A step is one pass of the hot path over the Llama-3.1-8B-shaped decoder linears
(qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096; GPTQ-like
8-bit parent codes from N(0, 0.02) weights with absmax group-128 bf16 scales;
X bf16 N(0, 1)) at batch 1: for each child width r in (4, 3, 2), slice the
parent (host-only view) and run qgemm on all four linears -- 12 launches that
read r/8 bytes per weight of bit-planes.  ``value`` is plane bytes read per
second over the timed steps (whole job, inputs resident in HBM).

A decode step is a chain of short launches, so the steps of one rotation over
the parent copies are captured into one HIP graph (a chain of steps, as a
captured multi-layer pass would be) and replayed, with a graph of the first m
steps for the remainder so that exactly --steps steps run (``value``); the same
step launched from Python one call at a time is reported as ``eager``.

Cache rule (everywhere): between two reads of the same bytes at least 600 MB of
other plane data is read, so the 256 MB MALL and the 4 MB L2s never serve a
launch's planes.  A step rotates over ceil(600 MB / smallest r-group) + 1
parent copies; a product timed on its own rotates over ceil(600 MB / its bytes)
+ 1 copies of its r planes and scales.  Per-product durations give every
product of a section the same number of launches (the largest rotation), so a
kernel trace of ``--only SECTION`` averages each kernel over its products the
way the roofline does.

Sections (``--only`` takes a comma list; default all):
  b1       the headline step, eager, per-product durations and read floors, roofline
  grouped  the 12 products as 3 grouped dispatches and as one mixed-precision dispatch;
           batch-16 products grouped
  pack     the packer (once per checkpoint, 1 byte read + 1 written per weight)
  variants asymmetric children and bf16 outputs on the batch-1 step
  choose   the data-free parent-code choice (fp64 brute force)
  b4_16    batch 4 and 16 steps on the same linears
  b256     batch 256, r = 8, 4, 3, 2 (TFLOP/s), per-product durations, roofline, GPU clock
  sweep    batch 32, 64, 128 (r = 8, 4, 3, 2) through the automatic kernel choice
  qwen3    Qwen3-8B-shaped linears, batch 1..256 x r = 6, 4, 3, 2; batch-1 products on their own
  l70      a 70B-shaped layer resident on the GPU, batch 1, 16, 128 x r = 3, 2; batch-1 products
  dense    dense bf16 torch.mm (hipBLASLt) on the Llama linears at batch 1 and 256 (context)
  cpu      the CPU oracle on a bounded sample of the batch-1 step, on all host threads and on one
"""
from __future__ import annotations

import argparse
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sliced int-r qgemm GB/s (batch 1) and TFLOP/s (batch 256) vs roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# fp64 vector issue rate: 78.6 TFLOP/s counts an FMA as two; single fp64 ops
# (add, mul) issue at half that many per second.
FP64_OPS_PEAK_T = 39.3
RS_B1 = (4, 3, 2)
RS_B256 = (8, 4, 3, 2)
RS_QWEN = (6, 4, 3, 2)
RS_70B = (3, 2)
QWEN_BATCHES = (1, 2, 4, 8, 16, 32, 64, 128, 256)
L70_BATCHES = (1, 16, 128)
ROTATE_BYTES = 600_000_000
CPU_SAMPLE_SECONDS = 12.0
CPU_1CORE_SECONDS = 10.0
MIN_STEPS = 20
SECTIONS = ("b1", "grouped", "pack", "variants", "choose", "b4_16", "b256", "sweep", "qwen3", "l70",
            "dense", "cpu")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default="", help="comma list of sections (default: all): " + ",".join(SECTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="leave out the cpu section")
    ap.add_argument("--b1-kernel", default="auto", help="kernel for the batch-1 step (auto, gemv, smallb)")
    ap.add_argument("--pmc-probe", metavar="KIND",
                    help="run only a counter probe (a plain device copy of known size, then a fixed set of "
                         "launches) for rocprofv3 --pmc passes")
    ap.add_argument("--pmc-summary", nargs="+", metavar=("KIND", "DIR"),
                    help="write profiles/counters_KIND.md from the counter_collection.csv folders of the passes")
    ap.add_argument("--trace-summary", nargs=2, metavar=("SECTION", "DIR"),
                    help="write profiles/trace_SECTION.md from a --kernel-trace folder of --only SECTION")
    ap.add_argument("--cpu-only", type=float, default=0.0, metavar="SECONDS",
                    help="(internal) time the CPU oracle alone for about SECONDS and print its record")
    return ap.parse_args()


def rule_copies(nbytes):
    """Copies in a rotation such that >= ROTATE_BYTES of other data is read between two
    reads of the same bytes, when each use reads at least nbytes."""
    return -(-ROTATE_BYTES // max(1, nbytes)) + 1


def make_linears(synth, workload):
    """synth.make_linear for every linear of the workload (threads: numpy's generators and
    array arithmetic release the GIL; every linear keeps its own seeded streams)."""
    from concurrent.futures import ThreadPoolExecutor
    n = len(synth.WORKLOADS[workload])
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(lambda sid: synth.make_linear(workload, sid, 1), range(n)))


class Layer:
    """The linears of one workload, packed on the GPU, in enough parent copies
    for the step rotation over child widths ``rs``."""

    def __init__(self, torch, nbw, synth, workload, rs):
        t = time.time()
        self.workload = workload
        self.wid = synth.WORKLOAD_IDS[workload]
        self.lin = []
        for sid, d in enumerate(make_linears(synth, workload)):
            codes = torch.from_numpy(d["codes"]).cuda()
            w = nbw.pack_bitplanes(codes)
            del codes
            self.lin.append({"sid": sid, "name": d["name"], "n": d["n"], "k": d["k"], "w": [w],
                             "s": [torch.from_numpy(d["scales"]).view(torch.bfloat16).cuda()],
                             "x1": torch.from_numpy(d["x"]).view(torch.bfloat16).cuda()})
            L = self.lin[-1]
            L["y1"] = torch.empty((1, L["n"]), dtype=torch.float32, device="cuda")
        self.parent_bytes = sum(8 * L["w"][0].plane_bytes for L in self.lin)
        smallest = min(sum(r * L["w"][0].plane_bytes + L["n"] * L["k"] // 64 for L in self.lin) for r in rs)
        self.copies = rule_copies(smallest)
        for L in self.lin:
            for _ in range(self.copies - 1):
                st = L["w"][0].storage.clone()
                L["w"].append(nbw.PackedWeight(st, L["n"], L["k"], 8))
                L["s"].append(L["s"][0].clone())
        torch.cuda.synchronize()
        log(f"{workload}: {self.copies} parent copies of {self.parent_bytes / 1e6:.1f} MB "
            f"({time.time() - t:.1f} s)")

    def add_batch(self, torch, synth, b):
        """Activations of batch b for every linear (the recipe's streams; outlier
        channels from batch 32) and fp32 outputs."""
        for L in self.lin:
            if f"x{b}" in L:
                continue
            xb = synth.activations(b, L["k"], synth.rng_for(0, self.wid, L["sid"], synth.T_X),
                                   outliers=b >= 32,
                                   outlier_rng=synth.rng_for(0, self.wid, L["sid"], synth.T_OUTLIERS))
            L[f"x{b}"] = torch.from_numpy(xb).view(torch.bfloat16).cuda()
            L[f"y{b}"] = torch.empty((b, L["n"]), dtype=torch.float32, device="cuda")

    def drop_batch(self, b):
        for L in self.lin:
            L.pop(f"x{b}", None)
            L.pop(f"y{b}", None)

    def release(self):
        self.lin = []


def copy_of(layer, rs, step, ri):
    return (step * len(rs) + ri) % layer.copies


def step_calls(nbw, layer, rs, step, xkey, ykey, kernel):
    """Prepared qgemm calls of one step: every r, every linear, in order."""
    calls = []
    for ri, r in enumerate(rs):
        c = copy_of(layer, rs, step, ri)
        for L in layer.lin:
            calls.append(nbw.QgemmCall(L[xkey], L["w"][c].slice_view(r), L["s"][c], r,
                                       out=L[ykey], kernel=kernel))
    return calls


def capture(torch, fn):
    """fn() captured into a HIP graph (fn launches on the current stream) and
    launched once.

    Python's cycle collector is held off during the capture (after a collection
    outside it): a graph freed by the collector mid-capture would be destroyed
    while the stream captures, which HIP refuses."""
    import gc
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # once eagerly on a side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    try:
        with torch.cuda.graph(g):
            fn()
    finally:
        gc.enable()
    torch.cuda.synchronize()
    g.replay()  # the first launch uploads the graph: part of making it, never timed
    torch.cuda.synchronize()
    return g


def event_time(torch, body, steps):
    """ms per step of body(i) for i in range(steps), HIP events on the current stream."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        body(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


class PeriodGraph:
    """Steps 0..period-1 of a copy rotation captured as ONE graph (a chain of
    steps, as a captured multi-layer pass would be), plus graphs of the first m
    steps for the remainder, so that exactly N steps replay.  (A graph per step
    left a gap of ~4-5 us between consecutive graph launches: 89 against 85 us
    per batch-1 step.)"""

    def __init__(self, torch, step_fn, period):
        self.torch, self.step_fn, self.period = torch, step_fn, period
        self.full = capture(torch, lambda: [step_fn(j) for j in range(period)])
        self.part = {}

    def _part(self, m):
        if m not in self.part:
            self.part[m] = capture(self.torch, lambda: [self.step_fn(j) for j in range(m)])
        return self.part[m]

    def run(self, steps):
        full, rem = divmod(steps, self.period)
        for _ in range(full):
            self.full.replay()
        if rem:
            self._part(rem).replay()

    def time(self, steps, warmup):
        """ms per step over exactly `steps` steps, after `warmup` untimed ones."""
        if warmup:
            self.run(warmup)
        if steps % self.period:
            self._part(steps % self.period)  # captured before the timed region
        return event_time(self.torch, lambda i: self.run(steps), 1) / steps


class Stepper:
    """One step (every r x every linear) as prepared calls and as HIP graphs:
    with ``chain`` the copy rotation's steps as one PeriodGraph (for short,
    launch-bound steps), else one graph per step (step i and step i + copies
    are the same launches, so one graph per residue covers every step)."""

    def __init__(self, torch, nbw, layer, rs, xkey, ykey, kernel="auto", chain=False):
        self.torch = torch
        self.period = layer.copies
        self.calls = [step_calls(nbw, layer, rs, j, xkey, ykey, kernel) for j in range(self.period)]
        # (closures over the calls, not bound methods: no reference cycle
        # through self, so the graphs go as soon as the stepper does)
        calls, period = self.calls, self.period
        self.pg = PeriodGraph(torch, lambda i: [c() for c in calls[i % period]], period) if chain else None
        self.graphs = None if chain else [capture(torch, lambda cl=cl: [c() for c in cl]) for cl in calls]

    def eager(self, i):
        for c in self.calls[i % self.period]:
            c()

    def replay(self, i):
        """Replay step i's graph (with ``chain``: the whole rotation's graph)."""
        if self.pg is not None:
            self.pg.full.replay()
        else:
            self.graphs[i % self.period].replay()

    def time(self, steps, warmup, graph=True):
        if graph and self.pg is not None:
            return self.pg.time(steps, warmup)
        if graph:
            g, P = self.graphs, self.period
            body = lambda i: g[i % P].replay()  # noqa: E731
        else:
            body = self.eager
        for i in range(warmup):
            body(i)
        return event_time(self.torch, lambda i: body(warmup + i), steps)


def timed_step(torch, nbw, layer, rs, batch, steps, warmup, kernel="auto"):
    """ms per step of every (r, linear) product at this batch (chained graph up to batch 16)."""
    st = Stepper(torch, nbw, layer, rs, f"x{batch}", f"y{batch}", kernel, chain=batch <= 16)
    ms = st.time(steps, warmup, graph=True)
    del st
    return ms


def product_durations(torch, nbw, layer, rs, batch, reps, floor=False, kernel="auto"):
    """Back-to-back duration of every (linear, r) product, one at a time.

    Each product rotates over rule_copies(its plane + scale bytes) copies of its r
    planes and scales; every product gets the same number of launches (the largest
    rotation of the section), captured in one graph and replayed ``reps`` times
    between two HIP events.  With ``floor``, a plain streaming read of the same
    plane bytes (nbw_stream_read) over the same copies, timed the same way: the
    time one launch needs to read those bytes and do nothing else.
    Returns {(linear, r): {"us", "n", "k", "kernel", "copies", "floor_us"}}."""
    need = {(L["name"], r): rule_copies(r * L["w"][0].plane_bytes + L["n"] * L["k"] // 64)
            for L in layer.lin for r in rs}
    launches = max(need.values())
    sink = nbw.stream_sink() if floor else None
    out = {}
    for r in rs:
        for L in layer.lin:
            nc = need[(L["name"], r)]
            nb = r * L["w"][0].plane_bytes
            bufs = [L["w"][0].storage[:nb].clone() for _ in range(nc)]
            scs = [L["s"][0].clone() for _ in range(nc)]
            ws = [nbw.PackedWeight(b, L["n"], L["k"], r) for b in bufs]
            calls = [nbw.QgemmCall(L[f"x{batch}"], ws[i % nc], scs[i % nc], r, out=L[f"y{batch}"], kernel=kernel)
                     for i in range(launches)]
            g = capture(torch, lambda cl=calls: [c() for c in cl])
            us = event_time(torch, lambda i: g.replay(), reps) * 1e3 / launches
            del g, calls
            e = {"us": us, "n": L["n"], "k": L["k"], "copies": nc, "launches": launches,
                 "kernel": nbw.kernel_name(batch, L["n"], L["k"], r, kernel)}
            if floor:
                gf = capture(torch, lambda bl=bufs, nb=nb: [nbw.stream_read(bl[i % nc], nb, sink)
                                                          for i in range(launches)])
                e["floor_us"] = event_time(torch, lambda i: gf.replay(), reps) * 1e3 / launches
                del gf
            out[(L["name"], r)] = e
            del ws, bufs, scs
    torch.cuda.synchronize()
    return out


def dominant(durs, batch):
    """Kernel with the largest total time in one step, and its launches' totals."""
    tot = {}
    for (nm, r), d in durs.items():
        t = tot.setdefault(d["kernel"], {"us": 0.0, "launches": 0, "bytes": 0, "flops": 0, "products": []})
        t["us"] += d["us"]
        t["launches"] += 1
        t["bytes"] += r * d["n"] * d["k"] // 8
        t["flops"] += 2 * batch * d["n"] * d["k"]
        t["products"].append((nm, r))
    name, t = max(tot.items(), key=lambda kv: kv[1]["us"])
    return name, t


def b1_products_table(durs):
    out = []
    for (nm, r), d in sorted(durs.items()):
        pb = r * d["n"] * d["k"] // 8
        gbs = pb / (d["us"] * 1e-6) / 1e9
        # planes, plus the scales (2 bytes per 128 weights), X (bf16) and Y (fp32) of one batch row
        eff = pb + d["n"] * d["k"] // 64 + 2 * d["k"] + 4 * d["n"]
        e = {"linear": nm, "r": r, "us": round(d["us"], 2), "GBps": round(gbs, 1),
             "GBps_effective": round(eff / (d["us"] * 1e-6) / 1e9, 1),
             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "ge_5us_at_peak": pb / (HBM_PEAK_GBS * 1e3) >= 5.0,
             "kernel": d["kernel"], "rotation_copies": d["copies"]}
        if "floor_us" in d:
            e["read_floor_us"] = round(d["floor_us"], 2)
            e["frac_of_read_floor"] = round(d["floor_us"] / d["us"], 3)
        out.append(e)
    return out


# ---------------------------------------------------------------- environment

def host_info():
    info = {"rocm": None, "cpu_model": None, "host_threads": None, "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        info["host_threads"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["host_threads"] = os.cpu_count()
    return info


def clock_under_load(torch, replay, ms_per_replay, seconds=1.5):
    """The shader clock, the package power and the power cap rocm-smi reports while ~seconds of replays run."""
    n = max(1, int(seconds * 1e3 / max(ms_per_replay, 1e-3)))
    torch.cuda.synchronize()
    for i in range(n):
        replay(i)
    time.sleep(min(0.5, seconds / 3))
    out = ""
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showmaxpower"], capture_output=True,
                             text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        pass
    torch.cuda.synchronize()
    res = {"sclk_mhz": None, "source": "rocm-smi --showclocks --showpower --showmaxpower during batch-256 replays"}
    for line in out.splitlines():
        low = line.lower()
        if "sclk" in low and res["sclk_mhz"] is None:
            m = re.search(r"(\d+)\s*mhz", line, re.I)
            if m:
                res["sclk_mhz"] = int(m.group(1))
                res["line"] = line.strip()
        elif "max graphics package power" in low:
            m = re.search(r":\s*([\d.]+)\s*$", line.strip())
            if m:
                res["power_cap_w"] = float(m.group(1))
        elif "graphics package power" in low:
            m = re.search(r":\s*([\d.]+)\s*$", line.strip())
            if m:
                res["power_w"] = float(m.group(1))
    return res


# ---------------------------------------------------------------- sections

def section_b1(torch, nbw, synth, args, layer, result):
    bytes_step = sum(r * L["n"] * L["k"] // 8 for r in RS_B1 for L in layer.lin)
    st1 = Stepper(torch, nbw, layer, RS_B1, "x1", "y1", args.b1_kernel, chain=True)
    ms = st1.time(args.steps, args.warmup, graph=True)
    value = bytes_step / (ms * 1e-3) / 1e9
    log(f"batch 1 (graph): {ms * 1e3:.1f} us/step, {value:.1f} GB/s")
    ms_eager = st1.time(args.steps, args.warmup, graph=False)
    log(f"batch 1 (eager): {ms_eager * 1e3:.1f} us/step, {bytes_step / (ms_eager * 1e-3) / 1e9:.1f} GB/s")
    del st1

    durs = product_durations(torch, nbw, layer, RS_B1, 1, reps=max(10, args.steps // 4), floor=True,
                             kernel=args.b1_kernel)
    dom_name, dom = dominant(durs, 1)
    dom_avg_us = dom["us"] / dom["launches"]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    import bench_counters
    traffic = bench_counters.stored_traffic("gemv_b1", [(bench_counters.LLAMA, nm, 1, r) for nm, r in dom["products"]])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic else None,
                "kernel": dom_name, "avg_launch_us": round(dom_avg_us, 2),
                "bytes_per_launch": dom["bytes"] // dom["launches"],
                "launches_per_step": dom["launches"],
                "products": [f"{nm} r={r}" for nm, r in dom["products"]]}
    dom_floor = sum(durs[p]["floor_us"] for p in dom["products"])
    roofline["read_floor_us_per_launch"] = round(dom_floor / dom["launches"], 2)
    roofline["frac_of_read_floor"] = round(dom_floor / dom["us"], 3)
    per_shape = b1_products_table(durs)
    log(f"dominant kernel {dom_name}: {dom_avg_us:.2f} us avg, {achieved:.1f} GB/s; "
        f"a plain read of the same bytes takes {dom_floor / dom['launches']:.2f} us")
    for p in per_shape:
        log(f"  {p['linear']:8s} r={p['r']} {p['us']:7.2f} us {p['GBps']:7.1f} GB/s  "
            f"(read floor {p['read_floor_us']:6.2f} us, {p['frac_of_read_floor']:.2f})  {p['kernel']}")
    result.update({"value": round(value, 1), "ms_per_step": round(ms, 5)})
    result["config"].update({"parent_copies": layer.copies, "bytes_per_step": bytes_step})
    result["roofline"] = roofline
    result["eager"] = {"GBps": round(bytes_step / (ms_eager * 1e-3) / 1e9, 1), "ms_per_step": round(ms_eager, 5),
                       "note": "same step, one Python call per launch, no graph"}
    result["per_shape"] = per_shape
    return bytes_step


def section_grouped(torch, nbw, synth, args, layer, result, bytes_step):
    # the same 12 products as 3 grouped dispatches (one per r over the four linears).
    # Within a real decoder layer the linears depend on each other, so this is
    # reported beside the headline, not as it.
    def grouped_step(step):
        for ri, r in enumerate(RS_B1):
            c = copy_of(layer, RS_B1, step, ri)
            nbw.qgemm_grouped([(L["x1"], L["w"][c].slice_view(r), L["s"][c], r) for L in layer.lin],
                              outs=[L["y1"] for L in layer.lin])
    steps = max(MIN_STEPS, args.steps)
    gpg = PeriodGraph(torch, grouped_step, layer.copies)
    gms = gpg.time(steps, args.warmup)
    del gpg
    result["grouped"] = {"GBps": round(bytes_step / (gms * 1e-3) / 1e9, 1), "ms_per_step": round(gms, 5),
                         "dispatches_per_step": len(RS_B1),
                         "note": "4 linears per dispatch, one dispatch per r; independent products"}
    log(f"batch 1 grouped: {gms * 1e3:.1f} us/step, {result['grouped']['GBps']} GB/s")

    # all 12 products (every linear at every r) as ONE grouped dispatch, each with its own output
    ymix = {(L["name"], r): torch.empty((1, L["n"]), dtype=torch.float32, device="cuda")
            for L in layer.lin for r in RS_B1}

    def mixed_step(step):
        items, outs = [], []
        for ri, r in enumerate(RS_B1):
            c = copy_of(layer, RS_B1, step, ri)
            for L in layer.lin:
                items.append((L["x1"], L["w"][c].slice_view(r), L["s"][c], r))
                outs.append(ymix[(L["name"], r)])
        nbw.qgemm_grouped(items, outs=outs)
    mpg = PeriodGraph(torch, mixed_step, layer.copies)
    mms = mpg.time(steps, args.warmup)
    del mpg, ymix
    result["grouped_mixed"] = {"GBps": round(bytes_step / (mms * 1e-3) / 1e9, 1), "ms_per_step": round(mms, 5),
                               "dispatches_per_step": 1,
                               "note": "the 12 products (4 linears x r = 4, 3, 2) in one dispatch; "
                                       "independent products"}
    log(f"batch 1 grouped, one mixed-precision dispatch: {mms * 1e3:.1f} us/step, "
        f"{result['grouped_mixed']['GBps']} GB/s")

    # batch 16: the 12 products in one grouped call against the same 12 products launched one by one
    b = 16
    layer.add_batch(torch, synth, b)
    y16 = {(L["name"], r): torch.empty((b, L["n"]), dtype=torch.float32, device="cuda")
           for L in layer.lin for r in RS_B1}

    def mixed16(step):
        items, outs = [], []
        for ri, r in enumerate(RS_B1):
            c = copy_of(layer, RS_B1, step, ri)
            for L in layer.lin:
                items.append((L[f"x{b}"], L["w"][c].slice_view(r), L["s"][c], r))
                outs.append(y16[(L["name"], r)])
        nbw.qgemm_grouped(items, outs=outs)
    pg16 = PeriodGraph(torch, mixed16, layer.copies)
    ms16 = pg16.time(steps, args.warmup)
    del pg16, y16
    ms16_single = timed_step(torch, nbw, layer, RS_B1, b, steps, args.warmup)
    result["grouped_b16"] = {"GBps": round(bytes_step / (ms16 * 1e-3) / 1e9, 1), "ms_per_step": round(ms16, 5),
                             "single_launches_GBps": round(bytes_step / (ms16_single * 1e-3) / 1e9, 1),
                             "single_launches_ms_per_step": round(ms16_single, 5),
                             "note": "the 12 batch-16 products (4 linears x r = 4, 3, 2) through one grouped call "
                                     "against the same products launched one by one"}
    log(f"batch 16 grouped: {ms16 * 1e3:.1f} us/step ({result['grouped_b16']['GBps']} GB/s) against "
        f"{ms16_single * 1e3:.1f} us launched one by one")


def section_pack(torch, nbw, layer, result):
    L0 = layer.lin
    codes = [torch.randint(0, 256, (L["n"], L["k"]), dtype=torch.uint8, device="cuda") for L in L0]
    copies = rule_copies(min(2 * L["n"] * L["k"] for L in L0))
    outs = [[torch.empty(8 * L["w"][0].plane_bytes, dtype=torch.uint8, device="cuda")
             for _ in range(max(1, copies // 4))] for L in L0]
    for c, o in zip(codes, outs):
        nbw.pack_bitplanes(c, out=o[0])

    def pack_all(i):
        for c, o in zip(codes, outs):
            nbw.pack_bitplanes(c, out=o[i % len(o)])
    pms = event_time(torch, pack_all, 8)
    pack_gbs = sum(2 * L["n"] * L["k"] for L in L0) / (pms * 1e-3) / 1e9
    result["pack"] = {"GBps": round(pack_gbs, 1), "frac_hbm": round(pack_gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_weight": 2}
    del codes, outs
    log(f"pack: {pack_gbs:.1f} GB/s")


def section_variants(torch, nbw, synth, args, layer, result, bytes_step):
    zrng = synth.rng_for(0, layer.wid, 0, synth.T_WEIGHTS)
    for L in layer.lin:
        z = zrng.integers(96, 160, size=(L["n"], L["k"] // 128)).astype("float32")
        L["z"] = torch.from_numpy(synth.f32_to_bf16_bits(z)).view(torch.bfloat16).cuda()
        L["y1b"] = torch.empty((1, L["n"]), dtype=torch.bfloat16, device="cuda")

    def variant_step(i, **kw):
        for ri, r in enumerate(RS_B1):
            c = copy_of(layer, RS_B1, i, ri)
            for L in layer.lin:
                out = L["y1b"] if kw.get("out_dtype") is torch.bfloat16 else L["y1"]
                nbw.qgemm(L["x1"], L["w"][c].slice_view(r), L["s"][c], r, out=out,
                          zeros=L["z"] if kw.get("asym") else None,
                          out_dtype=kw.get("out_dtype", torch.float32))
    variants = {}
    for name, kw in (("asymmetric", {"asym": True}), ("bf16_out", {"out_dtype": torch.bfloat16})):
        vpg = PeriodGraph(torch, lambda j, kw=kw: variant_step(j, **kw), layer.copies)
        vms = vpg.time(max(MIN_STEPS, args.steps // 4), 5)
        variants[name] = {"GBps": round(bytes_step / (vms * 1e-3) / 1e9, 1), "ms_per_step": round(vms, 5)}
        del vpg
        log(f"batch 1 {name}: {variants[name]['GBps']} GB/s")
    result["variants_b1"] = variants


def section_choose(torch, nbw, layer, result):
    # data-free parent-code choice (offline, like pack): weights per second on the
    # gate_up matrix, fp64 brute force over 256 codes x widths (3, 4, 8)
    Lg = [L for L in layer.lin if L["name"] == "gate_up"][0]
    gen = torch.Generator(device="cuda").manual_seed(0)
    wf = torch.randn((Lg["n"], Lg["k"]), device="cuda", generator=gen) * 0.02  # N(0, 0.02) weights
    nbw.choose_codes(wf, Lg["s"][0])
    cms = event_time(torch, lambda i: nbw.choose_codes(wf, Lg["s"][0]), 3)
    nweights = Lg["n"] * Lg["k"]
    # fp64 arithmetic per (code, width): q + 1/2, - 2^(r-1), x s*2^(8-r), w - d, square,
    # x lambda, + loss (7; s*2^(8-r) is per weight and width, q's conversion is not counted)
    ops = nweights * 256 * 3 * 7
    result["choose_codes"] = {
        "weights_per_s": round(nweights / (cms * 1e-3), 1), "ms": round(cms, 3),
        "shape": [Lg["n"], Lg["k"]], "widths": [3, 4, 8],
        "roofline": {"bound": "alu", "achieved": round(ops / (cms * 1e-3) / 1e12, 2),
                     "peak": FP64_OPS_PEAK_T, "unit": "T fp64 op/s",
                     "frac": round(ops / (cms * 1e-3) / 1e12 / FP64_OPS_PEAK_T, 4)}}
    del wf
    log(f"choose_codes: {cms:.2f} ms for {nweights} weights")


def section_b4_16(torch, nbw, synth, args, layer, result, bytes_step):
    other = {}
    for b in (4, 16):
        layer.add_batch(torch, synth, b)
        msb = timed_step(torch, nbw, layer, RS_B1, b, max(MIN_STEPS, args.steps // 4), 5)
        other[f"batch{b}"] = {"GBps": round(bytes_step / (msb * 1e-3) / 1e9, 1), "ms_per_step": round(msb, 5),
                              "kernels": sorted({nbw.kernel_name(b, L["n"], L["k"], r) for r in RS_B1
                                                 for L in layer.lin})}
        log(f"batch {b}: {other[f'batch{b}']['GBps']} GB/s")
    result["other_batches"] = other


def mfma_rate_context(torch, nbw, reps=5):
    """The matrix-unit rate loop (nbw_mfma_rate: v_mfma_f32_32x32x16_bf16 and nothing else, two waves per
    SIMD on every compute unit) with random N(0, 1) bf16 operands and with all operands 1.0: the ceiling
    the large-batch products meet on this chip and their kind of data (the clock under this load depends
    on the data)."""
    gen = torch.Generator(device="cuda").manual_seed(0)
    n = nbw.MFMA_RATE_OPS_BYTES // 2
    operands = {"random": torch.randn(n, device="cuda", generator=gen).to(torch.bfloat16),
                "constant": torch.ones(n, device="cuda", dtype=torch.bfloat16)}
    sink = nbw.mfma_rate_sink()
    iters = 1000
    flops = nbw.mfma_rate_flops(sink, iters)
    out = {}
    for name, ops in operands.items():
        nbw.mfma_rate(ops, 20, sink)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            nbw.mfma_rate(ops, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[f"{name}_TFLOPs"] = round(flops / (us * 1e-6) / 1e12, 1)
    out["frac_of_peak_random"] = round(out["random_TFLOPs"] / BF16_PEAK_TFLOPS, 4)
    out["note"] = ("nbw_mfma_rate: 64 v_mfma_f32_32x32x16_bf16 per wave and round, four accumulator chains, "
                   "operands cycling through 8 A and 8 B register fragments, no memory traffic")
    return out


def section_b256(torch, nbw, synth, args, layer, result):
    B = 256
    layer.add_batch(torch, synth, B)
    flops_step = sum(2 * B * L["n"] * L["k"] for _ in RS_B256 for L in layer.lin)
    st = Stepper(torch, nbw, layer, RS_B256, f"x{B}", f"y{B}")
    steps = max(MIN_STEPS, args.steps // 4)
    ms = st.time(steps, 3, graph=True)
    tflops = flops_step / (ms * 1e-3) / 1e12
    clock = clock_under_load(torch, st.replay, ms)
    del st
    d256 = product_durations(torch, nbw, layer, RS_B256, B, reps=3)
    name, t = dominant(d256, B)
    ach = t["flops"] / (t["us"] * 1e-6) / 1e12
    import bench_counters
    traffic = bench_counters.stored_traffic("gemm_b256", [(bench_counters.LLAMA, nm, B, r) for nm, r in t["products"]])
    mrate = mfma_rate_context(torch, nbw)
    result["batch256"] = {
        "TFLOPs": round(tflops, 2), "frac_mfma": round(tflops / BF16_PEAK_TFLOPS, 4), "ms_per_step": round(ms, 5),
        "frac_of_mfma_rate": round(tflops / mrate["random_TFLOPs"], 4),
        "steps": steps, "r": list(RS_B256),
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": round(traffic) if traffic else None,
                     "kernel": name, "avg_launch_us": round(t["us"] / t["launches"], 2),
                     "flops_per_launch": t["flops"] // t["launches"],
                     "products": [f"{nm} r={r}" for nm, r in t["products"]],
                     "note": "a launch is the product's dispatch plus its second-pass add where k is split",
                     "frac_of_mfma_rate": round(ach / mrate["random_TFLOPs"], 4)},
        "gpu_clock": clock,
        "mfma_rate": mrate,
        "per_shape": [{"linear": nm, "r": r, "us": round(d["us"], 2),
                       "TFLOPs": round(2 * B * d["n"] * d["k"] / (d["us"] * 1e-6) / 1e12, 1),
                       "kernel": d["kernel"]}
                      for (nm, r), d in sorted(d256.items())]}
    log(f"batch 256: {tflops:.1f} TFLOP/s over {steps} steps; {name} {ach:.1f} TFLOP/s; clock {clock.get('sclk_mhz')}; "
        f"matrix-unit rate loop {mrate['random_TFLOPs']} TFLOP/s (random operands), {mrate['constant_TFLOPs']} (constant)")
    layer.drop_batch(B)


def section_sweep(torch, nbw, synth, args, layer, result):
    # batch 32, 64, 128 (r = 8, 4, 3, 2; activations with outlier channels) through the
    # automatic kernel choice
    sweep = {}
    for b in (32, 64, 128):
        layer.add_batch(torch, synth, b)
        msb = timed_step(torch, nbw, layer, RS_B256, b, max(MIN_STEPS, args.steps // 4), 3)
        sweep[f"batch{b}"] = step_record(nbw, layer, RS_B256, b, msb)
        layer.drop_batch(b)
        log(f"batch {b}: {sweep[f'batch{b}']}")
    result["batch_sweep"] = sweep


def step_record(nbw, layer, rs, b, ms):
    fl = sum(2 * b * L["n"] * L["k"] for _ in rs for L in layer.lin)
    pb = sum(r * L["n"] * L["k"] // 8 for r in rs for L in layer.lin)
    fams = sorted({nbw.kernel_name(b, L["n"], L["k"], r).split("<")[0].replace("nbw::", "")
                   for r in rs for L in layer.lin})
    tf = fl / (ms * 1e-3) / 1e12
    gbs = pb / (ms * 1e-3) / 1e9
    return {"ms_per_step": round(ms, 5), "plane_GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOPs": round(tf, 1), "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4), "kernels": fams}


def section_config(torch, nbw, synth, args, workload, rs, batches, label):
    """A whole workload: one step (every linear x every r) per batch, then the batch-1
    products on their own with their read floors."""
    layer = Layer(torch, nbw, synth, workload, rs)
    out = {"workload": workload, "r": list(rs), "parent_copies": layer.copies,
           "plane_bytes_per_step": sum(r * L["n"] * L["k"] // 8 for r in rs for L in layer.lin),
           "batches": {}}
    for b in batches:
        layer.add_batch(torch, synth, b)
        ms = timed_step(torch, nbw, layer, rs, b, max(MIN_STEPS, args.steps // 4), 3)
        out["batches"][f"batch{b}"] = step_record(nbw, layer, rs, b, ms)
        log(f"{label} batch {b}: {out['batches'][f'batch{b}']}")
        if b != 1:
            layer.drop_batch(b)
    durs = product_durations(torch, nbw, layer, rs, 1, reps=5, floor=True)
    out["b1_products"] = b1_products_table(durs)
    for e in out["b1_products"]:
        log(f"{label} b1 {e['linear']} r={e['r']}: {e['us']} us, {e['GBps']} GB/s, {e['frac_hbm']:.3f} of HBM, "
            f"{e['frac_of_read_floor']:.3f} of the read floor")
    layer.release()
    del layer
    torch.cuda.empty_cache()
    return out


def dense_context(torch, layer, result):
    """Dense bf16 Y = X . W^T per Llama-3.1-8B linear at batch 1 and 256 (torch.mm on contiguous
    operands, W^T stored [k][n]), graph-replayed over weight copies; beside it the sliced products'
    times from this run and the speedup over dense."""
    gen = torch.Generator(device="cuda").manual_seed(0)
    ours = {}
    for e in result.get("per_shape", []):
        ours[(e["linear"], e["r"], 1)] = e["us"]
    for e in result.get("batch256", {}).get("per_shape", []):
        ours[(e["linear"], e["r"], 256)] = e["us"]
    out = []
    for L in layer.lin:
        n, k = L["n"], L["k"]
        copies = rule_copies(2 * n * k)
        wts = [(torch.randn((k, n), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
               for _ in range(copies)]
        for b in (1, 256):
            x = torch.randn((b, k), device="cuda", generator=gen).to(torch.bfloat16)
            y = torch.empty((b, n), dtype=torch.bfloat16, device="cuda")
            g = capture(torch, lambda wl=wts, xx=x, yy=y: [torch.mm(xx, wt, out=yy) for wt in wl])
            us = event_time(torch, lambda i: g.replay(), 3) * 1e3 / copies
            del g
            e = {"linear": L["name"], "batch": b, "dense_us": round(us, 2),
                 "dense_TFLOPs": round(2 * b * n * k / (us * 1e-6) / 1e12, 1)}
            e["speedup_of_sliced_by_r"] = {str(r): round(us / ours[(L["name"], r, b)], 2)
                                           for (nm, r, bb) in sorted(ours) if nm == L["name"] and bb == b}
            out.append(e)
        del wts
        torch.cuda.empty_cache()
    return out


def cpu_sample(synth, seconds):
    """The CPU oracle, as it stands, on the batch-1 step's products in step order,
    repeated until ``seconds`` have passed; plane bytes of the completed products
    per second."""
    import oracle

    wl = "llama3.1-8b"
    ins = [(d, oracle.pack(d["codes"])) for d in make_linears(synth, wl)]
    t0 = time.time()
    total = products = 0
    while time.time() - t0 < seconds:
        for r in RS_B1:
            for d, planes in ins:
                oracle.qgemm(d["x"], planes, d["scales"], d["n"], d["k"], r)
                total += r * d["n"] * d["k"] // 8
                products += 1
                if time.time() - t0 >= seconds:
                    break
            else:
                continue
            break
    dt = time.time() - t0
    return {"value": round(total / dt / 1e9, 4), "seconds": round(dt, 2), "products": products}


def start_one_core_oracle():
    """The one-thread oracle sample in a child process (OMP_NUM_THREADS=1), started
    before this process touches the GPU; it runs on one host core beside the GPU
    sections and is collected by cpu_baseline."""
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        return subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-only", str(CPU_1CORE_SECONDS)],
                                stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env)
    except OSError:
        return None


def cpu_baseline(synth, one_core_proc):
    one = {"value": None, "unit": "GB/s", "cores": 1}
    if one_core_proc is not None:
        try:
            out, _ = one_core_proc.communicate(timeout=int(CPU_1CORE_SECONDS * 6 + 60))
            rec = json.loads(out.strip().splitlines()[-1])
            one.update({"value": rec["value"], "seconds": rec["seconds"], "products": rec["products"]})
            log(f"cpu oracle, 1 thread: {rec['products']} products in {rec['seconds']} s, {rec['value']} GB/s")
        except (subprocess.SubprocessError, ValueError, IndexError, KeyError) as e:
            one_core_proc.kill()
            one["error"] = str(e)[:200]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    s = cpu_sample(synth, CPU_SAMPLE_SECONDS)
    log(f"cpu oracle: {s['products']} products in {s['seconds']} s, {s['value']} GB/s on {threads} threads")
    return {"value": s["value"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": s["seconds"], "products": s["products"],
            "sample": f"{s['products']} batch-1 products of the step (Llama-3.1-8B linears qkv, o, gate_up, down "
                      "x r = 4, 3, 2 in step order, repeated), fp64 oracle (oracle/nbw_oracle.c, OpenMP over "
                      "output rows)",
            "cpu_model": host_info()["cpu_model"], "one_core": one}


def main():
    args = parse()
    if args.pmc_summary:
        import bench_counters
        bench_counters.pmc_summary(args.pmc_summary[0], args.pmc_summary[1:])
        return
    if args.trace_summary:
        import bench_counters
        sec, folder = args.trace_summary
        bench_counters.trace_summary(
            sec, folder, f"rocprofv3 --kernel-trace --stats -f csv -d {folder} -- python3 bench.py --only {sec} "
                         "--steps 20 --warmup 5")
        return
    if args.cpu_only:
        import synth
        print(json.dumps(cpu_sample(synth, args.cpu_only)), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    only = set(s for s in args.only.split(",") if s) or set(SECTIONS)
    unknown = only - set(SECTIONS)
    if unknown:
        raise SystemExit(f"unknown sections {sorted(unknown)}; known: {', '.join(SECTIONS)}")
    if args.no_cpu_baseline or args.pmc_probe:
        only.discard("cpu")
    one_core = start_one_core_oracle() if "cpu" in only else None

    import torch

    import nested_bit_weight_amd as nbw
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    nbw.library()  # fails loudly if the HIP library is not built
    log(f"libnbw {nbw.version()} on {torch.cuda.get_device_name(0)}")

    if args.pmc_probe:
        import bench_counters
        bench_counters.run_probe(torch, nbw, args.pmc_probe)
        return

    result = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic",
              "config": {"workload": "llama3.1-8b decoder linears qkv/o/gate_up/down, batch 1, "
                                     "r=4,3,2 (12 qgemm launches per step, HIP graph replay)",
                         "batch": 1, "r": list(RS_B1)},
              "sections": sorted(only, key=SECTIONS.index),
              "host": host_info(), "library": nbw.version()}

    llama_secs = {"b1", "grouped", "pack", "variants", "choose", "b4_16", "b256", "sweep", "dense"}
    layer = Layer(torch, nbw, synth, "llama3.1-8b", RS_B1) if only & llama_secs else None
    bytes_step = sum(r * L["n"] * L["k"] // 8 for r in RS_B1 for L in layer.lin) if layer else 0
    if "b1" in only:
        section_b1(torch, nbw, synth, args, layer, result)
    if "grouped" in only:
        section_grouped(torch, nbw, synth, args, layer, result, bytes_step)
    if "pack" in only:
        section_pack(torch, nbw, layer, result)
    if "variants" in only:
        section_variants(torch, nbw, synth, args, layer, result, bytes_step)
    if "choose" in only:
        section_choose(torch, nbw, layer, result)
    if "b4_16" in only:
        section_b4_16(torch, nbw, synth, args, layer, result, bytes_step)
    if "b256" in only:
        section_b256(torch, nbw, synth, args, layer, result)
    if "sweep" in only:
        section_sweep(torch, nbw, synth, args, layer, result)
    if "dense" in only:
        result["dense_bf16"] = dense_context(torch, layer, result)
    if layer is not None:
        layer.release()
        del layer
        torch.cuda.empty_cache()
    large = []
    if "qwen3" in only:
        result["qwen3_8b"] = section_config(torch, nbw, synth, args, "qwen3-8b", RS_QWEN, QWEN_BATCHES, "qwen3-8b")
        large += [dict(e, linear="qwen3-8b " + e["linear"]) for e in result["qwen3_8b"]["b1_products"]
                  if e["ge_5us_at_peak"]]
    if "l70" in only:
        result["llama_70b_layer"] = section_config(torch, nbw, synth, args, "llama-70b", RS_70B, L70_BATCHES, "70b")
        large += [dict(e, linear="70b " + e["linear"]) for e in result["llama_70b_layer"]["b1_products"]
                  if e["ge_5us_at_peak"]]
    if large:
        result["large_b1"] = large
    if "cpu" in only:
        result["cpu_baseline"] = cpu_baseline(synth, one_core)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
