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
step launched from Python one call at a time is reported as ``eager``.  Packing is once per
checkpoint and is timed separately (``pack`` field).

To measure HBM and not the 256 MB MALL, every (step, r) uses its own parent
copy from a rotation of copies totalling >1.2 GB.

Extra fields: per-kernel durations (each product replayed back to back in a
graph over the copy rotation, HIP events around the replays) giving the
dominant kernel's roofline, and beside each product the time a plain streaming
read of the same plane bytes takes in one launch (nbw_stream_read, same rotation
and timing: the floor a launch of that size cannot beat, well under the 8 TB/s
peak for tens of MB); the 12 products as 3 grouped dispatches, and as one
mixed-precision dispatch (``grouped_mixed``); batch 4
and 16 on the same linears; batch 256 (TFLOP/s, r in 8, 4, 3, 2, activations
with 1% outlier channels x10) and the rest of that sweep, batch 32, 64 and 128
through the automatic kernel choice (``batch_sweep``); batch 1 on the largest single linears (70B-shaped
gate_up and down, Qwen3-8B-shaped gate_up: plane bytes worth >= 5 us at the HBM
peak) with their read floors (``large_b1``); dense bf16 torch.matmul (hipBLASLt) on
the Llama linears at batch 1 and 256 with the sliced products' speedup over it
(``dense_bf16``, context only); the CPU oracle timed on this host on a bounded sample
of the batch-1 step.
"""
from __future__ import annotations

import argparse
import json
import os
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
CPU_SAMPLE_SECONDS = 12.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip batch 4/16/256 and pack timing")
    ap.add_argument("--copies", type=int, default=0, help="parent copies in the rotation (0 = auto)")
    ap.add_argument("--b1-kernel", default="auto", help="kernel for the batch-1 step (auto, gemv, smallb)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run only a plain device copy of known size and the dominant batch-1 "
                         "kernel's launches (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="derive per-launch HBM traffic from two rocprofv3 --pmc output folders "
                         "of --pmc-probe and write it under profiles/")
    ap.add_argument("--pmc-rbits", action="store_true",
                    help="run only a plain device copy and the batch-1 gate_up product at r = 1..8 "
                         "(for a rocprofv3 --pmc FETCH_SIZE pass)")
    ap.add_argument("--rbits-from", metavar="FETCH_DIR",
                    help="bytes fetched per child width from a FETCH_SIZE pass of --pmc-rbits, "
                         "written under profiles/")
    return ap.parse_args()


class Layer:
    """Four linears of one workload, packed on the GPU, in several parent copies."""

    def __init__(self, torch, nbw, synth, workload, copies):
        self.lin = []
        for sid, (name, n, k) in enumerate(synth.WORKLOADS[workload]):
            d = synth.make_linear(workload, sid, 1)
            codes = torch.from_numpy(d["codes"]).cuda()
            w = nbw.pack_bitplanes(codes)
            del codes
            self.lin.append({"name": name, "n": n, "k": k, "w": [w],
                             "s": [torch.from_numpy(d["scales"]).view(torch.bfloat16).cuda()],
                             "x1": torch.from_numpy(d["x"]).view(torch.bfloat16).cuda()})
        parent_bytes = sum(8 * L["w"][0].plane_bytes for L in self.lin)
        if copies <= 0:
            copies = max(6, -(-int(1.2e9) // parent_bytes))
        for L in self.lin:
            for _ in range(copies - 1):
                st = L["w"][0].storage.clone()
                L["w"].append(nbw.PackedWeight(st, L["n"], L["k"], 8))
                L["s"].append(L["s"][0].clone())
        self.copies = copies
        self.parent_bytes = parent_bytes
        torch.cuda.synchronize()


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


# Rotations of the parent copies captured into one graph where a single
# product is timed back to back (per-product durations, read floors, the large
# linears, the dense context).  One: measured on one box, graphs of four
# rotations made the 70B-shaped gate_up at r = 3 20% slower (47.5-49.8 against
# 39.7-41.5 us) with the same read floor, and batch-256 products ~10% slower.
# The batch-1, -4 and -16 steps do run as chains of steps (PeriodGraph): there
# the same-box comparison favoured the chain (86.5-87.2 against 89.0 us).
GRAPH_ROTATIONS = 1


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


def kernel_durations(torch, nbw, layer, rs, xkey, ykey, batch, kernel, reps, rotations=1):
    """Back-to-back duration of every product of the step.

    For each (linear, r) a graph holds that product once per parent copy (so no
    launch re-reads what the previous one left in cache), ``rotations`` times
    over; the graph is replayed ``reps`` times between two HIP events.  Returns
    {(linear, r): us per launch}."""
    out = {}
    for r in rs:
        for L in layer.lin:
            calls = [nbw.QgemmCall(L[xkey], L["w"][c].slice_view(r), L["s"][c], r, out=L[ykey],
                                   kernel=kernel) for c in range(layer.copies)]
            g = capture(torch, lambda cl=calls: [c() for _ in range(rotations) for c in cl])
            ms = event_time(torch, lambda i: g.replay(), reps)
            out[(L["name"], r)] = {"us": ms * 1e3 / (len(calls) * rotations), "n": L["n"], "k": L["k"],
                                   "kernel": nbw.kernel_name(batch, L["n"], L["k"], r, kernel)}
            del g
    return out


def stream_floor(torch, nbw, layer, rs, reps):
    """Back-to-back duration of a plain streaming read of each product's plane bytes.

    The same rotation and timing as kernel_durations, with the library's
    streaming-read reference (nbw_stream_read) in place of the product: the
    time one launch needs to read those bytes and do nothing else.  Returns
    {(linear, r): us per launch}."""
    sink = nbw.stream_sink()
    out = {}
    for r in rs:
        for L in layer.lin:
            nbytes = r * L["w"][0].plane_bytes
            bufs = [L["w"][c].storage for c in range(layer.copies)]
            g = capture(torch, lambda bl=bufs, nb=nbytes: [nbw.stream_read(b, nb, sink)
                                                           for _ in range(GRAPH_ROTATIONS) for b in bl])
            g.replay()
            ms = event_time(torch, lambda i: g.replay(), reps)
            out[(L["name"], r)] = ms * 1e3 / (len(bufs) * GRAPH_ROTATIONS)
            del g
    return out


def dominant(durs, batch):
    """Kernel with the largest total time in one step, and its launches' totals."""
    tot = {}
    for (nm, r), d in durs.items():
        t = tot.setdefault(d["kernel"], {"us": 0.0, "launches": 0, "bytes": 0, "flops": 0})
        t["us"] += d["us"]
        t["launches"] += 1
        t["bytes"] += r * d["n"] * d["k"] // 8
        t["flops"] += 2 * batch * d["n"] * d["k"]
    name, t = max(tot.items(), key=lambda kv: kv[1]["us"])
    return name, t


# ---------------------------------------------------------------- HBM traffic
#
# rocprofv3's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the
# same counters read for a plain device copy of known size.  The probe launches
# the dominant batch-1 kernel on the shapes it runs in the step (r = 4:
# gate_up and down), each from its own parent copy.

PROBE_COPY_BYTES = 512 << 20
PROBE_SHAPES = ("gate_up", "down")
PROBE_R = 4
PROBE_LAUNCHES = 6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_r4_b1.txt")
KERNEL_SOURCES = ("nested_bit_weight_amd/csrc/gemv.hip", "nested_bit_weight_amd/csrc/decode.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_probe(torch, nbw, synth):
    src = torch.empty(PROBE_COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)  # the reference dispatch: PROBE_COPY_BYTES read + written
    torch.cuda.synchronize()
    del src, dst
    layer = Layer(torch, nbw, synth, "llama3.1-8b", PROBE_LAUNCHES)
    for L in layer.lin:
        if L["name"] not in PROBE_SHAPES:
            continue
        y = torch.empty((1, L["n"]), dtype=torch.float32, device="cuda")
        for c in range(layer.copies):
            nbw.qgemm(L["x1"], L["w"][c].slice_view(PROBE_R), L["s"][c], PROBE_R, out=y)
            torch.cuda.synchronize()
    log(f"pmc probe: copy {PROBE_COPY_BYTES} B; kernel {nbw.kernel_name(1, 28672, 4096, PROBE_R)} "
        f"x {PROBE_LAUNCHES} on {PROBE_SHAPES}")


RBITS_FILE = os.path.join(ROOT, "profiles", "fetch_by_r_gemv_gate_up_b1.txt")
RBITS_RS = (1, 2, 3, 4, 5, 6, 7, 8)


def pmc_rbits_probe(torch, nbw, synth):
    """The reference copy, then the batch-1 product on the Llama-3.1-8B gate_up
    linear at every child width, one launch per parent copy (for a FETCH_SIZE
    pass: bytes fetched from memory against r/8 bytes per weight)."""
    src = torch.empty(PROBE_COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    layer = Layer(torch, nbw, synth, "llama3.1-8b", PROBE_LAUNCHES)
    L = next(L for L in layer.lin if L["name"] == "gate_up")
    y = torch.empty((1, L["n"]), dtype=torch.float32, device="cuda")
    for r in RBITS_RS:
        for c in range(layer.copies):
            nbw.qgemm(L["x1"], L["w"][c].slice_view(r), L["s"][c], r, out=y)
            torch.cuda.synchronize()
    log(f"pmc r-bits probe: copy {PROBE_COPY_BYTES} B; gate_up batch 1, r = {RBITS_RS}, "
        f"{layer.copies} launches each")


def rbits_from(fetch_dir):
    import synth
    rows = _pmc_rows(fetch_dir, "FETCH_SIZE")
    copy = [v for _, name, v in rows if "copybuffer" in name.lower()]
    if not copy:
        raise SystemExit(f"the reference copy is not in {fetch_dir}")
    factor = PROBE_COPY_BYTES / (max(copy) * 1024.0)
    n, k = next((n, k) for nm, n, k in synth.WORKLOADS["llama3.1-8b"] if nm == "gate_up")
    lines = [
        f"# Bytes fetched from memory by the batch-1 product on the Llama-3.1-8B gate_up linear ({n} x {k}) at each child width",
        "",
        "Commands (repository root, one MI355X):",
        "  rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_rbits -- python3 bench.py --pmc-rbits",
        "  python3 bench.py --rbits-from gpurun_out/pmc_rbits",
        "",
        f"FETCH_SIZE scaled by what it reads for a plain copy of {PROBE_COPY_BYTES} bytes: factor {factor:.4f}",
        "planes = r n k / 8 bytes; scales = n k / 64 bytes (bf16, one per 128 weights); X = 2 k bytes",
        "",
        "| r | kernel | launches | fetched bytes | planes + scales + X | fetched / (planes + scales + X) | fetched / planes |",
        "|---|---|---|---|---|---|---|",
    ]
    for r in RBITS_RS:
        kern = [(name, v) for _, name, v in rows if f"gemv_kernel<{r}," in name]
        if not kern:
            raise SystemExit(f"r={r}: no gemv_kernel<{r}, *> dispatches in {fetch_dir}")
        avg = sum(v for _, v in kern) / len(kern) * 1024.0 * factor
        planes = r * n * k // 8
        expect = planes + n * k // 64 + 2 * k
        kname = kern[0][0].split("(")[0].replace("void ", "")
        lines.append(f"| {r} | `{kname}` | {len(kern)} | {avg:.0f} | {expect} | {avg / expect:.4f} | {avg / planes:.4f} |")
    with open(RBITS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_rows(folder, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    out = []
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    out.append((int(row["Dispatch_Id"]), row["Kernel_Name"], float(row["Counter_Value"])))
    return sorted(out)


def traffic_from(fetch_dir, write_dir):
    import synth
    res = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(folder, counter)
        copy = [v for _, name, v in rows if "copybuffer" in name.lower()]
        kern = [v for _, name, v in rows if "gemv_kernel<4" in name]
        if not copy or not kern:
            raise SystemExit(f"{counter}: probe dispatches not found in {folder}")
        factor = PROBE_COPY_BYTES / (max(copy) * 1024.0)
        res[counter] = {"copy_kib": max(copy), "factor": factor,
                        "kernel_kib_avg": sum(kern) / len(kern), "launches": len(kern),
                        "kernel_bytes_avg": sum(kern) / len(kern) * 1024.0 * factor}
    shapes = {nm: (n, k) for nm, n, k in synth.WORKLOADS["llama3.1-8b"]}
    alg = sum(PROBE_R * shapes[s][0] * shapes[s][1] // 8 for s in PROBE_SHAPES) / len(PROBE_SHAPES)
    traffic = res["FETCH_SIZE"]["kernel_bytes_avg"] + res["WRITE_SIZE"]["kernel_bytes_avg"]
    lines = [
        "# HBM traffic of the dominant batch-1 kernel (gemv_kernel<4, *>, Llama-3.1-8B gate_up and down, r = 4)",
        "",
        "Commands (repository root, one MI355X; one counter per pass):",
        "  rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_fetch -- python3 bench.py --pmc-probe",
        "  rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_write -- python3 bench.py --pmc-probe",
        "  python3 bench.py --traffic-from gpurun_out/pmc_fetch gpurun_out/pmc_write",
        "",
        f"reference copy: {PROBE_COPY_BYTES} bytes read and written by one device copy dispatch",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        lines.append(f"{c}: copy counts {r['copy_kib']:.1f} KiB -> factor {r['factor']:.4f} bytes per reported byte; "
                     f"kernel {r['kernel_kib_avg']:.1f} KiB avg over {r['launches']} launches -> "
                     f"{r['kernel_bytes_avg']:.0f} bytes")
    lines += [f"algorithmic plane bytes per launch (avg of the two shapes): {alg:.0f}",
              f"traffic_bytes_per_launch: {traffic:.0f}",
              f"traffic_over_algorithmic: {traffic / alg:.4f}",
              f"kernel_source_sha256_16: {kernel_source_hash()}"]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stored_traffic():
    """Per-launch HBM bytes from the committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line)
        if kv.get("kernel_source_sha256_16", "").strip() != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.rbits_from:
        rbits_from(args.rbits_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

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
        pmc_probe(torch, nbw, synth)
        return
    if args.pmc_rbits:
        pmc_rbits_probe(torch, nbw, synth)
        return

    t = time.time()
    layer = Layer(torch, nbw, synth, "llama3.1-8b", args.copies)
    log(f"workload ready: {layer.copies} parent copies of {layer.parent_bytes / 1e6:.1f} MB "
        f"({time.time() - t:.1f} s)")
    for L in layer.lin:
        L["y1"] = torch.empty((1, L["n"]), dtype=torch.float32, device="cuda")

    # ---- headline: batch 1, r = 4, 3, 2, the step replayed as a HIP graph
    bytes_step = sum(r * L["n"] * L["k"] // 8 for r in RS_B1 for L in layer.lin)
    st1 = Stepper(torch, nbw, layer, RS_B1, "x1", "y1", args.b1_kernel, chain=True)
    ms = st1.time(args.steps, args.warmup, graph=True)
    value = bytes_step / (ms * 1e-3) / 1e9
    log(f"batch 1 (graph): {ms * 1e3:.1f} us/step, {value:.1f} GB/s")
    ms_eager = st1.time(args.steps, args.warmup, graph=False)
    log(f"batch 1 (eager): {ms_eager * 1e3:.1f} us/step, {bytes_step / (ms_eager * 1e-3) / 1e9:.1f} GB/s")
    del st1

    durs = kernel_durations(torch, nbw, layer, RS_B1, "x1", "y1", 1, args.b1_kernel, rotations=GRAPH_ROTATIONS,
                            reps=max(10, args.steps // 4))
    dom_name, dom = dominant(durs, 1)
    dom_avg_us = dom["us"] / dom["launches"]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    traffic = stored_traffic() if dom_name.startswith("nbw::gemv_kernel<4") else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic else None,
                "kernel": dom_name, "avg_launch_us": round(dom_avg_us, 2),
                "bytes_per_launch": dom["bytes"] // dom["launches"],
                "launches_per_step": dom["launches"]}
    floor = stream_floor(torch, nbw, layer, RS_B1, reps=max(10, args.steps // 4))
    per_shape = [{"linear": nm, "r": r, "us": round(d["us"], 2),
                  "GBps": round(r * d["n"] * d["k"] / 8 / (d["us"] * 1e-6) / 1e9, 1),
                  "read_floor_us": round(floor[(nm, r)], 2),
                  "frac_of_read_floor": round(floor[(nm, r)] / d["us"], 3),
                  "kernel": d["kernel"]}
                 for (nm, r), d in sorted(durs.items())]
    dom_floor = sum(floor[key] for key, d in durs.items() if d["kernel"] == dom_name)
    roofline["read_floor_us_per_launch"] = round(dom_floor / dom["launches"], 2)
    roofline["frac_of_read_floor"] = round(dom_floor / dom["us"], 3)
    log(f"dominant kernel {dom_name}: {dom_avg_us:.2f} us avg, {achieved:.1f} GB/s; "
        f"a plain read of the same bytes takes {dom_floor / dom['launches']:.2f} us")
    for p in per_shape:
        log(f"  {p['linear']:8s} r={p['r']} {p['us']:7.2f} us {p['GBps']:7.1f} GB/s  "
            f"(read floor {p['read_floor_us']:6.2f} us, {p['frac_of_read_floor']:.2f})  {p['kernel']}")

    result = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic",
              "config": {"workload": "llama3.1-8b decoder linears qkv/o/gate_up/down, batch 1, "
                                     "r=4,3,2 (12 qgemm launches per step, HIP graph replay)",
                         "batch": 1, "r": list(RS_B1), "parent_copies": layer.copies,
                         "bytes_per_step": bytes_step},
              "roofline": roofline,
              "eager": {"GBps": round(bytes_step / (ms_eager * 1e-3) / 1e9, 1),
                        "ms_per_step": round(ms_eager, 5),
                        "note": "same step, one Python call per launch, no graph"},
              "per_shape": per_shape}

    # ---- the same 12 products as 3 grouped dispatches (one per r over the four
    # linears).  Within a real decoder layer the linears depend on each other,
    # so this is reported beside the headline, not as it.
    def grouped_step(step):
        for ri, r in enumerate(RS_B1):
            c = copy_of(layer, RS_B1, step, ri)
            nbw.qgemm_grouped([(L["x1"], L["w"][c].slice_view(r), L["s"][c], r) for L in layer.lin],
                              outs=[L["y1"] for L in layer.lin])
    gpg = PeriodGraph(torch, grouped_step, layer.copies)
    gms = gpg.time(args.steps, args.warmup)
    del gpg
    result["grouped"] = {"GBps": round(bytes_step / (gms * 1e-3) / 1e9, 1), "ms_per_step": round(gms, 5),
                         "dispatches_per_step": len(RS_B1),
                         "note": "4 linears per dispatch, one dispatch per r; independent products"}
    log(f"batch 1 grouped: {gms * 1e3:.1f} us/step, {result['grouped']['GBps']} GB/s")

    # ---- all 12 products (every linear at every r) as ONE grouped dispatch, each product
    # with its own output: mixed precision in a single launch
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
    mms = mpg.time(args.steps, args.warmup)
    del mpg, ymix
    result["grouped_mixed"] = {"GBps": round(bytes_step / (mms * 1e-3) / 1e9, 1), "ms_per_step": round(mms, 5),
                               "dispatches_per_step": 1,
                               "note": "the 12 products (4 linears x r = 4, 3, 2) in one dispatch; independent products"}
    log(f"batch 1 grouped, one mixed-precision dispatch: {mms * 1e3:.1f} us/step, "
        f"{result['grouped_mixed']['GBps']} GB/s")

    if not args.no_extra:
        # ---- pack (once per checkpoint): 1 byte read + 1 byte written per weight
        L0 = layer.lin
        codes = [torch.randint(0, 256, (L["n"], L["k"]), dtype=torch.uint8, device="cuda") for L in L0]
        outs = [torch.empty(8 * L["w"][0].plane_bytes, dtype=torch.uint8, device="cuda") for L in L0]
        for c, o in zip(codes, outs):
            nbw.pack_bitplanes(c, out=o)

        def pack_all(_):
            for c, o in zip(codes, outs):
                nbw.pack_bitplanes(c, out=o)
        pms = event_time(torch, pack_all, 5)
        pack_gbs = sum(2 * L["n"] * L["k"] for L in L0) / (pms * 1e-3) / 1e9
        result["pack"] = {"GBps": round(pack_gbs, 1), "frac_hbm": round(pack_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_weight": 2}
        del codes, outs
        log(f"pack: {pack_gbs:.1f} GB/s")

        # ---- variants (same batch-1 step): asymmetric children and bf16 outputs
        wid = synth.WORKLOAD_IDS["llama3.1-8b"]
        zrng = synth.rng_for(0, wid, 0, synth.T_WEIGHTS)
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
            vms = vpg.time(max(10, args.steps // 4), 5)
            variants[name] = {"GBps": round(bytes_step / (vms * 1e-3) / 1e9, 1), "ms_per_step": round(vms, 5)}
            del vpg
            log(f"batch 1 {name}: {variants[name]['GBps']} GB/s")
        result["variants_b1"] = variants

        # ---- data-free parent-code choice (offline, like pack): weights per second on the
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

        # ---- batch 4 and 16 (same linears, same recipe)
        other = {}
        for b in (4, 16):
            for sid, L in enumerate(layer.lin):
                xb = synth.activations(b, L["k"], synth.rng_for(0, wid, sid, synth.T_X))
                L[f"x{b}"] = torch.from_numpy(xb).view(torch.bfloat16).cuda()
                L[f"y{b}"] = torch.empty((b, L["n"]), dtype=torch.float32, device="cuda")
            stb = Stepper(torch, nbw, layer, RS_B1, f"x{b}", f"y{b}", chain=True)
            msb = stb.time(max(10, args.steps // 4), 5, graph=True)
            del stb
            other[f"batch{b}"] = {"GBps": round(bytes_step / (msb * 1e-3) / 1e9, 1),
                                  "ms_per_step": round(msb, 5)}
            log(f"batch {b}: {other[f'batch{b}']['GBps']} GB/s")
        result["other_batches"] = other

        # ---- batch 256, r = 8, 4, 3, 2: TFLOP/s
        B = 256
        for sid, L in enumerate(layer.lin):
            d = synth.activations(B, L["k"], synth.rng_for(0, wid, sid, synth.T_X), outliers=True,
                                  outlier_rng=synth.rng_for(0, wid, sid, synth.T_OUTLIERS))
            L["x256"] = torch.from_numpy(d).view(torch.bfloat16).cuda()
            L["y256"] = torch.empty((B, L["n"]), dtype=torch.float32, device="cuda")
        flops_step = sum(2 * B * L["n"] * L["k"] for _ in RS_B256 for L in layer.lin)
        st256 = Stepper(torch, nbw, layer, RS_B256, "x256", "y256")
        ms256 = st256.time(max(4, args.steps // 20), 2, graph=True)
        del st256
        tflops = flops_step / (ms256 * 1e-3) / 1e12
        d256 = kernel_durations(torch, nbw, layer, RS_B256, "x256", "y256", B, "auto", reps=3)
        n256, t256 = dominant(d256, B)
        ach256 = t256["flops"] / (t256["us"] * 1e-6) / 1e12
        result["batch256"] = {"TFLOPs": round(tflops, 2), "ms_per_step": round(ms256, 5),
                              "r": list(RS_B256),
                              "roofline": {"bound": "mfma", "achieved": round(ach256, 2),
                                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                           "frac": round(ach256 / BF16_PEAK_TFLOPS, 4),
                                           "kernel": n256,
                                           "avg_launch_us": round(t256["us"] / t256["launches"], 2)},
                              "per_shape": [{"linear": nm, "r": r, "us": round(d["us"], 2),
                                             "TFLOPs": round(2 * B * d["n"] * d["k"] / (d["us"] * 1e-6)
                                                             / 1e12, 1)}
                                            for (nm, r), d in sorted(d256.items())]}
        log(f"batch 256: {tflops:.1f} TFLOP/s; {n256} {ach256:.1f} TFLOP/s")

        # ---- the rest of the large-batch sweep (batch 32, 64, 128; r = 8, 4, 3, 2; activations
        # with outlier channels), through the automatic kernel choice: time per step of the 16
        # products, TFLOP/s, plane bytes per second, and the kernel family each product used
        sweep = {}
        for b in (32, 64, 128):
            for sid, L in enumerate(layer.lin):
                d = synth.activations(b, L["k"], synth.rng_for(0, wid, sid, synth.T_X), outliers=True,
                                      outlier_rng=synth.rng_for(0, wid, sid, synth.T_OUTLIERS))
                L[f"x{b}"] = torch.from_numpy(d).view(torch.bfloat16).cuda()
                L[f"y{b}"] = torch.empty((b, L["n"]), dtype=torch.float32, device="cuda")
            stb = Stepper(torch, nbw, layer, RS_B256, f"x{b}", f"y{b}")
            msb = stb.time(max(4, args.steps // 20), 2, graph=True)
            del stb
            fl = sum(2 * b * L["n"] * L["k"] for _ in RS_B256 for L in layer.lin)
            pb = sum(r * L["n"] * L["k"] // 8 for r in RS_B256 for L in layer.lin)
            fams = sorted({nbw.kernel_name(b, L["n"], L["k"], r).split("<")[0].replace("nbw::", "")
                           for r in RS_B256 for L in layer.lin})
            sweep[f"batch{b}"] = {"ms_per_step": round(msb, 5), "TFLOPs": round(fl / (msb * 1e-3) / 1e12, 1),
                                  "plane_GBps": round(pb / (msb * 1e-3) / 1e9, 1), "kernels": fams}
            for L in layer.lin:
                del L[f"x{b}"], L[f"y{b}"]
            log(f"batch {b}: {sweep[f'batch{b}']}")
        result["batch_sweep"] = sweep

        # ---- batch 1 on the largest single linears (70B-shaped gate_up and down at r = 3, 2;
        # Qwen3-8B-shaped gate_up at r = 6, 4): the shapes whose plane bytes take >= 5 us at the
        # 8 TB/s peak, so that launch latency does not dominate the HBM fraction.  Uniform
        # random codes and U(0.001, 0.01) scales generated on the GPU (the kernels' work does
        # not depend on the values); each shape rotates over its own parent copies (> 1.2 GB).
        result["large_b1"] = large_shapes_b1(torch, nbw, gen)

        # ---- context: dense bf16 torch.matmul (hipBLASLt) on the same linears, batch 1 and 256,
        # and the sliced products' speedup over it (the pages' Figure 1 sets its kernels against a
        # dense FP16 matmul); the weights rotate over copies past the 256 MB MALL as above
        result["dense_bf16"] = dense_context(torch, layer, result, gen)
        for e in result["large_b1"]:
            log(f"large b1 {e['linear']} r={e['r']}: {e['us']} us, {e['GBps']} GB/s, "
                f"{e['frac_hbm']:.3f} of HBM peak, {e['frac_of_read_floor']:.3f} of the read floor")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth)

    print(json.dumps(result), flush=True)


def dense_context(torch, layer, result, gen):
    """Dense bf16 Y = X . W^T per Llama-3.1-8B linear at batch 1 and 256 (torch.mm on contiguous
    operands, W^T stored [k][n]), graph-replayed over weight copies; beside it the sliced products'
    times from this run and the speedup over dense."""
    ours = {}
    for e in result["per_shape"]:
        ours[(e["linear"], e["r"], 1)] = e["us"]
    for e in result.get("batch256", {}).get("per_shape", []):
        ours[(e["linear"], e["r"], 256)] = e["us"]
    out = []
    for L in layer.lin:
        n, k = L["n"], L["k"]
        copies = max(2, -(-1_200_000_000 // (2 * n * k)) + 1)
        wts = [(torch.randn((k, n), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
               for _ in range(copies)]
        for b in (1, 256):
            x = torch.randn((b, k), device="cuda", generator=gen).to(torch.bfloat16)
            y = torch.empty((b, n), dtype=torch.bfloat16, device="cuda")
            rot = GRAPH_ROTATIONS if b == 1 else 1  # as the sliced products at this batch
            g = capture(torch, lambda wl=wts, xx=x, yy=y, rot=rot: [torch.mm(xx, wt, out=yy)
                                                                    for _ in range(rot) for wt in wl])
            us = event_time(torch, lambda i: g.replay(), 3) * 1e3 / (copies * rot)
            del g
            e = {"linear": L["name"], "batch": b, "dense_us": round(us, 2),
                 "dense_TFLOPs": round(2 * b * n * k / (us * 1e-6) / 1e12, 1)}
            sp = {str(r): round(us / ours[(L["name"], r, b)], 2)
                  for (nm, r, bb) in sorted(ours) if nm == L["name"] and bb == b}
            e["speedup_of_sliced_by_r"] = sp
            out.append(e)
        del wts
        torch.cuda.empty_cache()
    return out


LARGE_SHAPES = (("70b gate_up", 57344, 8192, (3, 2)), ("70b down", 8192, 28672, (3, 2)),
                ("qwen3-8b gate_up", 24576, 4096, (6, 4)))


def large_shapes_b1(torch, nbw, gen, kernel="auto"):
    """Batch-1 product time, plane bytes per second, and the plain read of the same bytes,
    per (shape, r) of LARGE_SHAPES; every launch reads its own parent copy."""
    sink = nbw.stream_sink()
    out = []
    for name, n, k, rs in LARGE_SHAPES:
        pb = nbw.plane_bytes(n, k)
        copies = max(2, -(-1_200_000_000 // (8 * pb)) + 1)
        codes = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        ws, ss = [], []
        for _ in range(copies):
            codes.random_(0, 256, generator=gen)
            ws.append(nbw.pack_bitplanes(codes))
            ss.append((torch.rand((n, k // 128), device="cuda", generator=gen) * 0.009 + 0.001)
                      .to(torch.bfloat16))
        del codes
        x = torch.randn((1, k), device="cuda", generator=gen).to(torch.bfloat16)
        y = torch.empty((1, n), dtype=torch.float32, device="cuda")
        for r in rs:
            calls = [nbw.QgemmCall(x, ws[c].slice_view(r), ss[c], r, out=y, kernel=kernel)
                     for c in range(copies)]
            g = capture(torch, lambda cl=calls: [c() for _ in range(GRAPH_ROTATIONS) for c in cl])
            g.replay()
            us = event_time(torch, lambda i: g.replay(), 3) * 1e3 / (copies * GRAPH_ROTATIONS)
            del g
            bufs = [w.storage for w in ws]
            gf = capture(torch, lambda bl=bufs: [nbw.stream_read(b, r * pb, sink)
                                                 for _ in range(GRAPH_ROTATIONS) for b in bl])
            gf.replay()
            fus = event_time(torch, lambda i: gf.replay(), 3) * 1e3 / (copies * GRAPH_ROTATIONS)
            del gf
            gbs = r * pb / (us * 1e-6) / 1e9
            out.append({"linear": name, "n": n, "k": k, "r": r, "us": round(us, 2),
                        "GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "read_floor_us": round(fus, 2), "frac_of_read_floor": round(fus / us, 4),
                        "kernel": nbw.kernel_name(1, n, k, r, kernel)})
        del ws, ss
        torch.cuda.empty_cache()
    return out


def cpu_baseline(synth):
    """The CPU oracle, as it stands, on a bounded sample of the batch-1 step.

    Whole steps (all 12 products) are repeated until CPU_SAMPLE_SECONDS have
    passed; the rate is plane bytes of the completed steps over their time."""
    import oracle

    wl = "llama3.1-8b"
    ins = []
    for sid in range(len(synth.WORKLOADS[wl])):
        d = synth.make_linear(wl, sid, 1)
        ins.append((d, oracle.pack(d["codes"])))
    t0 = time.time()
    total = 0
    steps = 0
    while True:
        for r in RS_B1:
            for d, planes in ins:
                oracle.qgemm(d["x"], planes, d["scales"], d["n"], d["k"], r)
                total += r * d["n"] * d["k"] // 8
        steps += 1
        if time.time() - t0 >= CPU_SAMPLE_SECONDS:
            break
    dt = time.time() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    log(f"cpu oracle: {steps} steps in {dt:.1f} s, {total / dt / 1e9:.3f} GB/s on {cores} threads")
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2), "steps": steps,
            "sample": f"{steps} whole batch-1 steps (4 Llama-3.1-8B linears x r=4,3,2 each), "
                      "fp64 oracle (oracle/nbw_oracle.c, OpenMP over output rows)"}


if __name__ == "__main__":
    main()
