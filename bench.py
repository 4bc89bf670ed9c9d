#!/usr/bin/env python3
"""Throughput of sliced r-bit qgemm on one MI355X.

A step is one pass of the hot path over the Llama-3.1-8B-shaped decoder linears
(qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096; GPTQ-like
8-bit parent codes from N(0, 0.02) weights with absmax group-128 bf16 scales;
X bf16 N(0, 1)) at batch 1: for each child width r in (4, 3, 2), slice the
parent (host-only view) and run qgemm on all four linears -- 12 launches that
read r/8 bytes per weight of bit-planes.  ``value`` is plane bytes read per
second over the timed steps (whole job, inputs resident in HBM).  Packing is
once per checkpoint and is timed separately (``pack`` field).

To measure HBM and not the 256 MB MALL, every (step, r) uses its own parent
copy from a rotation of copies totalling >1.2 GB.

Extra fields: the dominant kernel's roofline (HIP events around every launch
in a second timed pass), batch 4 and 16 on the same linears, batch 256
(TFLOP/s, r in 8, 4, 3, 2, activations with 1% outlier channels x10), and the
CPU oracle timed on this host on the same batch-1 step.
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
RS_B1 = (4, 3, 2)
RS_B256 = (8, 4, 3, 2)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip batch 4/16/256 and pack timing")
    ap.add_argument("--copies", type=int, default=0, help="parent copies in the rotation (0 = auto)")
    ap.add_argument("--b1-kernel", default="auto", help="kernel for the batch-1 step (auto, gemv, smallb)")
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
            copies = max(3, -(-int(1.2e9) // parent_bytes))
        for L in self.lin:
            for _ in range(copies - 1):
                st = L["w"][0].storage.clone()
                L["w"].append(nbw.PackedWeight(st, L["n"], L["k"], 8))
                L["s"].append(L["s"][0].clone())
        self.copies = copies
        self.parent_bytes = parent_bytes
        torch.cuda.synchronize()


def launches(layer, rs, step):
    """(linear, r, copy) for every launch of one step."""
    out = []
    for ri, r in enumerate(rs):
        c = (step * len(rs) + ri) % layer.copies
        for L in layer.lin:
            out.append((L, r, c))
    return out


def run_step(nbw, layer, rs, step, xkey, ykey, kernel="auto", events=None, torch=None):
    for (L, r, c) in launches(layer, rs, step):
        child = L["w"][c].slice_view(r)
        if events is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            nbw.qgemm(L[xkey], child, L["s"][c], r, out=L[ykey], kernel=kernel)
            e1.record()
            events.append((L, r, e0, e1))
        else:
            nbw.qgemm(L[xkey], child, L["s"][c], r, out=L[ykey], kernel=kernel)


def timed(torch, nbw, layer, rs, steps, warmup, xkey, ykey, kernel="auto"):
    for s in range(warmup):
        run_step(nbw, layer, rs, s, xkey, ykey, kernel=kernel)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        run_step(nbw, layer, rs, warmup + s, xkey, ykey, kernel=kernel)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps  # ms per step


def per_launch(torch, nbw, layer, rs, steps, xkey, ykey, batch, kernel="auto"):
    """Second timed pass with HIP events around every launch (same stream)."""
    events = []
    for s in range(steps):
        run_step(nbw, layer, rs, s, xkey, ykey, kernel=kernel, events=events, torch=torch)
    torch.cuda.synchronize()
    groups = {}
    shapes = {}
    for (L, r, e0, e1) in events:
        ms = e0.elapsed_time(e1)
        name = nbw.kernel_name(batch, L["n"], L["k"], r, kernel)
        g = groups.setdefault(name, {"ms": 0.0, "launches": 0, "bytes": 0, "flops": 0})
        g["ms"] += ms
        g["launches"] += 1
        g["bytes"] += r * L["n"] * L["k"] // 8
        g["flops"] += 2 * batch * L["n"] * L["k"]
        sh = shapes.setdefault((L["name"], r), [0.0, 0])
        sh[0] += ms
        sh[1] += 1
    return groups, shapes


def main():
    args = parse()
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

    t = time.time()
    layer = Layer(torch, nbw, synth, "llama3.1-8b", args.copies)
    log(f"workload ready: {layer.copies} parent copies of {layer.parent_bytes / 1e6:.1f} MB "
        f"({time.time() - t:.1f} s)")
    for L in layer.lin:
        L["y1"] = torch.empty((1, L["n"]), dtype=torch.float32, device="cuda")

    # ---- headline: batch 1, r = 4, 3, 2
    bytes_step = sum(r * L["n"] * L["k"] // 8 for r in RS_B1 for L in layer.lin)
    ms = timed(torch, nbw, layer, RS_B1, args.steps, args.warmup, "x1", "y1", args.b1_kernel)
    value = bytes_step / (ms * 1e-3) / 1e9
    log(f"batch 1: {ms * 1e3:.1f} us/step, {value:.1f} GB/s")

    groups, shapes = per_launch(torch, nbw, layer, RS_B1, args.steps, "x1", "y1", 1, args.b1_kernel)
    dom_name, dom = max(groups.items(), key=lambda kv: kv[1]["ms"])
    dom_avg_us = dom["ms"] / dom["launches"] * 1e3
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": dom_name, "avg_launch_us": round(dom_avg_us, 2),
                "bytes_per_launch": dom["bytes"] // dom["launches"]}
    size = {L["name"]: L["n"] * L["k"] for L in layer.lin}
    per_shape = []
    for (nm, r), (tot_ms, cnt) in sorted(shapes.items()):
        us = tot_ms / cnt * 1e3
        per_shape.append({"linear": nm, "r": r, "us": round(us, 2),
                          "GBps": round(r * size[nm] / 8 / (us * 1e-6) / 1e9, 1)})
    log(f"dominant kernel {dom_name}: {dom_avg_us:.2f} us avg, {achieved:.1f} GB/s")

    result = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic",
              "config": {"workload": "llama3.1-8b decoder linears qkv/o/gate_up/down, batch 1, "
                                     "r=4,3,2 (12 qgemm launches per step)",
                         "batch": 1, "r": list(RS_B1), "parent_copies": layer.copies,
                         "bytes_per_step": bytes_step},
              "roofline": roofline, "per_shape": per_shape}

    # ---- the same 12 products as 3 grouped dispatches (one per r over the four
    # linears).  Within a real decoder layer the linears depend on each other,
    # so this is reported beside the headline, not as it.
    def grouped_step(step):
        for ri, r in enumerate(RS_B1):
            c = (step * len(RS_B1) + ri) % layer.copies
            nbw.qgemm_grouped([(L["x1"], L["w"][c].slice_view(r), L["s"][c], r) for L in layer.lin],
                              outs=[L["y1"] for L in layer.lin])
    for s_ in range(args.warmup):
        grouped_step(s_)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for s_ in range(args.steps):
        grouped_step(args.warmup + s_)
    g1.record()
    torch.cuda.synchronize()
    gms = g0.elapsed_time(g1) / args.steps
    result["grouped"] = {"GBps": round(bytes_step / (gms * 1e-3) / 1e9, 1), "ms_per_step": round(gms, 4),
                         "dispatches_per_step": len(RS_B1),
                         "note": "4 linears per dispatch, one dispatch per r; independent products"}
    log(f"batch 1 grouped: {gms * 1e3:.1f} us/step, {result['grouped']['GBps']} GB/s")

    if not args.no_extra:
        # ---- pack (once per checkpoint): 1 byte read + 1 byte written per weight
        L0 = layer.lin
        codes = [torch.randint(0, 256, (L["n"], L["k"]), dtype=torch.uint8, device="cuda") for L in L0]
        outs = [torch.empty(8 * L["w"][0].plane_bytes, dtype=torch.uint8, device="cuda") for L in L0]
        for c, o in zip(codes, outs):
            nbw.pack_bitplanes(c, out=o)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            for c, o in zip(codes, outs):
                nbw.pack_bitplanes(c, out=o)
        e1.record()
        torch.cuda.synchronize()
        pack_bytes = reps * sum(2 * L["n"] * L["k"] for L in L0)
        pack_gbs = pack_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        result["pack"] = {"GBps": round(pack_gbs, 1), "frac_hbm": round(pack_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_weight": 2}
        del codes, outs
        log(f"pack: {pack_gbs:.1f} GB/s")

        # ---- batch 4 and 16 (same linears, same recipe)
        other = {}
        for b in (4, 16):
            wid = synth.WORKLOAD_IDS["llama3.1-8b"]
            for sid, L in enumerate(layer.lin):
                xb = synth.activations(b, L["k"], synth.rng_for(0, wid, sid, synth.T_X))
                L[f"x{b}"] = torch.from_numpy(xb).view(torch.bfloat16).cuda()
                L[f"y{b}"] = torch.empty((b, L["n"]), dtype=torch.float32, device="cuda")
            msb = timed(torch, nbw, layer, RS_B1, max(5, args.steps // 2), 2, f"x{b}", f"y{b}")
            other[f"batch{b}"] = {"GBps": round(bytes_step / (msb * 1e-3) / 1e9, 1),
                                  "ms_per_step": round(msb, 4)}
            log(f"batch {b}: {other[f'batch{b}']['GBps']} GB/s")
        result["other_batches"] = other

        # ---- batch 256, r = 8, 4, 3, 2: TFLOP/s
        B = 256
        wid = synth.WORKLOAD_IDS["llama3.1-8b"]
        for sid, L in enumerate(layer.lin):
            d = synth.activations(B, L["k"], synth.rng_for(0, wid, sid, synth.T_X), outliers=True,
                                  outlier_rng=synth.rng_for(0, wid, sid, synth.T_OUTLIERS))
            L["x256"] = torch.from_numpy(d).view(torch.bfloat16).cuda()
            L["y256"] = torch.empty((B, L["n"]), dtype=torch.float32, device="cuda")
        flops_step = sum(2 * B * L["n"] * L["k"] for _ in RS_B256 for L in layer.lin)
        ms256 = timed(torch, nbw, layer, RS_B256, 3, 1, "x256", "y256")
        tflops = flops_step / (ms256 * 1e-3) / 1e12
        g256, _ = per_launch(torch, nbw, layer, RS_B256, 2, "x256", "y256", B)
        n256, d256 = max(g256.items(), key=lambda kv: kv[1]["ms"])
        ach256 = d256["flops"] / (d256["ms"] * 1e-3) / 1e12
        result["batch256"] = {"TFLOPs": round(tflops, 2), "ms_per_step": round(ms256, 4),
                              "r": list(RS_B256),
                              "roofline": {"bound": "mfma", "achieved": round(ach256, 2),
                                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                           "frac": round(ach256 / BF16_PEAK_TFLOPS, 4),
                                           "kernel": n256,
                                           "avg_launch_us": round(d256["ms"] / d256["launches"] * 1e3, 2)}}
        log(f"batch 256: {tflops:.1f} TFLOP/s; {n256} {ach256:.1f} TFLOP/s")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth)

    print(json.dumps(result), flush=True)


def cpu_baseline(synth):
    """The CPU oracle, as it stands, on the same batch-1 step (all 12 products)."""
    import numpy as np

    import oracle

    wl = "llama3.1-8b"
    ins = []
    for sid in range(len(synth.WORKLOADS[wl])):
        d = synth.make_linear(wl, sid, 1)
        ins.append((d, oracle.pack(d["codes"])))
    t0 = time.time()
    total = 0
    for r in RS_B1:
        for d, planes in ins:
            oracle.qgemm(d["x"], planes, d["scales"], d["n"], d["k"], r)
            total += r * d["n"] * d["k"] // 8
    dt = time.time() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    log(f"cpu oracle: {dt:.1f} s, {total / dt / 1e9:.3f} GB/s on {cores} threads")
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": "the full batch-1 step: 4 Llama-3.1-8B linears x r=4,3,2, fp64 oracle "
                      "(oracle/nbw_oracle.c, OpenMP over output rows)"}


if __name__ == "__main__":
    main()
