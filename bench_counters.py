"""rocprofv3 counter probes, counter summaries and kernel-trace summaries for bench.py.

Counter probes (``bench.py --pmc-probe KIND``): one plain device copy of known
size (the reference that turns FETCH_SIZE / WRITE_SIZE into bytes), then a
fixed list of products, each launched ``PROBE_LAUNCHES`` times on parent copies
of its own with a synchronisation after every launch.  Every input is made and
every product is launched once before the reference copy, so the dispatches
after it are exactly the measured launches (and, where k is split, their
second-pass adds), in the order of the list.  Inputs are uniform random codes,
U(0.001, 0.01) scales and N(0, 1) activations drawn on the GPU: the kernels do
the same work whatever the values.

``bench.py --pmc-summary KIND DIR...`` reads the counter_collection.csv files
of one or more passes over the same probe (one rocprofv3 --pmc run per pass,
PASSES below) and writes profiles/counters_KIND.md.  ``bench.py --trace-summary
SECTION DIR`` does the same for a kernel trace of ``bench.py --only SECTION``.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")

PROBE_COPY_BYTES = 512 << 20
PROBE_LAUNCHES = 3
N_SIMD = 1024      # 256 compute units x 4 SIMDs
N_SE = 32          # shader engines (8 XCDs x 4; 8 CUs each): SQ_BUSY_CYCLES adds one count per busy SE per cycle
VALU_CYCLES = 4    # a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles

# counter passes: at most 8 SQ and 4 TCC counters per run (FETCH_SIZE takes 3 TCC, WRITE_SIZE 2)
PASSES = {
    "sq": ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
           "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"],
    "sq2": ["SQ_ACTIVE_INST_LDS", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_INSTS_VMEM_RD",
            "SQ_INSTS_SALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INST_LEVEL_VMEM", "SQ_ACTIVE_INST_ANY",
            "GRBM_GUI_ACTIVE"],
    "fetch": ["FETCH_SIZE", "GRBM_GUI_ACTIVE"],
    "write": ["WRITE_SIZE"],
}

LLAMA = "llama3.1-8b"
L70 = "llama-70b"
QWEN = "qwen3-8b"

# KIND -> (title, kernel sources whose hash stamps the summary, products)
# a product is (workload, linear, batch, r); the pack probe packs (workload, linear)
PROBES = {
    "gemv_b1": ("batch-1 streaming kernel on the Llama-3.1-8B linears (the batch-1 step: r = 4, 3, 2)",
                ("gemv.hip", "decode.h"),
                [(LLAMA, lin, 1, r) for r in (4, 3, 2) for lin in ("qkv", "o", "gate_up", "down")]),
    "gemv_large_b1": ("batch-1 streaming kernel on the largest linears (70B-shaped gate_up and down "
                      "at r = 3, 2; Qwen3-8B-shaped gate_up at r = 6, 4)",
                      ("gemv.hip", "decode.h"),
                      [(L70, "gate_up", 1, 3), (L70, "gate_up", 1, 2), (L70, "down", 1, 3),
                       (L70, "down", 1, 2), (QWEN, "gate_up", 1, 6), (QWEN, "gate_up", 1, 4)]),
    "gemv_b4": ("streaming kernel with four batch rows per launch on the Llama-3.1-8B linears (the batch-4 "
                "step: r = 4, 3, 2)",
                ("gemv.hip", "decode.h"),
                [(LLAMA, lin, 4, r) for r in (4, 3, 2) for lin in ("qkv", "o", "gate_up", "down")]),
    "smallb_b16": ("small-batch MFMA kernel on the Llama-3.1-8B linears (batch 16 at r = 4, 2; batch 8 at r = 4)",
                   ("smallb.hip", "decode.h"),
                   [(LLAMA, lin, 16, r) for r in (4, 2) for lin in ("qkv", "o", "gate_up", "down")]
                   + [(LLAMA, lin, 8, 4) for lin in ("qkv", "o", "gate_up", "down")]),
    "gemm_b256": ("large-batch GEMM on the Llama-3.1-8B linears (batch 256 at r = 8, 4)",
                  ("gemm_wide.hip", "gemm.hip", "decode.h"),
                  [(LLAMA, lin, 256, r) for r in (8, 4) for lin in ("qkv", "o", "gate_up", "down")]),
    "gemv_rbits": ("batch-1 streaming kernel on the Llama-3.1-8B gate_up linear at every child width r = 1..8 "
                   "(bytes fetched against r/8 bytes per weight)",
                   ("gemv.hip", "decode.h"),
                   [(LLAMA, "gate_up", 1, r) for r in range(1, 9)]),
    "pack": ("bit-plane packer on the Llama-3.1-8B gate_up and down codes",
             ("pack.hip",),
             [(LLAMA, "gate_up", 0, 8), (LLAMA, "down", 0, 8)]),
}


def source_hash(files) -> str:
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, "nested_bit_weight_amd", "csrc", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _shape(workload, linear):
    import synth
    for nm, n, k in synth.WORKLOADS[workload]:
        if nm == linear:
            return n, k
    raise KeyError((workload, linear))


def algorithmic(prod):
    """Bytes (planes + scales + X + Y) and flops one launch of the product needs."""
    wl, lin, b, r = prod
    n, k = _shape(wl, lin)
    if b == 0:  # pack: one code byte read, one plane byte written per weight
        return {"bytes": 2 * n * k, "planes": n * k, "flops": 0, "weights": n * k}
    planes = r * n * k // 8
    return {"bytes": planes + n * k // 64 + 2 * b * k + 4 * b * n, "planes": planes,
            "flops": 2 * b * n * k, "weights": n * k}


# ------------------------------------------------------------------ probes

def run_probe(torch, nbw, kind):
    title, _, prods = PROBES[kind]
    gen = torch.Generator(device="cuda").manual_seed(0)
    weights = {}
    for wl, lin, b, r in prods:
        if (wl, lin) in weights:
            continue
        n, k = _shape(wl, lin)
        codes = torch.randint(0, 256, (n, k), dtype=torch.uint8, device="cuda", generator=gen)
        ws = [nbw.pack_bitplanes(codes) for _ in range(PROBE_LAUNCHES + 1)]
        s = (torch.rand((n, k // 128), device="cuda", generator=gen) * 0.009 + 0.001).to(torch.bfloat16)
        weights[(wl, lin)] = (codes, ws, s)
    calls = []
    for wl, lin, b, r in prods:
        codes, ws, s = weights[(wl, lin)]
        n, k = _shape(wl, lin)
        if b == 0:
            out = torch.empty(8 * nbw.plane_bytes(n, k), dtype=torch.uint8, device="cuda")
            calls.append([lambda c=codes, o=out: nbw.pack_bitplanes(c, out=o)] * (PROBE_LAUNCHES + 1))
            continue
        x = torch.randn((b, k), device="cuda", generator=gen).to(torch.bfloat16)
        y = torch.empty((b, n), dtype=torch.float32, device="cuda")
        calls.append([nbw.QgemmCall(x, w.slice_view(r), s, r, out=y) for w in ws])
    for cl in calls:          # first launches: code objects, workspaces, nothing measured
        cl[0]()
    torch.cuda.synchronize()
    src = torch.empty(PROBE_COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)            # the reference dispatch: PROBE_COPY_BYTES read and written
    torch.cuda.synchronize()
    for cl in calls:
        for c in cl[1:]:
            c()
            torch.cuda.synchronize()
    print(f"pmc probe {kind}: copy {PROBE_COPY_BYTES} B, then {len(prods)} products x {PROBE_LAUNCHES} "
          f"launches ({title})", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ summaries

def _csv_files(folder, suffix):
    """The newest *suffix file under folder (one profiled process per folder; an
    older file left by an earlier run of the same command is ignored)."""
    files = glob.glob(os.path.join(folder, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {folder}")
    newest = max(files, key=os.path.getmtime)
    if len(files) > 1:
        print(f"{folder}: {len(files)} *{suffix} files, using the newest ({os.path.basename(newest)})",
              file=sys.stderr)
    return [newest]


def _dispatches(folder):
    """{dispatch id: {"name", "counters": {name: value}, "ns": duration or None}} of one pass."""
    out = {}
    for fn in _csv_files(folder, "counter_collection.csv"):
        with open(fn) as f:
            for row in csv.DictReader(f):
                d = out.setdefault(int(row["Dispatch_Id"]), {"name": row["Kernel_Name"], "counters": {},
                                                             "ns": None})
                c = row["Counter_Name"]
                d["counters"][c] = d["counters"].get(c, 0.0) + float(row["Counter_Value"])
                if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                    d["ns"] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    return out


def _short(name):
    return name.split("(")[0].replace("void ", "").strip()


def _split_probe(kind, disp):
    """The reference copy and, per product, its launches (main dispatch + the
    second-pass add when k is split), from one pass's dispatches."""
    ids = sorted(disp)
    copies = [i for i in ids if "copybuffer" in disp[i]["name"].lower()]
    if not copies:
        raise SystemExit("the reference copy is not among the dispatches")
    # the reference copy is the last device copy before the measured launches
    ref = copies[-1]
    after = [i for i in ids if i > ref and "nbw::" in disp[i]["name"]]
    launches = []
    for i in after:
        if "reduce" in disp[i]["name"] and launches:
            launches[-1].append(i)
        else:
            launches.append([i])
    prods = PROBES[kind][2]
    if len(launches) != len(prods) * PROBE_LAUNCHES:
        raise SystemExit(f"{kind}: {len(launches)} launches after the reference copy, "
                         f"expected {len(prods) * PROBE_LAUNCHES}")
    per = [launches[j * PROBE_LAUNCHES:(j + 1) * PROBE_LAUNCHES] for j in range(len(prods))]
    return ref, per


def pmc_summary(kind, folders):
    title, sources, prods = PROBES[kind]
    merged = {}      # product index -> {"main": {counter: [values]}, "extra": {counter: [values]}, ...}
    factors = {}
    names = {}
    ns_main = {}
    for folder in folders:
        disp = _dispatches(folder)
        ref, per = _split_probe(kind, disp)
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            if counter in disp[ref]["counters"]:
                factors[counter] = PROBE_COPY_BYTES / (disp[ref]["counters"][counter] * 1024.0)
        for j, launches in enumerate(per):
            m = merged.setdefault(j, {"main": {}, "extra": {}, "n_extra": 0})
            # second-pass adds per product (the same in every pass)
            m["n_extra"] = max(m["n_extra"], sum(len(lau) - 1 for lau in launches))
            for lau in launches:
                main = disp[lau[0]]
                names[j] = _short(main["name"])
                if main["ns"]:
                    ns_main.setdefault(j, []).append(main["ns"])
                for c, v in main["counters"].items():
                    m["main"].setdefault(c, []).append(v)
                for e in lau[1:]:
                    names.setdefault(("extra", j), _short(disp[e]["name"]))
                    for c, v in disp[e]["counters"].items():
                        m["extra"].setdefault(c, []).append(v)

    def avg(d, c):
        v = d.get(c)
        return sum(v) / len(v) if v else None

    # (the recorded commands name the folders given, one per pass in order)
    pass_dirs = list(folders) if len(folders) == len(PASSES) else [f"DIR_{p}" for p in PASSES]
    cmd_lines = []
    for (pname, ctrs), d in zip(PASSES.items(), pass_dirs):
        cmd_lines.append(f"  rocprofv3 --pmc {' '.join(ctrs)} -f csv -d {d} "
                         f"-- python3 bench.py --pmc-probe {kind}")
    cmd_lines.append(f"  python3 bench.py --pmc-summary {kind} {' '.join(folders)}")
    lines = [f"# Counters: {title}", "",
             "Commands (repository root, one MI355X; each --pmc pass in a run of its own, "
             "under `cd /tmp && export TMPDIR=/tmp` with absolute paths):", *cmd_lines, "",
             f"Each product runs {PROBE_LAUNCHES} launches, each on its own parent copy, synchronised one by one, "
             "after a plain device copy of "
             f"{PROBE_COPY_BYTES} bytes; the values are per launch (averaged).  Uniform random codes, U(0.001, 0.01) "
             "scales, N(0, 1) activations (the kernels' work does not depend on the values).",
             "",
             "Derived: cycles = SQ_BUSY_CYCLES / 32 (one count per busy shader engine per cycle; 32 engines of "
             "8 CUs; GRBM_GUI_ACTIVE also counts the counter window around the kernel, so it is listed raw "
             "only); clock = cycles / the launch's duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs "
             "x cycles); VALU busy (estimate) = 4 x (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (1024 x cycles) (a wave64 "
             "VALU instruction holds a 16-lane SIMD for 4 cycles); VALU/weight = 64 x (SQ_INSTS_VALU - "
             "SQ_INSTS_MFMA) / weights (lane operations per weight); LDS conflict share = SQ_LDS_BANK_CONFLICT / "
             "SQ_ACTIVE_INST_LDS; wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES; HBM bytes = FETCH_SIZE (and WRITE_SIZE) KiB x 1024 x the factor that maps the "
             "reference copy's count onto its true size; algorithmic bytes = planes + scales + X + Y "
             "(pack: codes read + planes written); GB/s and the clock use the duration the counter run "
             "recorded (serialised launches, so a lower bound on speed).",
             ""]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in factors:
            lines.append(f"{c} factor: {factors[c]:.4f} bytes per reported byte")
    lines += ["", "| product | kernel | cycles | clock GHz | MFMA busy | VALU busy | VALU/MFMA | LDS conflict "
              "| wait share | HBM bytes | algorithmic bytes | HBM / alg | HBM GB/s (counter run) | VALU/weight | us |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    summary = {}
    for j, prod in enumerate(prods):
        m = merged.get(j, {"main": {}, "extra": {}})
        mm = m["main"]
        cyc = avg(mm, "SQ_BUSY_CYCLES")
        cyc = cyc / N_SE if cyc else None
        ns = sum(ns_main[j]) / len(ns_main[j]) if ns_main.get(j) else None
        mfma = avg(mm, "SQ_VALU_MFMA_BUSY_CYCLES")
        valu, nmf = avg(mm, "SQ_INSTS_VALU"), avg(mm, "SQ_INSTS_MFMA")
        lds_c, lds_a = avg(mm, "SQ_LDS_BANK_CONFLICT"), avg(mm, "SQ_ACTIVE_INST_LDS")
        wait, wcyc = avg(mm, "SQ_WAIT_ANY"), avg(mm, "SQ_WAVE_CYCLES")
        fetch = avg(mm, "FETCH_SIZE")
        write = avg(mm, "WRITE_SIZE")
        hbm = None
        if fetch is not None and "FETCH_SIZE" in factors:
            hbm = fetch * 1024 * factors["FETCH_SIZE"]
            if write is not None and "WRITE_SIZE" in factors:
                hbm += write * 1024 * factors["WRITE_SIZE"]
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                ev = avg(m["extra"], c)
                if ev is not None and c in factors:
                    hbm += ev * 1024 * factors[c] * (m["n_extra"] / PROBE_LAUNCHES if m["n_extra"] else 0)
        alg = algorithmic(prod)
        row = {"kernel": names.get(j, "?"), "cycles": cyc, "ns": ns,
               "clock_ghz": cyc / ns if cyc and ns else None,
               "mfma_busy": mfma / (N_SIMD * cyc) if mfma is not None and cyc else None,
               "valu_busy": VALU_CYCLES * (valu - (nmf or 0)) / (N_SIMD * cyc) if valu is not None and cyc else None,
               "valu_per_mfma": (valu - nmf) / nmf if valu is not None and nmf else None,
               "lds_conflict": lds_c / lds_a if lds_c is not None and lds_a else None,
               "wait_share": wait / wcyc if wait is not None and wcyc else None,
               "hbm_bytes": hbm, "alg_bytes": alg["bytes"],
               "hbm_over_alg": hbm / alg["bytes"] if hbm else None,
               "hbm_gbs": hbm / ns if hbm and ns else None,
               "valu_per_weight": 64 * (valu - (nmf or 0)) / alg["weights"] if valu is not None else None,
               "raw": {c: avg(mm, c) for c in sorted(mm)},
               "extra": ({"kernel": names.get(("extra", j)), "launches_per_product_launch": m["n_extra"] / PROBE_LAUNCHES,
                          "raw": {c: avg(m["extra"], c) for c in sorted(m["extra"])}} if m["n_extra"] else None)}
        summary[prod] = row

        def f(v, fmt):
            return "-" if v is None else format(v, fmt)
        wl, lin, b, r = prod
        label = f"{wl} {lin} pack" if b == 0 else f"{wl} {lin} b={b} r={r}"
        lines.append(f"| {label} | `{row['kernel']}` | {f(cyc, '.0f')} | {f(row['clock_ghz'], '.2f')} | "
                     f"{f(row['mfma_busy'], '.3f')} | {f(row['valu_busy'], '.3f')} | {f(row['valu_per_mfma'], '.2f')} | "
                     f"{f(row['lds_conflict'], '.3f')} | {f(row['wait_share'], '.3f')} | {f(hbm, '.0f')} | "
                     f"{alg['bytes']} | {f(row['hbm_over_alg'], '.4f')} | {f(row['hbm_gbs'], '.1f')} | "
                     f"{f(row['valu_per_weight'], '.3f')} | {f(ns / 1e3 if ns else None, '.2f')} |")
    lines += ["", "Raw counters per launch (averages; the second-pass add of a split launch listed on its own line):", ""]
    for prod, row in summary.items():
        wl, lin, b, r = prod
        label = f"{wl} {lin} pack" if b == 0 else f"{wl} {lin} b={b} r={r}"
        lines.append(f"- {label} `{row['kernel']}`: " + ", ".join(f"{c}={v:.0f}" for c, v in row["raw"].items()))
        if row["extra"]:
            ex = row["extra"]
            lines.append(f"  - + `{ex['kernel']}` x{ex['launches_per_product_launch']:.0f}: "
                         + ", ".join(f"{c}={v:.0f}" for c, v in ex["raw"].items()))
    lines += ["", f"kernel_source_sha256_16: {source_hash(sources)}"]
    path = os.path.join(PROFILES, f"counters_{kind}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return summary


def stored_traffic(kind, prods):
    """HBM bytes per launch averaged over ``prods`` from profiles/counters_KIND.md, or
    None when the file is missing or the kernel sources changed since it was written."""
    path = os.path.join(PROFILES, f"counters_{kind}.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    stamp = [ln.split(": ", 1)[1].strip() for ln in text.splitlines() if ln.startswith("kernel_source_sha256_16: ")]
    if not stamp or stamp[0] != source_hash(PROBES[kind][1]):
        return None
    vals = []
    for prod in prods:
        wl, lin, b, r = prod
        label = f"| {wl} {lin} b={b} r={r} |"
        row = [ln for ln in text.splitlines() if ln.startswith(label)]
        if not row:
            return None
        cells = [c.strip() for c in row[0].strip("|").split("|")]
        try:
            vals.append(float(cells[9]))
        except (ValueError, IndexError):
            return None
    return sum(vals) / len(vals) if vals else None


# ------------------------------------------------------------------ kernel traces

def trace_summary(section, folder, command):
    """Kernel durations from a kernel trace of ``bench.py --only SECTION``.

    Dispatches are grouped by kernel template instance, and by instance and grid;
    a second-pass add (a kernel whose name holds "reduce") is attributed to the
    dispatch before it, so "launch" figures are main dispatch + its add."""
    rows = []
    for fn in _csv_files(folder, "kernel_trace.csv"):
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"empty kernel trace under {folder}")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    gcols = sorted(c for c in rows[0] if c.startswith("Grid_Size"))
    by_name, by_grid, order = {}, {}, []
    last = None
    for r in rows:
        name = _short(r["Kernel_Name"])
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if "nbw::" not in name:
            continue
        if "reduce" in name and last is not None:
            for g in last:
                g["add_ns"] += ns
                g["adds"] += 1
            continue
        key = (name, "x".join(r[c] for c in gcols))
        gn = by_name.setdefault(name, {"ns": 0, "calls": 0, "add_ns": 0, "adds": 0, "all": []})
        gg = by_grid.setdefault(key, {"ns": 0, "calls": 0, "add_ns": 0, "adds": 0, "all": []})
        if key not in order:
            order.append(key)
        for g in (gn, gg):
            g["ns"] += ns
            g["calls"] += 1
            g["all"].append(ns)
        last = (gn, gg)

    def row(label, g):
        avg = g["ns"] / g["calls"] / 1e3
        med = statistics.median(g["all"]) / 1e3
        add = g["add_ns"] / g["calls"] / 1e3
        return f"| {label} | {g['calls']} | {avg:.2f} | {med:.2f} | {g['adds']} | {add:.2f} | {avg + add:.2f} |"
    lines = [f"# Kernel trace: bench.py --only {section}", "",
             "Commands (repository root, one MI355X):", "", "```", command,
             f"python3 bench.py --trace-summary {section} {folder}", "```", "",
             "Every dispatch of the run: the qgemm kernels (warm-up, graph capture and replay, per-product timing) and "
             "the reference launches timed beside them (nbw::stream_read_kernel, nbw::mfma_rate_kernel).  A second-pass add "
             "of a split launch is attributed to the launch before it: avg us is the main dispatch, add us its add "
             "spread over all calls of the group, launch us the two together (what the bench's HIP events time per "
             "product); median us is the median main dispatch.", "",
             "| kernel | calls | avg us | median us | adds | add us | launch us |", "|---|---|---|---|---|---|---|"]
    out = {}
    for name, g in sorted(by_name.items(), key=lambda kv: -kv[1]["ns"]):
        lines.append(row(f"`{name}`", g))
        out[name] = {"calls": g["calls"], "avg_us": g["ns"] / g["calls"] / 1e3,
                     "launch_us": (g["ns"] + g["add_ns"]) / g["calls"] / 1e3}
    lines += ["", "By kernel and grid (work-items x, y, z):", "",
              "| kernel, grid | calls | avg us | median us | adds | add us | launch us |", "|---|---|---|---|---|---|---|"]
    for key in order:
        lines.append(row(f"`{key[0]}` {key[1]}", by_grid[key]))
    path = os.path.join(PROFILES, f"trace_{section}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return out
