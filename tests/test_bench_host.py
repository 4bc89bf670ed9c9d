"""bench.py on the CPU: its one-GPU contract, and the counter and trace
summaries that write the committed profiling evidence.

Asked for more than one GPU (by flag or by a launcher's WORLD_SIZE) it exits
with status 2 and says why, before touching a GPU.  The summaries are fed
synthetic rocprofv3 CSV files whose true values are known."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")
sys.path.insert(0, ROOT)


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_by_flag_exits_2():
    res = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert res.returncode == 2
    assert "one GPU only" in res.stderr and res.stdout == ""


def test_more_than_one_rank_by_world_size_exits_2():
    res = _run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert res.returncode == 2
    assert "WORLD_SIZE=4" in res.stderr and res.stdout == ""


def test_unknown_section_is_refused():
    res = _run(["--only", "b1,nonsense"])
    assert res.returncode != 0 and "nonsense" in res.stderr


def test_rotation_rule():
    import bench
    # >= 600 MB of other bytes between two uses: ceil(600 MB / bytes) + 1 copies
    assert bench.rule_copies(600_000_000) == 2
    assert bench.rule_copies(599_999_999) == 3
    assert bench.rule_copies(4_194_304) == 145
    for nb in (1_000_000, 54_525_952, 176_160_768):
        c = bench.rule_copies(nb)
        assert (c - 1) * nb >= bench.ROTATE_BYTES > (c - 2) * nb


def test_b1_products_table_bytes():
    import bench
    # Llama-3.1-8B down at r = 3 in 10 us: planes 3nk/8; effective adds the scales
    # (2 bytes per 128 weights), one bf16 row of X and one fp32 row of Y
    n, k = 4096, 14336
    durs = {("down", 3): {"n": n, "k": k, "us": 10.0, "kernel": "kern", "copies": 5, "floor_us": 8.0}}
    (e,) = bench.b1_products_table(durs)
    planes = 3 * n * k // 8
    assert e["GBps"] == round(planes / 10e-6 / 1e9, 1)
    assert e["GBps_effective"] == round((planes + n * k // 64 + 2 * k + 4 * n) / 10e-6 / 1e9, 1)
    assert e["frac_hbm"] == round(planes / 10e-6 / 1e9 / bench.HBM_PEAK_GBS, 4)
    assert e["frac_of_read_floor"] == 0.8 and e["read_floor_us"] == 8.0
    assert e["ge_5us_at_peak"] == (planes / (bench.HBM_PEAK_GBS * 1e3) >= 5.0)


def _write_counters(path, rows):
    """rows: (dispatch id, kernel, counter, value, start ns, end ns)"""
    os.makedirs(os.path.join(path, "host"), exist_ok=True)
    with open(os.path.join(path, "host", "7_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        for d, name, c, v, t0, t1 in rows:
            f.write(f'{d},"{name}",{c},{v},{t0},{t1}\n')


def test_counter_summary_maps_launches_and_scales_bytes(tmp_path, monkeypatch):
    import bench_counters as bc
    monkeypatch.setattr(bc, "PROFILES", str(tmp_path))
    kind = "gemm_b256"
    prods = bc.PROBES[kind][2]
    copy_kib = bc.PROBE_COPY_BYTES / 2 / 1024   # a counter that reports half the bytes
    fetch, sq = [], []
    d = 0
    # set-up dispatches before the reference copy: a clone (a smaller copy) and a warm launch
    for rows in (fetch, sq):
        rows.append((0, "__amd_rocclr_copyBuffer", "FETCH_SIZE" if rows is fetch else "GRBM_GUI_ACTIVE",
                     10.0, 0, 1000))
        rows.append((1, "void nbw::gemm_wide_kernel<8, 4>(args)", "FETCH_SIZE" if rows is fetch else "GRBM_GUI_ACTIVE",
                     99.0, 0, 1000))
    fetch.append((2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib, 0, 1000))
    sq.append((2, "__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 8.0, 0, 1000))
    d = 3
    truth = {}
    for j, (wl, lin, b, r) in enumerate(prods):
        alg = bc.algorithmic((wl, lin, b, r))["bytes"]
        split = lin in ("o", "down")
        truth[j] = (alg, split)
        for _ in range(bc.PROBE_LAUNCHES):
            name = f"void nbw::gemm_wide_kernel<{r}, 4>(args)"
            fetch.append((d, name, "FETCH_SIZE", alg / 2 / 1024, 0, 20_000))
            sq.append((d, name, "SQ_BUSY_CYCLES", 32 * 44_000.0, 0, 20_000))   # 44000 cycles in 20 us: 2.2 GHz
            sq.append((d, name, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 11_000.0, 0, 20_000))
            sq.append((d, name, "SQ_INSTS_MFMA", 1000.0, 0, 20_000))
            sq.append((d, name, "SQ_INSTS_VALU", 5000.0, 0, 20_000))
            d += 1
            if split:
                red = "void nbw::gemm_wide_reduce_kernel<4>(args)"
                fetch.append((d, red, "FETCH_SIZE", 512.0, 0, 2000))
                sq.append((d, red, "GRBM_GUI_ACTIVE", 800.0, 0, 2000))
                d += 1
    _write_counters(str(tmp_path / "fetch"), fetch)
    _write_counters(str(tmp_path / "sq"), sq)
    summ = bc.pmc_summary(kind, [str(tmp_path / "fetch"), str(tmp_path / "sq")])
    text = open(tmp_path / f"counters_{kind}.md").read()
    assert "FETCH_SIZE factor: 2.0000" in text
    assert f"kernel_source_sha256_16: {bc.source_hash(bc.PROBES[kind][1])}" in text
    for j, prod in enumerate(prods):
        row = summ[prod]
        alg, split = truth[j]
        extra = 512.0 * 1024 * 2 if split else 0.0
        assert abs(row["hbm_bytes"] - (alg + extra)) < 1e-6 * alg
        assert abs(row["mfma_busy"] - 0.25) < 1e-12
        assert abs(row["clock_ghz"] - 2.2) < 1e-12
        assert abs(row["valu_per_mfma"] - 4.0) < 1e-12
        assert abs(row["valu_busy"] - 4 * 4000 / (1024 * 44_000)) < 1e-12
        assert row["kernel"].startswith("nbw::gemm_wide_kernel<")
    # the roofline's traffic: the file read back while the sources are unchanged
    t = bc.stored_traffic(kind, [prods[0], prods[2]])
    assert abs(t - (truth[0][0] + truth[2][0]) / 2) < 1.0
    # a stale stamp gives no traffic
    path = tmp_path / f"counters_{kind}.md"
    path.write_text(path.read_text().replace("kernel_source_sha256_16: ", "kernel_source_sha256_16: x"))
    assert bc.stored_traffic(kind, [prods[0]]) is None


def test_counter_summary_refuses_a_wrong_launch_count(tmp_path, monkeypatch):
    import pytest
    import bench_counters as bc
    monkeypatch.setattr(bc, "PROFILES", str(tmp_path))
    rows = [(0, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.0, 0, 1),
            (1, "void nbw::pack_kernel(args)", "FETCH_SIZE", 1.0, 0, 1)]
    _write_counters(str(tmp_path / "p"), rows)
    with pytest.raises(SystemExit):
        bc.pmc_summary("pack", [str(tmp_path / "p")])


def test_trace_summary_attributes_the_split_add(tmp_path, monkeypatch):
    import bench_counters as bc
    monkeypatch.setattr(bc, "PROFILES", str(tmp_path))
    os.makedirs(tmp_path / "t" / "host")
    rows = []
    t = 0
    for _ in range(4):   # unsplit 100 us launches, then split 20 us launches + 4 us adds
        rows.append(("void nbw::gemm_wide_kernel<8, 4>(a)", t, t + 100_000, "57344"))
        t += 101_000
        rows.append(("void nbw::gemm_wide_kernel<8, 4>(a)", t, t + 20_000, "8192"))
        t += 21_000
        rows.append(("void nbw::gemm_wide_reduce_kernel<4>(a)", t, t + 4_000, "4096"))
        t += 5_000
        rows.append(("__amd_rocclr_fillBufferAligned", t, t + 1_000, "64"))
        t += 2_000
    with open(tmp_path / "t" / "host" / "7_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp,Grid_Size_X,Grid_Size_Y,Grid_Size_Z\n")
        for name, a, b, gx in rows:
            f.write(f'"{name}",{a},{b},{gx},2,1\n')
    out = bc.trace_summary("b256", str(tmp_path / "t"), "cmd")
    g = out["nbw::gemm_wide_kernel<8, 4>"]
    assert g["calls"] == 8
    assert abs(g["avg_us"] - 60.0) < 1e-9
    assert abs(g["launch_us"] - 62.0) < 1e-9     # (4 x 100 + 4 x (20 + 4)) / 8
    text = open(tmp_path / "trace_b256.md").read()
    # avg, median, adds, add spread over the calls, launch
    assert "| `nbw::gemm_wide_kernel<8, 4>` | 8 | 60.00 | 60.00 | 4 | 2.00 | 62.00 |" in text
    assert "| `nbw::gemm_wide_kernel<8, 4>` 8192x2x1 | 4 | 20.00 | 20.00 | 4 | 4.00 | 24.00 |" in text
