"""bench.py on the CPU: its one-GPU contract, and the counter summaries that
write the committed traffic evidence.

Asked for more than one GPU (by flag
or by a launcher's WORLD_SIZE) it exits with status 2 and says why, before
touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


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


def _write_counters(folder, rows):
    os.makedirs(os.path.join(folder, "vm"), exist_ok=True)
    with open(os.path.join(folder, "vm", "1_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, counter, value) in enumerate(rows):
            f.write(f'{i},"{name}",{counter},{value}\n')


def test_counter_summaries_scale_by_the_reference_copy(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    import synth
    n, k = next((n, k) for nm, n, k in synth.WORKLOADS["llama3.1-8b"] if nm == "gate_up")
    copy_kib = bench.PROBE_COPY_BYTES / 2 / 1024  # a counter that reports half the bytes
    # per-width pass: every launch fetches exactly planes + scales + X
    rows = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib)]
    for r in bench.RBITS_RS:
        exact = r * n * k // 8 + n * k // 64 + 2 * k
        rows += [(f"void nbw::gemv_kernel<{r}, 2, false>(args)", "FETCH_SIZE", exact / 2 / 1024)] * 3
    _write_counters(str(tmp_path / "rb"), rows)
    monkeypatch.setattr(bench, "RBITS_FILE", str(tmp_path / "rbits.txt"))
    bench.rbits_from(str(tmp_path / "rb"))
    text = open(tmp_path / "rbits.txt").read()
    assert "factor 2.0000" in text
    table = [line for line in text.splitlines() if line.startswith("| ") and "`nbw::gemv_kernel<" in line]
    assert len(table) == len(bench.RBITS_RS)
    for line in table:
        assert line.split("|")[6].strip() == "1.0000"  # fetched / (planes + scales + X)
    # traffic pass: fetched and written bytes of the dominant kernel per launch
    fetch = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib),
             ("void nbw::gemv_kernel<4, 2, false>(args)", "FETCH_SIZE", 1000.0),
             ("void nbw::gemv_kernel<4, 2, false>(args)", "FETCH_SIZE", 3000.0)]
    write = [("__amd_rocclr_copyBuffer", "WRITE_SIZE", bench.PROBE_COPY_BYTES / 1024),
             ("void nbw::gemv_kernel<4, 2, false>(args)", "WRITE_SIZE", 64.0),
             ("void nbw::gemv_kernel<4, 2, false>(args)", "WRITE_SIZE", 64.0)]
    _write_counters(str(tmp_path / "f"), fetch)
    _write_counters(str(tmp_path / "w"), write)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))
    kv = dict(line.split(": ", 1) for line in open(tmp_path / "traffic.txt").read().splitlines() if ": " in line)
    assert float(kv["traffic_bytes_per_launch"]) == 2 * 2000.0 * 1024 + 64.0 * 1024
    assert kv["kernel_source_sha256_16"].strip() == bench.kernel_source_hash()
