"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, kernel-name
matching in profiler CSVs, the counter summaries' scaling by the copy
calibration, and the digest that ties a committed counter summary to the
kernel source it was taken on."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name,short", [
    ("void moe::k_update_dispatch<4, 8, false, false>(moe::DispatchArgs)", "k_update_dispatch"),
    ("moe::k_combine(unsigned short const*, int const*, float const*)", "k_combine"),
    ("moe::(anonymous namespace)::k_expert_gemm_mx(moe::(anonymous namespace)::GemmArgs)",
     "k_expert_gemm_mx"),
    ("k_expert_gemm_mx", "k_expert_gemm_mx"),
    ("void moe::k_dispatch<3, 16, false>(moe::DispatchArgs)", "k_dispatch"),
])
def test_kernel_short_names(name, short):
    assert load_bench().short_name(name) == short


def write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy_calibration(tmp_path):
    """The median over the named kernel's dispatches only (k_dispatch must not match
    k_update_dispatch), times 1024, times the calibration's scale."""
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_counter_csv(fetch, "FETCH_SIZE", [
        ("void moe::k_dispatch<4, 8, false>(moe::DispatchArgs)", 100.0),
        ("void moe::k_dispatch<4, 8, false>(moe::DispatchArgs)", 300.0),
        ("void moe::k_dispatch<4, 8, false>(moe::DispatchArgs)", 200.0),
        ("void moe::k_update_dispatch<4, 8, false, false>(moe::DispatchArgs)", 9999.0),
    ])
    write_counter_csv(write, "WRITE_SIZE", [
        ("void moe::k_dispatch<4, 8, false>(moe::DispatchArgs)", 50.0),
        ("moe::k_combine(int)", 7777.0),
    ])
    out = tmp_path / "traffic.txt"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-counters",
                        str(fetch), str(write), "--kernel", "k_dispatch", "--sources",
                        "dispatch_impl.h,dispatch.hip", "--out", str(out), "--command", "x"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    d = json.loads(out.read_text())
    with open(os.path.join(ROOT, "profiles", "copy_calibration.txt")) as f:
        cal = json.load(f)
    assert d["FETCH_SIZE_KiB_per_dispatch"] == 200.0
    assert d["WRITE_SIZE_KiB_per_dispatch"] == 50.0
    assert d["dispatches"] == [3, 1]
    assert d["hbm_read_bytes_per_launch"] == round(200.0 * 1024 * cal["fetch_scale"])
    assert d["hbm_write_bytes_per_launch"] == round(50.0 * 1024 * cal["write_scale"])
    assert d["hbm_bytes_per_launch"] == (d["hbm_read_bytes_per_launch"] +
                                         d["hbm_write_bytes_per_launch"])
    bench = load_bench()
    assert d["source_digest"] == bench.source_digest("dispatch_impl.h", "dispatch.hip")


def test_a_kernel_missing_from_the_csv_is_an_error(tmp_path):
    fetch = tmp_path / "fetch.csv"
    write_counter_csv(fetch, "FETCH_SIZE", [("moe::k_combine(int)", 1.0)])
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-counters",
                        str(fetch), str(fetch), "--kernel", "k_dispatch", "--out",
                        str(tmp_path / "o.txt")],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "no FETCH_SIZE rows" in (r.stderr + r.stdout)


def test_committed_traffic_summaries_match_their_digests():
    """Each committed counter summary names the sources it was taken on; the bench
    line reports its traffic only while the digest matches them."""
    bench = load_bench()
    for name in ("combine_c3_traffic.txt", "dispatch_c3_traffic.txt",
                 "update_dispatch_c3_traffic.txt", "combine_c4_traffic.txt",
                 "dispatch_c4_traffic.txt", "expert_gemm_g3_traffic.txt"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            d = json.load(f)
        current = bench.source_digest(*d["source_files"])
        got = bench.counter_traffic(name, tuple(d["source_files"]))
        if d["source_digest"] == current:
            assert got == d["hbm_bytes_per_launch"], name
        else:
            assert got is None, name


def test_cold_sets_bounds():
    bench = load_bench()
    assert bench.cold_sets(1) == 96
    assert bench.cold_sets(bench.COLD_BYTES) == 2
    assert bench.cold_sets(37 << 20, hi=64) == 64
    n = bench.cold_sets(200 << 20)
    assert n * (200 << 20) >= bench.COLD_BYTES and (n - 1) * (200 << 20) < bench.COLD_BYTES
