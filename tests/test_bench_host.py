"""Host-side logic of bench.py (no GPU): the source digest that keeps the
recorded HBM traffic tied to the code it was measured on, the conversion of
profiler byte counters into per-launch bytes, and the one-GPU guard."""
import csv
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _digest_of(bench, tmp_path, text):
    (tmp_path / "k.hip").write_text(text)
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        return bench.code_digest(["k.hip"])
    finally:
        bench.ROOT = old


def test_digest_ignores_comments_and_layout(bench, tmp_path):
    base = _digest_of(bench, tmp_path, 'int f(int x) {\n  return x + 1;  // add one\n}\n')
    same = [
        'int f(int x) { return x + 1; }\n',
        '// header\nint f(int x) {\n\n    return x + 1;\n}\n',
        'int f(int x) { /* multi\n line */ return x + 1; }\n',
    ]
    for text in same:
        assert _digest_of(bench, tmp_path, text) == base, text


def test_digest_sees_code_and_string_changes(bench, tmp_path):
    base = _digest_of(bench, tmp_path, 'int f(int x) { return x + 1; }\n')
    assert _digest_of(bench, tmp_path, 'int f(int x) { return x + 2; }\n') != base
    # comment markers inside a string are code, not comments
    s1 = _digest_of(bench, tmp_path, 'const char* s = "a // b"; int g;\n')
    s2 = _digest_of(bench, tmp_path, 'const char* s = "a // c"; int g;\n')
    assert s1 != s2
    e1 = _digest_of(bench, tmp_path, 'const char* s = "q\\" // x"; int g;\n')
    e2 = _digest_of(bench, tmp_path, 'const char* s = "q\\" // y"; int g;\n')
    assert e1 != e2


def _write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_summary_scales_by_copy_calibration(bench, tmp_path):
    gib_kib = 1024 * 1024  # KiB in the 1 GiB calibration copy
    # the copy reads FETCH = 0.5 counted byte per byte and WRITE = 1.0
    _write_counter_csv(tmp_path / "cf.csv", "FETCH_SIZE",
                       [(i, "__amd_rocclr_copyBuffer", 0.5 * gib_kib) for i in range(3)])
    _write_counter_csv(tmp_path / "cw.csv", "WRITE_SIZE",
                       [(i, "__amd_rocclr_copyBuffer", 1.0 * gib_kib) for i in range(3)])
    # two launches of one kernel, counters split over two rows each (summed per dispatch)
    name = "void flce::bwd_dw_kernel<__bf16>(flce::DwArgs)"
    _write_counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                       [(1, name, 100.0), (1, name, 100.0), (2, name, 300.0), (2, name, 100.0),
                        (3, "unrelated_kernel", 5.0)])
    _write_counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(1, name, 64.0), (2, name, 128.0)])
    rec = bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                  str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), "wl")
    assert rec["calibration"]["fetch_counter_bytes_per_byte"] == 0.5
    assert rec["calibration"]["write_counter_bytes_per_byte"] == 1.0
    k = rec["per_launch"]["bwd_dw"]
    assert k["launches_profiled"] == 2
    # mean fetch 300 KiB counted -> 600 KiB read; mean write 96 KiB
    assert k["read_bytes"] == 600 * 1024
    assert k["write_bytes"] == 96 * 1024
    assert k["traffic_bytes"] == (600 + 96) * 1024
    assert "unrelated" not in rec["per_launch"]
    assert rec["source_sha256"] == bench.code_digest(bench.TRAFFIC_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr
