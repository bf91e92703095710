"""Host-side logic of bench.py (no GPU): the device-code digest and plan key
that tie the recorded HBM traffic to the code and launch shapes it was
measured with, the conversion of profiler byte counters into per-launch
bytes, and the one-GPU guard."""
import csv
import importlib.util
import json
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


@pytest.fixture(scope="module")
def libpath():
    from linear_cross_entropy_flce_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from linear_cross_entropy_flce_amd import build
        build.build()
    return _lib.LIB_PATH


def _section_span(bench, path, name):
    data = open(path, "rb").read()
    sec = bench.elf_section(path, name)
    start = data.find(sec)
    return data, start, len(sec)


def test_device_code_digest_covers_gpu_code_only(bench, libpath, tmp_path):
    """The digest is the SHA-256 of the gfx950 code object's .text: a changed
    byte of that machine code changes it; a changed byte of host code, or of
    the bundle outside the machine code (where the per-build id lives), does
    not; the same sources built to another path give the same digest."""
    import hashlib
    fatbin = bench.elf_section(libpath, ".hip_fatbin")
    code = bench.gfx950_text(fatbin)
    assert code is not None and len(code) > 1024
    assert bench.device_code_digest(libpath) == hashlib.sha256(code).hexdigest()
    data = open(libpath, "rb").read()
    c0 = data.find(code)
    assert c0 > 0
    # a byte of gfx950 machine code changed: another digest
    gpu = bytearray(data)
    gpu[c0 + len(code) // 2] ^= 0xFF
    (tmp_path / "gpu.so").write_bytes(bytes(gpu))
    assert bench.device_code_digest(str(tmp_path / "gpu.so")) != bench.device_code_digest(libpath)
    # a byte of host code changed: the same digest
    text = bench.elf_section(libpath, ".text")
    t0 = data.find(text)
    host = bytearray(data)
    host[t0 + len(text) // 2] ^= 0xFF
    (tmp_path / "host.so").write_bytes(bytes(host))
    assert bench.device_code_digest(str(tmp_path / "host.so")) == bench.device_code_digest(libpath)
    # a byte of the bundle outside the machine code changed: the same digest
    f0 = data.find(fatbin)
    other = bytearray(data)
    other[f0 + len(fatbin) - 8] ^= 0xFF
    (tmp_path / "bundle.so").write_bytes(bytes(other))
    assert bench.device_code_digest(str(tmp_path / "bundle.so")) == bench.device_code_digest(libpath)
    assert bench.elf_section(str(tmp_path / "host.so"), ".no_such_section") is None
    # the same sources built to another path
    from linear_cross_entropy_flce_amd import build
    os.makedirs(tmp_path / "elsewhere")
    other_lib = build.build(out=str(tmp_path / "elsewhere" / "libflce.so"))
    assert bench.device_code_digest(other_lib) == bench.device_code_digest(libpath)


def test_recorded_traffic_needs_same_code_and_plan(bench, libpath, tmp_path, monkeypatch):
    plan = {"fwd_splits": 4, "bwd_block": 8192}
    rec = {"workload": "wl_x (one bench step)", "device_code_sha256": bench.device_code_digest(),
           "plan": plan, "per_launch": {"bwd_dw": {"traffic_bytes": 123}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("bwd_dw", "wl_x", plan) == 123
    assert bench.measured_traffic("bwd_dz", "wl_x", plan) is None
    assert bench.measured_traffic("bwd_dw", "wl_y", plan) is None
    assert bench.measured_traffic("bwd_dw", "wl_x", dict(plan, bwd_block=4096)) is None
    rec["device_code_sha256"] = "0" * 64
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("bwd_dw", "wl_x", plan) is None


def _write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_summary_scales_by_copy_calibration(bench, libpath, tmp_path):
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
                                  str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), "wl",
                                  {"bwd_block": 8192})
    assert rec["calibration"]["fetch_counter_bytes_per_byte"] == 0.5
    assert rec["calibration"]["write_counter_bytes_per_byte"] == 1.0
    k = rec["per_launch"]["bwd_dw"]
    assert k["launches_profiled"] == 2
    # mean fetch 300 KiB counted -> 600 KiB read; mean write 96 KiB
    assert k["read_bytes"] == 600 * 1024
    assert k["write_bytes"] == 96 * 1024
    assert k["traffic_bytes"] == (600 + 96) * 1024
    assert "unrelated" not in rec["per_launch"]
    assert rec["device_code_sha256"] == bench.device_code_digest()
    assert rec["plan"] == {"bwd_block": 8192}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr


def test_kernel_table_rates(bench):
    kernels = {"bwd_dw": dict(launches=4, total_ms=8.0, flops=4 * 2e12, bytes=4e9),
               "fwd_merge": dict(launches=2, total_ms=0.01, flops=0.0, bytes=2 * 3.2e7)}
    t = bench.kernel_table(kernels, steps=2, step_ms=10.0)
    # 8 TFLOP in 8 ms -> 1,000 TFLOP/s; 64 MB in 10 us -> 6,400 GB/s = 0.8 of 8 TB/s
    assert t["bwd_dw"]["tflops"] == 1000.0 and "gbs" not in t["bwd_dw"]
    assert t["bwd_dw"]["avg_ms"] == 2.0 and t["bwd_dw"]["share"] == 0.4
    assert t["fwd_merge"]["gbs"] == 6400.0 and t["fwd_merge"]["hbm_frac"] == 0.8


def test_device_code_digest_of_a_broken_file_is_none(bench, tmp_path):
    (tmp_path / "trunc.so").write_bytes(b"\x7fELF\x02\x01" + b"\0" * 20)
    (tmp_path / "text.so").write_bytes(b"not a library")
    assert bench.device_code_digest(str(tmp_path / "trunc.so")) is None
    assert bench.device_code_digest(str(tmp_path / "text.so")) is None
    assert bench.device_code_digest(str(tmp_path / "missing.so")) is None


class _Rec:
    def __init__(self, cu, t0, t1, kernel, xcc=0):
        self.hw_id, self.xcc_id = cu << 8, xcc
        self.t_start, self.t_end, self.kernel = t0, t1, kernel


def test_summarize_timeline_splits_compute_unit_time(bench):
    """Two compute units, a dZ launch then a dH/dW launch (stamps in ticks):
    the shares are the hand-computed ones and sum to one per kernel."""
    recs = [_Rec(0, 0, 100, 2), _Rec(0, 110, 200, 2), _Rec(1, 0, 150, 2),
            _Rec(0, 300, 500, 3), _Rec(1, 300, 400, 4), _Rec(1, 405, 480, 4)]
    tl = bench.summarize_timeline(recs)
    assert tl["records"] == 6 and tl["compute_units"] == 2
    dz, hw = tl["kernels"]["bwd_dz"], tl["kernels"]["bwd_dhdw"]
    # dZ: span 200 x 2 units = 400; workgroups 340, a 10-tick gap, a 50-tick tail
    assert (dz["launches"], dz["workgroups"]) == (1, 3)
    assert (dz["busy"], dz["head"], dz["turnover"], dz["tail"]) == (0.85, 0.0, 0.025, 0.125)
    # dH/dW: span 200 x 2 = 400; workgroups 375, a 5-tick gap, a 20-tick tail
    assert (hw["busy"], hw["turnover"], hw["tail"]) == (0.9375, 0.0125, 0.05)
    assert hw["dH_wg_us"]["median"] == 2.0 and hw["dW_wg_us"]["median"] == 0.88  # 0.875, rounded
    for e in tl["kernels"].values():
        assert abs(e["busy"] + e["head"] + e["turnover"] + e["tail"] - 1.0) < 1e-9


def test_summarize_timeline_separates_units_of_different_xcds(bench):
    """The same CU number on two XCDs is two compute units."""
    recs = [_Rec(3, 0, 10, 2, xcc=0), _Rec(3, 0, 10, 2, xcc=1)]
    tl = bench.summarize_timeline(recs)
    assert tl["compute_units"] == 2 and tl["kernels"]["bwd_dz"]["busy"] == 1.0
    assert bench.summarize_timeline([]) == {"records": 0}
