"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

flce_api.cpp -- planning, argument validation and launch sequencing -- is
compiled with g++ -fsanitize=address,undefined together with
tests/host/flce_host_check.cpp, which stands in for the kernel launchers (each
checks that every buffer its launch would touch lies inside a buffer the
caller passed) and drives every entry point over the planner cases below,
including the extremes of T, d, V and the workspace cap, T = 0, and the
validation paths (NULL and misaligned pointers, short workspaces, foreign
plans, unknown modes).  The plans it prints must equal the real library's.
"""
import os
import shutil
import subprocess

import pytest

import linear_cross_entropy_flce_amd as flce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "linear_cross_entropy_flce_amd", "csrc", "flce_api.cpp"),
       os.path.join(ROOT, "tests", "host", "flce_host_check.cpp")]

BF, F = flce.FLCE_BF16, flce.FLCE_F32
CASES = [
    # the workload shapes
    (256, 128, 1000, F, 0), (4096, 2048, 32000, BF, 0), (16384, 2048, 151936, BF, 0),
    (65536, 2048, 124160, BF, 0), (131072, 4096, 124160, BF, 0),
    # small and ragged shapes, T = 0
    (0, 64, 1000, F, 0), (0, 8, 1, BF, 0), (1, 8, 1, F, 0), (1, 8, 2, BF, 0), (5, 16, 7, F, 0),
    (300, 136, 515, BF, 0), (257, 72, 32007, F, 0), (520, 64, 2049, BF, 0),
    # caps: tiny, forcing several blocks and slabs, at and beyond 2^31
    (1100, 96, 3000, BF, 512 * (96 * 4 + 256 * 2)), (600, 64, 150000, BF, 124_000_000),
    (5000, 512, 20000, BF, 40_000_000), (3000, 256, 9000, F, 30_000_000),
    (9000, 1024, 50000, BF, (1 << 31) - 1), (9000, 1024, 50000, BF, (1 << 31) + 5),
    (9000, 1024, 50000, BF, (1 << 64) - 1), (1000, 64, 1000, BF, 1),
    # operands beyond 2 GiB, the widest hidden size, many tokens or ids
    (384, 8192, 131200, BF, 0), (131100, 8192, 1000, BF, 0), (1000, 4096, 1 << 18, F, 0),
    (4096, 65536, 50000, BF, 0), (64, 65536, 300, F, 0), (200_000_000, 8, 3, F, 0),
    (1000, 8, (1 << 31) - 1, BF, 0),
    # sized for the allocation-free variant's scratch array
    (6000, 1024, 30000, BF, flce.FLCE_SCRATCH_BYTES - 256),
    (65536, 2048, 124160, BF, flce.FLCE_SCRATCH_BYTES - 256),
    # rejected by the planner
    (-1, 128, 1000, BF, 0), (10, 0, 1000, BF, 0), (10, 128, 0, BF, 0), (10, 12, 1000, BF, 0),
    (10, 65544, 1000, BF, 0), (1 << 31, 128, 1000, BF, 0), ((1 << 31) - 1, 8, 3, F, 0),
]

PLAN_FIELDS = ("fwd_splits", "fwd_tiles_per_split", "bwd_block", "bwd_slab", "n_blocks",
               "n_slabs", "fwd_ws_bytes", "bwd_ws_bytes", "ws_bytes", "dh_split_bytes")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = tmp_path_factory.mktemp("host") / "flce_host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           *SRC, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(exe)


def test_host_code_under_sanitizers(checker):
    inp = "".join(f"{T} {d} {V} {dt} {cap}\n" for T, d, V, dt, cap in CASES)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([checker], input=inp, capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    lines = [l.split() for l in r.stdout.splitlines() if l.startswith("PLAN")]
    assert lines and f"CASES {len(CASES)} FAILURES 0" in r.stdout
    assert len(lines) == len(CASES)
    # the sanitized build plans exactly as the real library does
    for (T, d, V, dt, cap), f in zip(CASES, lines):
        st, p = flce.flce_plan_status(T, d, V, dt, cap)
        assert int(f[7]) == st, (T, d, V, dt, cap)
        if st == flce.FLCE_OK:
            got = [int(v) for v in f[9::2]]
            assert got == [getattr(p, k) for k in PLAN_FIELDS], (T, d, V, dt, cap)
