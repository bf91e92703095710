"""Host-side tests of the C-ABI library: symbols, planner, validation.

None of these launches a kernel: every call either plans (host-only integer
arithmetic) or fails validation before anything reaches the GPU.
"""
import ctypes
import json
import os
import re
import subprocess

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import linear_cross_entropy_flce_amd as flce
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "pages_memory_figures.json")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(flce._lib.LIB_PATH):
        from linear_cross_entropy_flce_amd import build
        build.build()
    return flce.load()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(flce_\w+)\s*\(", src, re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(flce.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", flce._lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert getattr(lib, name) is not None


def test_timeline_is_absent_from_the_default_library(lib):
    """libflce.so is built without the workgroup timeline: both calls say so
    and touch nothing (no device call is made)."""
    assert lib.flce_timeline_reset() == flce.FLCE_ERR_UNSUPPORTED
    buf = (flce.WgRecord * 4)()
    n = ctypes.c_int(-1)
    assert lib.flce_timeline_read(buf, 4, ctypes.byref(n)) == flce.FLCE_ERR_UNSUPPORTED
    assert n.value == 0
    assert lib.flce_timeline_read(None, 4, ctypes.byref(n)) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_timeline_read(buf, 4, None) == flce.FLCE_ERR_INVALID_ARG


def test_timeline_library_exports_every_declared_symbol():
    """libflce_timeline.so (the profiling build) has the same C-ABI."""
    path = flce.TIMELINE_LIB_PATH
    if not os.path.exists(path):
        from linear_cross_entropy_flce_amd import build
        build.build(extra=["-DFLCE_TIMELINE=1"], out=path)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name


def test_timeline_record_layout_matches_header(tmp_path):
    """The ctypes mirror of flce_wg_record_t has the C compiler's layout."""
    fields = [f for f, _ in flce.WgRecord._fields_]
    src = tmp_path / "wg.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"flce.h\"\n"
                   "int main(void) {\n  printf(\"%zu\\n\", sizeof(flce_wg_record_t));\n" +
                   "".join(f"  printf(\"%zu\\n\", offsetof(flce_wg_record_t, {f}));\n"
                           for f in fields) + "  return 0;\n}\n")
    exe = tmp_path / "wg"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(flce.WgRecord)
    assert out[1:] == [getattr(flce.WgRecord, f).offset for f in fields]


def test_plan_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of flce_plan_t has the C compiler's size and field
    offsets (include/flce.h built as plain C99)."""
    fields = [f for f, _ in flce.Plan._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"flce.h\"\n"
                   "int main(void) {\n  printf(\"%zu\\n\", sizeof(flce_plan_t));\n" +
                   "".join(f"  printf(\"%zu\\n\", offsetof(flce_plan_t, {f}));\n" for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(flce.Plan)
    assert out[1:] == [getattr(flce.Plan, f).offset for f in fields]


def test_scratch_size_constant_matches_header(tmp_path):
    """FLCE_SCRATCH_BYTES of the binding is the header's."""
    src = tmp_path / "scratch.c"
    src.write_text("#include <stdio.h>\n#include \"flce.h\"\n"
                   "int main(void) { printf(\"%llu\\n\", FLCE_SCRATCH_BYTES); return 0; }\n")
    exe = tmp_path / "scratch"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    assert int(out) == flce.FLCE_SCRATCH_BYTES


def test_scratch_call_refuses_a_plan_beyond_the_array(lib):
    """A plan whose workspace exceeds the scratch array is refused before any
    device call (the default plan at 65,536 x 2,048 x 124,160 needs 902 MB)."""
    p = flce.flce_plan(65536, 2048, 124160, flce.FLCE_BF16)
    assert p.ws_bytes > flce.FLCE_SCRATCH_BYTES
    st = lib.flce_forward_backward_scratch(ctypes.byref(p), 16, 16, 16, -100, 0, 1.0, 16, 16,
                                           None, 16, 16, 0, None, None)
    assert st == flce.FLCE_ERR_WORKSPACE
    assert "scratch" in flce.last_error()
    q = flce.flce_plan(65536, 2048, 124160, flce.FLCE_BF16, flce.FLCE_SCRATCH_BYTES - 256)
    assert q.ws_bytes <= flce.FLCE_SCRATCH_BYTES


def test_version_and_status_strings(lib):
    assert flce.version() == "0.1.0"
    for st in (0, -1, -2, -3, -4):
        assert lib.flce_status_string(st)


@pytest.mark.parametrize("args,status", [
    ((-1, 128, 1000, 1), flce.FLCE_ERR_INVALID_ARG),
    ((10, 0, 1000, 1), flce.FLCE_ERR_INVALID_ARG),
    ((10, 128, 0, 1), flce.FLCE_ERR_INVALID_ARG),
    ((10, 128, 1000, 7), flce.FLCE_ERR_INVALID_ARG),
    ((10, 12, 1000, 1), flce.FLCE_ERR_UNSUPPORTED),
    ((10, 65544, 1000, 1), flce.FLCE_ERR_UNSUPPORTED),
    ((1 << 31, 128, 1000, 1), flce.FLCE_ERR_UNSUPPORTED),
    ((10, 128, 1 << 31, 1), flce.FLCE_ERR_UNSUPPORTED),
])
def test_plan_rejects(lib, args, status):
    st, _ = flce.flce_plan_status(*args)
    assert st == status
    assert flce.last_error()


@pytest.mark.parametrize("T,d,V,dt", [
    (1 << 20, 1024, 1000, flce.FLCE_BF16),      # H of 2 GiB
    (1000, 4096, 1 << 18, flce.FLCE_F32),       # fp32 W of 4 GiB
    (384, 8192, 131200, flce.FLCE_BF16),        # bf16 W of 2.15 GB
    (4096, 65536, 50000, flce.FLCE_BF16),       # the widest hidden size
    (200_000_000, 8, 3, flce.FLCE_F32),         # 6.4 GB of fp32 H (the token order fills the cap)
])
def test_plan_accepts_operands_beyond_2GiB(lib, T, d, V, dt):
    """H and W may exceed 2^31 bytes (each kernel tile has its own base);
    a vocab slab's rows of W, which dH addresses from one base, stay below."""
    st, p = flce.flce_plan_status(T, d, V, dt)
    assert st == flce.FLCE_OK, flce.last_error()
    esz = 2 if dt == flce.FLCE_BF16 else 4
    assert p.bwd_slab * d * esz < 2 ** 31
    assert p.n_slabs * p.bwd_slab >= V and p.bwd_ws_bytes <= p.vocab_ws_cap


def test_plan_accepts_dW_beyond_2GiB(lib):
    # bf16 W of 1.02 GiB plans; its fp32 dW (2.03 GiB) is addressed per tile
    st, p = flce.flce_plan_status(320, 3584, 152064, flce.FLCE_BF16)
    assert st == flce.FLCE_OK
    assert 152064 * 3584 * 4 > 2 ** 31


def test_plan_dH_split_policy(lib):
    split = 256 * 256 * 256 * 4  # 256 partial tiles of 256 x 256 fp32
    # the pages' shape: 902 MB without the buffer, no room for it under the cap
    p = flce.flce_plan(65536, 2048, 124160, flce.FLCE_BF16)
    assert p.dh_split_bytes == 0 and (p.bwd_block, p.bwd_slab) == (8192, 46848)
    # 4,096 tokens at d = 2,048: 128 dH tiles, the buffer is planned
    p = flce.flce_plan(4096, 2048, 32000, flce.FLCE_BF16)
    assert p.dh_split_bytes == split
    assert p.bwd_ws_bytes == (p.dz_ws_bytes + p.dh_acc_bytes + 2 * p.bwd_block * 2048 * 2 +
                              4096 * 4 + 256 + 256 + split)
    # a cap too small for the buffer: planned without it
    cap = 512 * (96 * 4 + 256 * 2)
    p = flce.flce_plan(1100, 96, 3000, flce.FLCE_BF16, cap)
    assert p.dh_split_bytes == 0 and p.bwd_ws_bytes <= cap
    # planned inside the cap, before the slab: several slabs and the buffer
    p = flce.flce_plan(600, 64, 150000, flce.FLCE_BF16, 124_000_000)
    assert p.dh_split_bytes == split and p.n_slabs >= 3 and p.bwd_ws_bytes <= 124_000_000
    # fp32 tiles are 128 x 128
    p = flce.flce_plan(256, 128, 1000, flce.FLCE_F32)
    assert p.dh_split_bytes == 256 * 128 * 128 * 4


def test_plan_null_out(lib):
    assert lib.flce_plan(10, 128, 1000, 1, 0, None) == flce.FLCE_ERR_INVALID_ARG


def test_plan_cap_too_small(lib):
    st, _ = flce.flce_plan_status(65536, 2048, 124160, flce.FLCE_BF16, cap=1000)
    assert st == flce.FLCE_ERR_WORKSPACE
    assert "cap" in flce.last_error()


@pytest.mark.parametrize("cfg", wl.CONFIGS, ids=lambda c: c.name)
def test_plan_invariants_on_configs(lib, cfg):
    p = flce.flce_plan(cfg.T, cfg.d, cfg.V, cfg.dtype)
    esz = 2 if cfg.dtype == wl.DTYPE_BF16 else 4
    # vocab-axis workspace below 1 GB, and exactly [block x slab]
    assert p.bwd_ws_bytes < 10 ** 9
    assert p.dz_ws_bytes == p.bwd_block * p.bwd_slab * esz
    assert p.dh_acc_bytes == (p.bwd_block * cfg.d * 4 if p.n_slabs > 1 else 0)
    # blocks and slabs are tile multiples and cover T and V
    assert p.bwd_block % p.tile_t == 0 and p.bwd_slab % p.tile_v == 0
    assert p.n_blocks * p.bwd_block >= cfg.T > (p.n_blocks - 1) * p.bwd_block
    assert p.n_slabs * p.bwd_slab >= cfg.V > (p.n_slabs - 1) * p.bwd_slab
    # forward splits cover the vocab tiles, none empty
    n_vt = -(-cfg.V // p.tile_v)
    assert p.fwd_splits * p.fwd_tiles_per_split >= n_vt
    assert (p.fwd_splits - 1) * p.fwd_tiles_per_split < n_vt
    assert p.ws_bytes == max(p.fwd_ws_bytes, p.bwd_ws_bytes) + 256


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(T=st.integers(0, 300_000), d8=st.integers(1, 2048), V=st.integers(1, 300_000),
       bf16=st.booleans(), cap=st.one_of(st.just(0), st.integers(100_000, 2_000_000_000)))
def test_plan_invariants_hold_for_any_shape(lib, T, d8, V, bf16, cap):
    """For any shape, dtype and cap the planner either refuses with
    FLCE_ERR_WORKSPACE (the cap cannot hold the smallest block and slab) or
    returns a plan whose blocks and slabs are tile multiples covering T and V,
    whose workspace sizes follow their definitions and stay under the cap,
    and whose slab of W rows stays below 2 GiB."""
    d = 8 * d8
    dt = flce.FLCE_BF16 if bf16 else flce.FLCE_F32
    esz = 2 if bf16 else 4
    st_, p = flce.flce_plan_status(T, d, V, dt, cap=cap)
    if st_ == flce.FLCE_ERR_WORKSPACE:
        assert 0 < cap < 950_000_000
        return
    assert st_ == flce.FLCE_OK, flce.last_error()
    assert p.bwd_ws_bytes <= (cap if cap else 950_000_000)
    assert p.dz_ws_bytes == p.bwd_block * p.bwd_slab * esz
    assert p.dh_acc_bytes == (p.bwd_block * d * 4 if p.n_slabs > 1 else 0)
    assert p.bwd_block % p.tile_t == 0 and p.bwd_slab % p.tile_v == 0
    assert 0 < p.bwd_block <= 8192
    if T > 0:
        assert p.n_blocks * p.bwd_block >= T > (p.n_blocks - 1) * p.bwd_block
    else:
        assert p.n_blocks == 0
    assert p.n_slabs * p.bwd_slab >= V > (p.n_slabs - 1) * p.bwd_slab
    assert p.bwd_slab * d * esz < 2 ** 31
    n_vt = -(-V // p.tile_v)
    assert p.fwd_splits * p.fwd_tiles_per_split >= n_vt > (p.fwd_splits - 1) * p.fwd_tiles_per_split
    assert p.ws_bytes == max(p.fwd_ws_bytes, p.bwd_ws_bytes) + 256


def test_plan_blocks_of_the_pages_shape(lib):
    """65,536 tokens x 124,160 vocab: 8 blocks of 8,192 tokens x 3 vocab slabs.

    The slab width is the planner's round-count optimum: 183 vocab tiles of
    256, so the recompute grid of a full slab is 183 x 32 = 5,856 tiles
    (22.9 rounds of 256 compute units) and the dW grid 1,464 (5.7 rounds),
    the same round count as any narrower 3-slab choice but with fewer
    launches than 4 slabs."""
    p = flce.flce_plan(65536, 2048, 124160, "bf16")
    assert (p.bwd_block, p.n_blocks, p.n_slabs, p.bwd_slab) == (8192, 8, 3, 46848)
    assert p.dz_ws_bytes == 8192 * 46848 * 2
    assert p.bwd_ws_bytes < 950_000_000


def test_naive_footprint_matches_pages(lib):
    """The pages' printed figures for the materialised logits."""
    g = json.load(open(GOLDEN))
    for it in g["items"]:
        dt = "bf16" if it["bytes_per_elem"] == 2 else "f32"
        p = flce.flce_plan(it["T"], 128, it["V"], dt)
        total = p.naive_logits_bytes * it["copies"]
        assert round(total / 1e9, 2) == it["GB_decimal"], it
        if "GiB" in it:
            # the page's GiB figure is within 0.01 of the exact 30.3125
            assert abs(total / 2 ** 30 - it["GiB"]) < 0.01
    va = g["vocab_alignment"]
    assert va["V"] == va["factor"] * va["quotient"]


def test_cap_is_honoured(lib):
    for cap in (50_000_000, 200_000_000, 950_000_000):
        p = flce.flce_plan(65536, 2048, 124160, "bf16", cap)
        assert p.bwd_ws_bytes <= cap


def _fwd(lib, plan, H=16, W=16, y=16, loss=16, lse=16, ws=16, ws_bytes=1 << 40):
    return lib.flce_forward(ctypes.byref(plan) if plan is not None else None, H, W, y, -100, 1.0,
                            loss, lse, None, ws, ws_bytes, None)


def test_forward_validation(lib):
    p = flce.flce_plan(100, 64, 1000, "bf16")
    assert _fwd(lib, None) == flce.FLCE_ERR_INVALID_ARG
    bad = flce.Plan()
    assert _fwd(lib, bad) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd(lib, p, W=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd(lib, p, H=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd(lib, p, loss=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd(lib, p, H=24) == flce.FLCE_ERR_UNSUPPORTED
    assert _fwd(lib, p, ws_bytes=p.fwd_ws_bytes - 1) == flce.FLCE_ERR_WORKSPACE


def _bwd(lib, plan, H=16, W=16, y=16, lse=16, dH=16, dW=16, ws=16, ws_bytes=1 << 40):
    return lib.flce_backward(ctypes.byref(plan), H, W, y, lse, -100, 1.0, dH, dW, 0, ws, ws_bytes,
                             None)


def test_backward_validation(lib):
    p = flce.flce_plan(100, 64, 1000, "bf16")
    assert _bwd(lib, flce.Plan()) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd(lib, p, dW=None) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd(lib, p, lse=None) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd(lib, p, dW=20) == flce.FLCE_ERR_UNSUPPORTED
    assert _bwd(lib, p, ws_bytes=p.bwd_ws_bytes - 1) == flce.FLCE_ERR_WORKSPACE


def _fwd_shard(lib, plan, start, total, H=16, W=16, y=16, lse=16, zt=16, ws=16, ws_bytes=1 << 40):
    return lib.flce_forward_shard(ctypes.byref(plan), H, W, y, -100, start, total, lse, zt, ws,
                                  ws_bytes, None)


def test_forward_shard_validation(lib):
    p = flce.flce_plan(100, 64, 1000, "bf16")          # a shard of 1000 rows
    assert _fwd_shard(lib, flce.Plan(), 0, 2000) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd_shard(lib, p, -1, 2000) == flce.FLCE_ERR_INVALID_ARG       # starts before 0
    assert _fwd_shard(lib, p, 1001, 2000) == flce.FLCE_ERR_INVALID_ARG     # ends past the vocab
    assert _fwd_shard(lib, p, 0, 999) == flce.FLCE_ERR_INVALID_ARG         # vocab smaller than shard
    assert _fwd_shard(lib, p, 0, 1 << 31) == flce.FLCE_ERR_INVALID_ARG     # vocab ids beyond int32
    assert _fwd_shard(lib, p, 0, 2000, zt=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd_shard(lib, p, 0, 2000, lse=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fwd_shard(lib, p, 0, 2000, W=24) == flce.FLCE_ERR_UNSUPPORTED
    assert _fwd_shard(lib, p, 1000, 2000, ws_bytes=p.fwd_ws_bytes - 1) == flce.FLCE_ERR_WORKSPACE


def _merge(lib, T=100, P=2, lse=16, zt=16, y=16, total=2000, loss=16, out_lse=16):
    return lib.flce_merge_shards(T, P, lse, zt, y, -100, total, 1.0, loss, out_lse, None, None)


def test_merge_shards_validation(lib):
    assert _merge(lib, T=-1) == flce.FLCE_ERR_INVALID_ARG
    assert _merge(lib, P=0) == flce.FLCE_ERR_INVALID_ARG
    assert _merge(lib, P=3, total=2) == flce.FLCE_ERR_INVALID_ARG           # more shards than ids
    assert _merge(lib, total=0) == flce.FLCE_ERR_INVALID_ARG
    assert _merge(lib, zt=None) == flce.FLCE_ERR_INVALID_ARG
    assert _merge(lib, loss=None) == flce.FLCE_ERR_INVALID_ARG
    # T == 0 with no reduced loss launches nothing and succeeds without buffers
    assert _merge(lib, T=0, lse=None, zt=None, y=None, loss=None, out_lse=None) == flce.FLCE_OK


def _bwd_shard(lib, plan, start, total, H=16, W=16, y=16, lse=16, dH=16, dW=16, ws=16,
               ws_bytes=1 << 40):
    return lib.flce_backward_shard(ctypes.byref(plan), H, W, y, lse, -100, start, total, 1.0, dH,
                                   dW, 0, ws, ws_bytes, None)


def test_backward_shard_validation(lib):
    p = flce.flce_plan(100, 64, 1000, "bf16")
    assert _bwd_shard(lib, flce.Plan(), 0, 2000) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd_shard(lib, p, 1001, 2000) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd_shard(lib, p, -5, 2000) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd_shard(lib, p, 0, 2000, dW=None) == flce.FLCE_ERR_INVALID_ARG
    assert _bwd_shard(lib, p, 0, 2000, dH=20) == flce.FLCE_ERR_UNSUPPORTED
    assert _bwd_shard(lib, p, 1000, 2000, ws_bytes=p.bwd_ws_bytes - 1) == flce.FLCE_ERR_WORKSPACE


def _tok(lib, T=10, d=64, V=100, dt=flce.FLCE_BF16, H=16, W=16, tok=16, K=2, lse=None, out=16):
    return lib.flce_token_logprobs(T, d, V, dt, H, W, tok, K, lse, out, None)


def test_token_logprobs_validation(lib):
    assert _tok(lib, dt=7) == flce.FLCE_ERR_INVALID_ARG
    assert _tok(lib, T=-1) == flce.FLCE_ERR_INVALID_ARG
    assert _tok(lib, V=0) == flce.FLCE_ERR_INVALID_ARG
    assert _tok(lib, K=-1) == flce.FLCE_ERR_INVALID_ARG
    assert _tok(lib, d=60) == flce.FLCE_ERR_UNSUPPORTED
    assert _tok(lib, d=65544) == flce.FLCE_ERR_UNSUPPORTED
    assert _tok(lib, V=1 << 31) == flce.FLCE_ERR_UNSUPPORTED
    assert _tok(lib, out=None) == flce.FLCE_ERR_INVALID_ARG
    assert _tok(lib, tok=None) == flce.FLCE_ERR_INVALID_ARG
    assert _tok(lib, W=40) == flce.FLCE_ERR_UNSUPPORTED
    # nothing to score: no launch, no buffers needed
    assert _tok(lib, T=0, H=None, W=None, tok=None, out=None) == flce.FLCE_OK
    assert _tok(lib, K=0, H=None, W=None, tok=None, out=None) == flce.FLCE_OK


def _fb(lib, plan, red=0, H=16, W=16, y=16, loss=16, lse=16, dH=16, dW=16, dWb=None, ws=16,
        ws_bytes=1 << 40):
    return lib.flce_forward_backward(ctypes.byref(plan), H, W, y, -100, red, 1.0, loss, lse, None,
                                     dH, dW, 0, dWb, ws, ws_bytes, None)


def test_forward_backward_validation(lib):
    p = flce.flce_plan(100, 64, 1000, "bf16")
    assert _fb(lib, flce.Plan()) == flce.FLCE_ERR_INVALID_ARG
    assert _fb(lib, p, red=2) == flce.FLCE_ERR_INVALID_ARG
    assert _fb(lib, p, red=-1) == flce.FLCE_ERR_INVALID_ARG
    assert _fb(lib, p, dW=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fb(lib, p, loss=None) == flce.FLCE_ERR_INVALID_ARG
    assert _fb(lib, p, dWb=24) == flce.FLCE_ERR_UNSUPPORTED
    # the fused call needs the whole plan workspace (device scalars included)
    assert _fb(lib, p, ws_bytes=p.ws_bytes - 1) == flce.FLCE_ERR_WORKSPACE
