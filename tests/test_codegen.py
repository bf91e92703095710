"""Properties of the gfx950 code the kernels compile to (CPU only: hipcc
cross-compiles to assembly here).

* no kernel uses scratch memory (no register spills to memory, no private
  arrays left in memory), except a few dwords of the bf16 forward, and none
  inside a K loop;
* no packed-fp32 VALU instructions (the build disables them);
* no writes through the scalar data cache: no scalar stores or atomics and no
  write-back or discard of that cache (every store is a vector store).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _compile(tmp_path_factory, extra=()):
    from linear_cross_entropy_flce_amd import build as b
    flags = [f for f in b.flags(extra) if f not in ("-fPIC", "-shared")]
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    cmd = [b.hipcc(), *flags, "--cuda-device-only", "-S",
           os.path.join(b.CSRC, "flce_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


# the default build (libflce.so) and the profiling build with the workgroup
# timeline (libflce_timeline.so) must both hold every property
@pytest.fixture(scope="module", params=["default", "timeline"])
def asm(request, tmp_path_factory):
    return _compile(tmp_path_factory, ["-DFLCE_TIMELINE=1"] if request.param == "timeline" else [])


def _kernels(text):
    return re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)


def test_every_kernel_is_there(asm):
    names = " ".join(_kernels(asm))
    for k in ("fwd_sweep", "fwd_merge", "bwd_dz", "bwd_dhdw", "bwd_dh_reduce",
              "token_logit", "loss_reduce", "cast_bf16", "compact_count", "gather_block",
              "target_logit"):
        assert k in names, k


# The bf16 forward keeps a few values of its vocab-tile loop in scratch while
# a tile's K loop runs (stored before it, reloaded after it: ~10 dwords per
# tile of 32 stages); inside the K loop nothing touches scratch.
SCRATCH_ALLOWED = {"_ZN4flce16fwd_sweep_kernelIDF16bLb1EEEvNS_7FwdArgsE": 64,
                   "_ZN4flce16fwd_sweep_kernelIDF16bLb0EEEvNS_7FwdArgsE": 64}


def _bodies(text):
    """kernel symbol -> its instruction text"""
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_ZN4flce\w+):", text, re.M)]
    return {name: text[a:(starts[i + 1][0] if i + 1 < len(starts) else len(text))]
            for i, (a, name) in enumerate(starts)}


def _scratch_in_inner_loops(body):
    """scratch instructions in basic blocks nested two or more loops deep"""
    depth, hits, label = 0, [], False
    for line in body.splitlines():
        m = re.search(r"Depth=(\d+)", line)
        if re.match(r"^(\.LBB\w+:|; %bb\.\d+:)", line):
            # a block's loop depth is noted on its label line or on the
            # comment line right after it
            depth, label = (int(m.group(1)) if m else 0), True
            continue
        if label and m and re.match(r"^\s*;", line):
            depth = int(m.group(1))
        label = False
        if depth >= 2 and re.match(r"^\s*scratch_", line):
            hits.append(line.strip())
    return hits


def test_no_scratch(asm):
    meta = re.findall(r"\.name:\s+(\S+)\s*\n\s*\.private_segment_fixed_size:\s+(\d+)", asm)
    assert meta and len(meta) == len(_kernels(asm))
    for name, size in meta:
        assert int(size) <= SCRATCH_ALLOWED.get(name, 0), (name, size)
    bodies = _bodies(asm)
    for name in SCRATCH_ALLOWED:
        assert name in bodies
        assert "Depth=2" in bodies[name]
        assert not _scratch_in_inner_loops(bodies[name]), name


def test_no_packed_fp32(asm):
    assert not re.search(r"^\s*v_pk_(fma|mul|add)_f32\b", asm, re.M)


def test_no_scalar_cache_writes(asm):
    assert not re.search(r"^\s*s_(store|atomic|buffer_store|buffer_atomic|scratch_store)\w*\b",
                         asm, re.M)
    assert not re.search(r"^\s*s_dcache_(wb|discard)\w*\b", asm, re.M)
