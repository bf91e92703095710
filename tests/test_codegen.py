"""Properties of the gfx950 code the kernels compile to (CPU only: hipcc
cross-compiles to assembly here).

* no kernel uses scratch memory (no register spills to memory, no private
  arrays left in memory);
* no packed-fp32 VALU instructions (the build disables them);
* no writes through the scalar data cache: no scalar stores or atomics and no
  write-back or discard of that cache (every store is a vector store).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from linear_cross_entropy_flce_amd import build as b
    flags = [f for f in b.flags() if f not in ("-fPIC", "-shared")]
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    cmd = [b.hipcc(), *flags, "--cuda-device-only", "-S",
           os.path.join(b.CSRC, "flce_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(text):
    return re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)


def test_every_kernel_is_there(asm):
    names = " ".join(_kernels(asm))
    for k in ("fwd_sweep", "fwd_merge", "bwd_dz", "bwd_dhdw", "bwd_dh_reduce",
              "token_logit", "loss_reduce", "cast_bf16", "compact_count", "gather_block"):
        assert k in names, k


def test_no_scratch(asm):
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes and len(sizes) == len(_kernels(asm))
    assert all(int(s) == 0 for s in sizes)


def test_no_packed_fp32(asm):
    assert not re.search(r"^\s*v_pk_(fma|mul|add)_f32\b", asm, re.M)


def test_no_scalar_cache_writes(asm):
    assert not re.search(r"^\s*s_(store|atomic|buffer_store|buffer_atomic|scratch_store)\w*\b",
                         asm, re.M)
    assert not re.search(r"^\s*s_dcache_(wb|discard)\w*\b", asm, re.M)
