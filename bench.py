#!/usr/bin/env python3
"""Fused linear cross-entropy forward + backward on one MI355X.

One step = flce_forward (per-token loss and lse) + flce_backward (dH, dW) over
one synthetic batch of the pages' per-rank shape: T = 65,536 tokens,
d = 2,048, V = 124,160, bf16 inputs, uniform targets, no ignored tokens,
grad scale 1 (no reduction).  Inputs are resident in HBM before the timed
region starts.

Prints ONE JSON line on stdout:
  value   = counted TFLOP/s = 8*T*d*V per step / step time (forward 2TdV,
            backward 6TdV including the logit recompute)
  roofline = the kernel with the largest share of the timed region, its
            algorithmic flops per launch over its average launch time,
            measured with hipEvents on the launch stream, against the
            2.5 PFLOP/s dense bf16 MFMA peak
  cpu_baseline = the CPU oracle (numpy float64) timed on a bounded sample of
            the same workload on this host's cores

Progress goes to stderr.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd TFLOP/s (8·T·d·V) and % MFMA peak at T=64K,V=124,160"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_table(kernels: dict, steps: int, step_ms: float) -> dict:
    """Per-kernel figures from the library's hipEvent timing: the contraction
    kernels in TFLOP/s of their algorithmic flops, the memory-bound passes
    (merges, reductions, casts, gathers) in GB/s of their algorithmic bytes
    against the 8 TB/s HBM peak."""
    out = {}
    for k, v in kernels.items():
        sec = v["total_ms"] / 1e3
        e = {"launches": v["launches"], "avg_ms": round(v["total_ms"] / v["launches"], 4),
             "share": round(v["total_ms"] / steps / step_ms, 4)}
        if v["flops"]:
            e["tflops"] = round(v["flops"] / sec / 1e12, 2) if sec else 0.0
        else:
            gbs = v["bytes"] / sec / 1e9 if sec else 0.0
            e["gbs"] = round(gbs, 1)
            e["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
        out[k] = e
    return out


def cpu_baseline(inp, cfg, n_rows: int):
    """The oracle as it stands, on n_rows seeded rows of the workload: loss,
    lse, dH and the rows' dW contribution, i.e. the whole step for those rows."""
    import numpy as np

    import oracle
    import workloads as wl
    threads = blas_threads()
    if cfg in wl.CONFIGS:
        rows = wl.sample_rows(cfg, n_rows)
    else:
        rows = np.sort(np.random.default_rng(cfg.seed_base).choice(cfg.T, min(n_rows, cfg.T),
                                                                   replace=False))
    Hs = inp.H_f32()[rows]
    Wf = inp.W_f32()
    ys = inp.y[rows]
    ls, gs = cfg.scales()
    t0 = time.perf_counter()
    oracle.forward_backward(Hs, Wf, ys, wl.IGNORE_INDEX, gs, row_chunk=256)
    dt = time.perf_counter() - t0
    counted = 8.0 * n_rows * cfg.d * cfg.V
    return {"value": counted / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_rows} seeded token rows of the same workload (all {cfg.V} vocab "
                      f"columns, d={cfg.d}): numpy float64 logits, lse, loss, dH and the rows' dW; "
                      f"{dt:.2f} s; counted as 8*rows*d*V like the GPU figure",
            "seconds": dt, "host_cpus": os.cpu_count(),
            # extrapolation, not a measurement: the sample's rate over the whole step
            "extrapolated_full_step_s": round(8.0 * cfg.T * cfg.d * cfg.V / (counted / dt), 1)}


def measured_traffic(kernel: str, workload: str, plan_key: dict):
    """HBM bytes per launch of `kernel` from the committed profiler summary,
    or None when there is none for this workload, or when the library's
    device code or the workload's plan (its launch shapes) differ from those
    the counters were taken with."""
    import glob
    code = device_code_digest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")):
        try:
            rec = json.load(open(path))
        except (OSError, ValueError):
            continue
        if not rec.get("workload", "").startswith(workload):
            continue
        if code is None or rec.get("device_code_sha256") != code or rec.get("plan") != plan_key:
            return None
        k = rec.get("per_launch", {}).get(kernel)
        return None if k is None else int(k["traffic_bytes"])
    return None


def elf_section(path, name: str):
    """Bytes of the named section of a 64-bit little-endian ELF file (a path,
    or the file's bytes), or None."""
    data = path if isinstance(path, (bytes, bytearray)) else open(path, "rb").read()
    if data[:4] != b"\x7fELF" or data[4] != 2 or data[5] != 1:
        return None
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def header(i):  # (name, type, flags, addr, offset, size, ...)
        return struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)

    names = header(shstrndx)[4]
    for i in range(shnum):
        h = header(i)
        start = names + h[0]
        if data[start:data.index(b"\0", start)].decode() == name:
            return data[h[4]:h[4] + h[5]]
    return None


def gfx950_text(fatbin: bytes):
    """The .text section (the kernels' machine code) of the gfx950 code object
    inside a clang offload bundle, or None."""
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    if fatbin[:len(magic)] != magic:
        return None
    n, = struct.unpack_from("<Q", fatbin, len(magic))
    p = len(magic) + 8
    for _ in range(n):
        off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
        p += 24
        triple = fatbin[p:p + tlen].decode(errors="replace")
        p += tlen
        if triple.endswith("gfx950"):
            return elf_section(fatbin[off:off + size], ".text")
    return None


def device_code_digest(lib_path: str = None):
    """SHA-256 of the gfx950 machine code in libflce.so: the .text section of
    the code object in its .hip_fatbin bundle.  Unchanged by host-only or
    comment edits and by where the library is built (the bundle's other
    sections carry a per-build id), changed by any edit that changes a
    kernel."""
    import hashlib
    if lib_path is None:
        from linear_cross_entropy_flce_amd import _lib
        lib_path = _lib.LIB_PATH
    try:
        fatbin = elf_section(lib_path, ".hip_fatbin")
        code = gfx950_text(fatbin) if fatbin is not None else None
    except (OSError, ValueError, IndexError, struct.error):
        return None
    return None if code is None else hashlib.sha256(code).hexdigest()


def plan_key(plan) -> dict:
    """The plan fields that shape the launches (grids, K loops, workspace)."""
    return {f: int(getattr(plan, f)) for f in ("fwd_splits", "fwd_tiles_per_split", "bwd_block",
                                                 "bwd_slab", "n_blocks", "n_slabs",
                                                 "dh_split_bytes")}


def summarize_traffic(fetch_csv: str, write_csv: str, cfetch_csv: str, cwrite_csv: str,
                      workload: str, plan: dict) -> dict:
    """HBM bytes per launch of each library kernel from four rocprofv3
    counter-collection CSVs: FETCH_SIZE and WRITE_SIZE over bench steps, and
    the same two counters over --copy-calibration, whose copy kernel moves a
    known number of bytes and so gives each counter's scale."""
    import csv
    import re
    from collections import defaultdict

    def per_dispatch(path, counter):
        vals, names = defaultdict(float), {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = int(r["Dispatch_Id"])
                vals[k] += float(r["Counter_Value"])
                names[k] = r["Kernel_Name"]
        return vals, names

    def scale(path, counter):
        vals, names = per_dispatch(path, counter)
        copies = [v for k, v in vals.items() if "copyBuffer" in names[k]]
        if not copies:
            raise SystemExit(f"{path}: no copy kernel found")
        return sum(copies) / len(copies) * 1024.0  # counter bytes per copy

    def short(name):
        m = re.search(r"flce(?:::|\d+)(\w+?)_kernel", name)
        return m.group(1) if m else None

    # each copy of bench.py --copy-calibration 1024 reads and writes 1 GiB
    cal_bytes = 1024 * (1 << 20)
    f_per_byte = scale(cfetch_csv, "FETCH_SIZE") / cal_bytes
    w_per_byte = scale(cwrite_csv, "WRITE_SIZE") / cal_bytes
    fv, fn = per_dispatch(fetch_csv, "FETCH_SIZE")
    wv, wn = per_dispatch(write_csv, "WRITE_SIZE")
    agg = defaultdict(lambda: {"n": 0, "fetch": 0.0, "nw": 0, "write": 0.0})
    for k, v in fv.items():
        n = short(fn[k])
        if n:
            agg[n]["n"] += 1
            agg[n]["fetch"] += v
    for k, v in wv.items():
        n = short(wn[k])
        if n:
            agg[n]["nw"] += 1
            agg[n]["write"] += v
    per = {}
    for n, a in agg.items():
        if not a["n"] or not a["nw"]:
            continue
        fk, wk = a["fetch"] / a["n"], a["write"] / a["nw"]
        rd, wr = fk * 1024 / f_per_byte, wk * 1024 / w_per_byte
        per[n] = {"launches_profiled": a["n"], "fetch_kib_raw": round(fk, 1),
                  "write_kib_raw": round(wk, 1), "read_bytes": int(rd), "write_bytes": int(wr),
                  "traffic_bytes": int(rd + wr)}
    return {
        "about": "HBM traffic per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                 "dispatch), each divided by the value the same counter reads per byte of a plain "
                 "1 GiB device copy (bench.py --copy-calibration 1024). Valid only while "
                 "libflce.so's gfx950 machine code (.text of its code object) hashes to device_code_sha256 and the "
                 "workload's plan is the one recorded.",
        "workload": workload,
        "device_code_sha256": device_code_digest(),
        "plan": plan,
        "calibration": {"copy_bytes": cal_bytes,
                        "fetch_counter_bytes_per_byte": round(f_per_byte, 4),
                        "write_counter_bytes_per_byte": round(w_per_byte, 4)},
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- python3 bench.py --steps 1 --warmup 0 --cpu-rows 0",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- python3 bench.py --steps 1 --warmup 0 --cpu-rows 0",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/cfetch -o run -- python3 bench.py --copy-calibration 1024",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/cwrite -o run -- python3 bench.py --copy-calibration 1024",
            "python3 bench.py --traffic-summary OUT/fetch/run_counter_collection.csv "
            "OUT/write/run_counter_collection.csv OUT/cfetch/run_counter_collection.csv "
            "OUT/cwrite/run_counter_collection.csv",
        ],
        "per_launch": per,
    }


def shard_leg(flce, wl, H, W, cfg, ws, stream, steps: int):
    """The vocab-parallel path at the same per-GPU shape: W taken as rank 1 of
    a two-way split of a 2V-id vocabulary (vocab_start = V), targets uniform
    over all 2V ids, so half fall in this shard.  One step = forward_shard +
    merge of two shards' statistics (the second shard's row stands in for the
    gathered one) + backward_shard.  Timed with hipEvents on `stream`."""
    import numpy as np
    import torch
    T, d, V = cfg.T, cfg.d, cfg.V
    dev = W.device
    y2 = torch.from_numpy(wl.uniform_targets(np.random.default_rng(cfg.seed_base + 97), T, 2 * V)).to(dev)
    plan = flce.flce_plan(T, d, V, cfg.dtype)
    stats = torch.empty((2, 2, T), dtype=torch.float32, device=dev)
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    dH = torch.empty((T, d), dtype=H.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)

    def step():
        flce.flce_forward_shard(plan, H, W, y2, V, 2 * V, wl.IGNORE_INDEX, lse_shard=stats[0, 1],
                                zt_shard=stats[1, 1], ws=ws, stream=stream)
        flce.flce_merge_shards(stats[0], stats[1], y2, 2 * V, wl.IGNORE_INDEX, 1.0, loss=loss,
                               lse=lse, stream=stream)
        flce.flce_backward_shard(plan, H, W, y2, lse, V, 2 * V, wl.IGNORE_INDEX, 1.0,
                                 dH_partial=dH, dW_shard=dW, ws=ws, stream=stream)

    # Stand-in for the other rank's gathered statistics: this shard's lse with
    # no target logits (tokens whose target lies in the stand-in get a NaN loss;
    # the merge's cost does not depend on the values).
    flce.flce_forward_shard(plan, H, W, y2, V, 2 * V, wl.IGNORE_INDEX, lse_shard=stats[0, 0],
                            zt_shard=stats[1, 0], ws=ws, stream=stream)
    stats[1, 0].fill_(float("-inf"))
    step()
    torch.cuda.synchronize()
    flce.flce_timing_collect()
    flce.flce_timing_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    flce.flce_timing_enable(False)
    k = flce.flce_timing_collect()
    ms = e0.elapsed_time(e1) / steps
    merge = k.get("shard_merge", {"total_ms": 0.0, "launches": 1})
    log(f"  shard leg: {ms:.2f} ms/step, {8.0 * T * d * V / ms / 1e9:.1f} TFLOP/s")
    return {"workload": f"{cfg.name} as vocab shard 1 of 2 (vocab_start={V}, vocab_total={2 * V})",
            "steps": steps, "ms_per_step": round(ms, 3),
            "tflops": round(8.0 * T * d * V / ms / 1e9, 2),
            "merge_avg_ms": round(merge["total_ms"] / max(1, merge["launches"]), 4),
            "kernels": kernel_table(k, steps, ms)}


def fused_leg(flce, wl, plan, H, W, y, ws, stream, steps: int):
    """The same step as one flce_forward_backward call with the mean over
    non-ignored tokens (count and gradient scale on the device) and the bf16
    copy of dW."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    dev = W.device
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    red = torch.empty(1, dtype=torch.float32, device=dev)
    dH = torch.empty((T, d), dtype=H.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    dWb = torch.empty((V, d), dtype=torch.bfloat16, device=dev)

    def step():
        flce.flce_forward_backward(plan, H, W, y, wl.IGNORE_INDEX, "mean_valid", 1.0, loss=loss,
                                   lse=lse, loss_reduced=red, dH=dH, dW=dW, dW_bf16=dWb, ws=ws,
                                   stream=stream)

    step()
    torch.cuda.synchronize()
    flce.flce_timing_collect()
    flce.flce_timing_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    flce.flce_timing_enable(False)
    k = flce.flce_timing_collect()
    ms = e0.elapsed_time(e1) / steps
    log(f"  fused call (mean over valid tokens, bf16 dW copy): {ms:.2f} ms/step")
    return {"reduction": "mean_valid", "dW_bf16": True, "steps": steps, "ms_per_step": round(ms, 3),
            "tflops": round(8.0 * T * d * V / ms / 1e9, 2), "kernels": kernel_table(k, steps, ms)}


def scoring_leg(flce, H, W, y, lse, stream, reps: int = 5):
    """flce_token_logprobs on the step's inputs: K = 1 (the targets) and K = 8
    tokens per position.  HBM-bound: algorithmic bytes = H once + K gathered
    W rows per position + tokens, lse and outputs, against the 8 TB/s peak."""
    import torch
    T, d = H.shape
    esz = H.element_size()
    out = {}
    for K in (1, 8):
        tok = y.view(-1, 1) if K == 1 else torch.randint(0, W.shape[0], (T, K), device=W.device,
                                                          generator=torch.Generator(W.device).manual_seed(5))
        res = torch.empty((T, K), dtype=torch.float32, device=W.device)
        flce.flce_token_logprobs(H, W, tok, lse, out=res, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            flce.flce_token_logprobs(H, W, tok, lse, out=res, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = T * d * esz * (1 + K) + T * K * 12 + T * 4
        gbs = nbytes / (ms / 1e3) / 1e9
        out[f"K{K}"] = {"ms": round(ms, 4), "bytes": int(nbytes), "GB/s": round(gbs, 1),
                        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"  token scoring K={K}: {ms:.3f} ms, {gbs:.0f} GB/s")
    return out


def forms_leg(flce, wl, plan, H, W, y, ws, stream, reps: int):
    """The forward alone in its two forms of the target logit: taken from the
    tile's accumulator (FLCE_TARGET_IN_TILE) and a pure log-sum-exp sweep
    followed by one gathered dot product per token (FLCE_TARGET_GATHER).
    Timed with hipEvents on `stream`, the forms interleaved rep by rep."""
    import torch
    T = plan.T
    dev = W.device
    gplan = type(plan).from_buffer_copy(plan)
    gplan.target_logit = flce.FLCE_TARGET_GATHER
    outs = {}
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    plans = {"in_tile": plan, "gather": gplan}
    for p in plans.values():
        flce.flce_forward(p, H, W, y, wl.IGNORE_INDEX, 1.0, loss=loss, lse=lse, ws=ws, stream=stream)
    torch.cuda.synchronize()
    ms = {k: [] for k in plans}
    flce.flce_timing_collect()
    flce.flce_timing_enable(True)
    for _ in range(reps):
        for k, p in plans.items():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            flce.flce_forward(p, H, W, y, wl.IGNORE_INDEX, 1.0, loss=loss, lse=lse, ws=ws,
                              stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms[k].append(e0.elapsed_time(e1))
    flce.flce_timing_enable(False)
    kt = flce.flce_timing_collect()
    for k, v in ms.items():
        v.sort()
        outs[k] = {"fwd_ms_median": round(v[len(v) // 2], 4), "fwd_ms_min": round(v[0], 4)}
    if "target_logit" in kt:
        t = kt["target_logit"]
        outs["gather"]["target_logit_avg_ms"] = round(t["total_ms"] / t["launches"], 4)
    log(f"  forward forms: in-tile {outs['in_tile']['fwd_ms_median']:.3f} ms, "
        f"gather {outs['gather']['fwd_ms_median']:.3f} ms")
    outs["default"] = "in_tile" if plan.target_logit == flce.FLCE_TARGET_IN_TILE else "gather"
    return outs


def config_leg(flce, wl, cfg, steps: int, warmup: int, oracle_rows):
    """One workload configuration, measured like the headline step: forward +
    backward with inputs resident, hipEvents on the stream around each
    forward and backward, the device memory the step holds, and the oracle's
    host time (all rows when `oracle_rows` is None, else that many seeded rows
    with the full-batch time extrapolated from them)."""
    import numpy as np
    import torch
    log(f"config {cfg.index} {cfg.name}: inputs")
    torch.cuda.empty_cache()
    free_before = torch.cuda.mem_get_info()[0]
    inp = wl.config_inputs(cfg)
    dev = torch.device("cuda:0")
    bf16 = cfg.dtype == wl.DTYPE_BF16
    if bf16:
        H = torch.from_numpy(inp.H.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H = torch.from_numpy(inp.H).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    y = torch.from_numpy(inp.y).to(dev)
    T, d, V = cfg.T, cfg.d, cfg.V
    ls, gs = cfg.scales()
    plan = flce.flce_plan(T, d, V, cfg.dtype)
    torch.cuda.reset_peak_memory_stats()
    ws = flce.workspace(plan, dev)
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    red = torch.empty(1, dtype=torch.float32, device=dev)
    dH = torch.empty((T, d), dtype=H.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

    def step(e=None):
        if e: e[0].record(stream)
        flce.flce_forward(plan, H, W, y, wl.IGNORE_INDEX, ls, loss=loss, lse=lse, loss_reduced=red,
                          ws=ws, stream=stream)
        if e: e[1].record(stream)
        flce.flce_backward(plan, H, W, y, lse, wl.IGNORE_INDEX, gs, dH=dH, dW=dW, ws=ws,
                           stream=stream)
        if e: e[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    fwd = sorted(e[0].elapsed_time(e[1]) for e in ev)
    bwd = sorted(e[1].elapsed_time(e[2]) for e in ev)
    ms = sum(e[0].elapsed_time(e[2]) for e in ev) / steps
    peak_alloc = torch.cuda.max_memory_allocated()
    used = free_before - torch.cuda.mem_get_info()[0]
    t_valid = int((inp.y != wl.IGNORE_INDEX).sum())
    counted = 8.0 * T * d * V
    effective = 2.0 * T * d * V + 6.0 * t_valid * d * V
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    out = {"workload": cfg.name, "T": T, "d": d, "V": V, "dtype": cfg.dtype,
           "reduction": cfg.reduction, "valid_tokens": t_valid, "steps": steps,
           "ms_per_step": round(ms, 4), "fwd_ms_median": round(fwd[len(fwd) // 2], 4),
           "bwd_ms_median": round(bwd[len(bwd) // 2], 4),
           "counted_tflops": round(counted / ms / 1e9, 2),
           "effective_tflops": round(effective / ms / 1e9, 2),
           "mfma_peak": peak, "mfma_peak_frac": round(counted / ms / 1e9 / peak, 4),
           "peak_allocated_bytes": int(peak_alloc), "device_used_delta_bytes": int(used),
           "workspace_bytes": int(plan.ws_bytes),
           "vocab_axis_workspace_bytes": int(plan.dz_ws_bytes),
           "naive_logits_one_copy_bytes": int(plan.naive_logits_bytes),
           "plan": {"fwd_splits": plan.fwd_splits, "bwd_block": plan.bwd_block,
                    "bwd_slab": plan.bwd_slab, "n_blocks": plan.n_blocks, "n_slabs": plan.n_slabs}}
    log(f"  {ms:.3f} ms/step (fwd {out['fwd_ms_median']:.3f}, bwd {out['bwd_ms_median']:.3f}), "
        f"{out['counted_tflops']:.1f} counted / {out['effective_tflops']:.1f} effective TFLOP/s, "
        f"peak allocated {peak_alloc / 1e9:.2f} GB, vocab-axis workspace "
        f"{plan.dz_ws_bytes / 1e9:.3f} GB")
    del H, W, y, ws, loss, lse, red, dH, dW
    torch.cuda.empty_cache()
    if oracle_rows != 0:
        out["oracle"] = oracle_time(wl, cfg, inp, oracle_rows)
    return out


def oracle_time(wl, cfg, inp, rows):
    """The oracle (numpy float64) on this host: the whole batch when `rows` is
    None, else `rows` seeded token rows (their loss, lse, dH and dW terms, i.e.
    the whole step for those rows) with the full-batch time extrapolated."""
    import oracle
    threads = blas_threads()
    ls, gs = cfg.scales()
    Wf = inp.W_f32()
    if rows is None:
        t0 = time.perf_counter()
        oracle.forward_backward(inp.H_f32(), Wf, inp.y, wl.IGNORE_INDEX, gs, row_chunk=256)
        dt = time.perf_counter() - t0
        log(f"  oracle: full batch in {dt:.1f} s on {threads} threads")
        return {"kind": "oracle", "seconds": round(dt, 2), "rows": cfg.T, "full": True,
                "cores": threads}
    r = wl.sample_rows(cfg, rows)
    Hs = inp.H_f32()[r]
    t0 = time.perf_counter()
    oracle.forward_backward(Hs, Wf, inp.y[r], wl.IGNORE_INDEX, gs, row_chunk=256)
    dt = time.perf_counter() - t0
    ext = dt * cfg.T / len(r)
    log(f"  oracle: {len(r)} rows in {dt:.1f} s on {threads} threads "
        f"(whole batch extrapolated: {ext:.0f} s)")
    return {"kind": "oracle", "seconds": round(dt, 2), "rows": int(len(r)), "full": False,
            "cores": threads, "extrapolated_full_batch_s": round(ext, 1),
            "note": "the sampled rows' step (loss, lse, dH, dW terms) timed; the whole-batch "
                    "figure is that rate over T rows, an extrapolation"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the core count
        return os.cpu_count() or 1


def library_gemm_leg(reps: int = 10):
    """The three GEMM shapes of one token block and vocab slab at the pages'
    shape, as plain library products (torch.matmul, which runs hipBLASLt), on
    data of the workload's distributions: the logits (8,192 x 2,048 times
    2,048 x 46,848), dH (8,192 x 46,848 times 46,848 x 2,048) and dW
    (46,848 x 8,192 times 8,192 x 2,048).  Every operand is a contiguous
    row-major bf16 matrix; hipEvents around `reps` products each."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(dev).manual_seed(11)
    B, d, Vs = 8192, 2048, 46848
    Hb = torch.randn((B, d), device=dev, generator=g).to(torch.bfloat16)
    Wt = (0.02 * torch.randn((d, Vs), device=dev, generator=g)).to(torch.bfloat16)
    Ws = Wt.t().contiguous()
    # a dZ block with the magnitudes of softmax - onehot at this shape
    dZ = (torch.rand((B, Vs), device=dev, generator=g) * (2.0 / Vs)).to(torch.bfloat16)
    dZt = dZ.t().contiguous()
    shapes = {"logits": (Hb, Wt), "dH": (dZ, Ws), "dW": (dZt, Hb)}
    out = {}
    for name, (a, b) in shapes.items():
        c = torch.matmul(a, b)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = 2.0 * a.shape[0] * a.shape[1] * b.shape[1]
        out[name] = {"M": a.shape[0], "K": a.shape[1], "N": b.shape[1], "ms": round(ms, 4),
                     "tflops": round(fl / ms / 1e9, 1)}
        log(f"  library GEMM {name}: {a.shape[0]} x {a.shape[1]} x {b.shape[1]}: {ms:.3f} ms, "
            f"{fl / ms / 1e9:.1f} TFLOP/s")
        del c
    return out


TIMELINE_LAUNCH = {1: "fwd_sweep", 2: "bwd_dz", 3: "bwd_dhdw", 4: "bwd_dhdw"}


def summarize_timeline(records) -> dict:
    """Splits each launch's compute-unit time into the workgroups' own time
    (busy), the time before a unit's first workgroup (head), between its
    consecutive workgroups (turnover) and after its last one until the launch's
    last workgroup ends (tail).  records: flce_wg_record_t-like objects (hw_id,
    xcc_id, t_start, t_end, kernel) from libflce_timeline.so.  A launch is a
    maximal run of records of one kernel in start order (the step's launches
    alternate kernels); stamps tick at 100 MHz."""
    import numpy as np
    if not records:
        return {"records": 0}
    hw = np.array([r.hw_id for r in records], np.int64)
    xcc = np.array([r.xcc_id for r in records], np.int64) & 0xF
    cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 50 + ((hw >> 8) & 15)
    t0 = np.array([r.t_start for r in records], np.int64)
    t1 = np.array([r.t_end for r in records], np.int64)
    kern = np.array([r.kernel for r in records], np.int64)
    name = np.array([TIMELINE_LAUNCH.get(int(k), "other") for k in kern])
    order = np.argsort(t0, kind="stable")
    cu, t0, t1, kern, name = cu[order], t0[order], t1[order], kern[order], name[order]
    n_cu = len(np.unique(cu))
    cuts = np.flatnonzero(name[1:] != name[:-1]) + 1
    out = {}
    for seg in np.split(np.arange(len(t0)), cuts):
        k = str(name[seg[0]])
        a, b = int(t0[seg].min()), int(t1[seg].max())
        acc = out.setdefault(k, dict(launches=0, workgroups=0, cu_time=0, busy=0, head=0,
                                     turnover=0, tail=0, durations={}))
        acc["launches"] += 1
        acc["workgroups"] += len(seg)
        acc["cu_time"] += (b - a) * n_cu
        for c in np.unique(cu[seg]):
            m = seg[cu[seg] == c]
            m = m[np.argsort(t0[m], kind="stable")]
            acc["busy"] += int((t1[m] - t0[m]).sum())
            acc["head"] += int(t0[m[0]] - a)
            acc["tail"] += int(b - t1[m[-1]])
            acc["turnover"] += int(np.clip(t0[m[1:]] - t1[m[:-1]], 0, None).sum())
        for kk in np.unique(kern[seg]):
            sel = seg[kern[seg] == kk]
            acc["durations"].setdefault(int(kk), []).extend((t1[sel] - t0[sel]).tolist())
    res = {"records": len(records), "compute_units": n_cu, "tick_ns": 10,
           "shares": "of the launches' compute-unit time (span x compute units)", "kernels": {}}
    for k, acc in out.items():
        ct = max(acc["cu_time"], 1)
        e = {"launches": acc["launches"], "workgroups": acc["workgroups"],
             "busy": round(acc["busy"] / ct, 4), "head": round(acc["head"] / ct, 4),
             "turnover": round(acc["turnover"] / ct, 4), "tail": round(acc["tail"] / ct, 4)}
        for kk, dur in sorted(acc["durations"].items()):
            d = np.array(dur, np.float64) / 100.0  # microseconds
            tag = {3: "dH_", 4: "dW_"}.get(kk, "")
            e[tag + "wg_us"] = {"median": round(float(np.median(d)), 2),
                                "p5": round(float(np.percentile(d, 5)), 2),
                                "p95": round(float(np.percentile(d, 95)), 2)}
        res["kernels"][k] = e
    return res


def copy_calibration(mib: int):
    """A plain copy of mib MiB (read mib, write mib), three times: the byte
    counters of a profiler run over it give the scale of FETCH_SIZE and
    WRITE_SIZE against known traffic."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB x 3")
    print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload index (default 3)")
    ap.add_argument("--shape", type=int, nargs=3, metavar=("T", "d", "V"),
                    help="a synthetic workload of this shape instead of --config: H ~ N(0,1), "
                         "W ~ N(0,0.02^2), uniform targets, none ignored, grad scale 1")
    ap.add_argument("--dtype", choices=("bf16", "f32"), default="bf16",
                    help="element type of the --shape workload")
    ap.add_argument("--shard-steps", type=int, default=3,
                    help="steps of each extra leg (vocab shard: W as rank 1 of 2 of a 2V-id "
                         "vocabulary; fused call; token scoring); 0 skips them")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="rows of the CPU-oracle sample (0 skips it)")
    ap.add_argument("--configs", default="0,1,2,4",
                    help="other workload configurations timed after the headline one (comma "
                         "list of indices, or 'none')")
    ap.add_argument("--data", choices=("random", "zeros", "const"), default="random",
                    help="headline inputs: the workload's seeded draws (default), or H and W "
                         "all zero, or constant (1 and 1/64): the same launches on data that "
                         "toggles no multiplier bits, to measure how much of the step time "
                         "is data-dependent power")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the block/slab GEMM shapes as plain torch.matmul (hipBLASLt)")
    ap.add_argument("--timeline", action="store_true",
                    help="only run the warm-up and one step in libflce_timeline.so (the same "
                         "kernels with per-workgroup stamps) and print how each kernel's "
                         "compute-unit time splits into workgroups, turnover gaps and tails")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this many MiB (a known-size "
                         "reference for the HBM byte counters) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="only turn four rocprofv3 counter CSVs (FETCH_SIZE and WRITE_SIZE over "
                         "bench steps, then over --copy-calibration 1024) into the per-launch "
                         "traffic JSON that bench.py reads from profiles/, print it and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.traffic_summary:
        import linear_cross_entropy_flce_amd as flce
        import workloads as wl
        cfg = wl.CONFIGS[args.config]
        print(json.dumps(summarize_traffic(*args.traffic_summary,
                                           workload=cfg.name + " (one bench step)",
                                           plan=plan_key(flce.flce_plan(cfg.T, cfg.d, cfg.V,
                                                                        cfg.dtype))),
                         indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X only: the fused linear cross-entropy path here is the "
              "single-GPU kernel set (no collectives).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_cross_entropy_flce_amd as flce
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    if args.timeline:
        flce.load(flce.TIMELINE_LIB_PATH)
    else:
        flce.load()
    torch.cuda.init()
    free_before = torch.cuda.mem_get_info()[0]  # hipMemGetInfo before any of the step's buffers
    if args.shape:
        T_, d_, V_ = args.shape
        cfg = wl.Config(f"synthetic_{args.dtype}_T{T_}_d{d_}_V{V_}", T_, d_, V_, args.dtype, 0.02,
                        "uniform")
    else:
        cfg = wl.CONFIGS[args.config]
    log(f"workload {cfg.name}: generating inputs")
    t0 = time.perf_counter()
    inp = (wl.config_inputs(cfg) if cfg in wl.CONFIGS else
           wl.make_inputs(cfg.T, cfg.d, cfg.V, cfg.dtype, cfg.seed_base, sigma_w=cfg.sigma_w))
    log(f"  inputs ready in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    bf16 = cfg.dtype == wl.DTYPE_BF16
    if bf16:
        H = torch.from_numpy(inp.H.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H = torch.from_numpy(inp.H).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    y = torch.from_numpy(inp.y).to(dev)
    if args.data == "zeros":
        H.zero_()
        W.zero_()
    elif args.data == "const":
        H.fill_(1.0)
        W.fill_(1.0 / 64)
    T, d, V = cfg.T, cfg.d, cfg.V
    ls, gs = cfg.scales()
    plan = flce.flce_plan(T, d, V, cfg.dtype)
    ws = flce.workspace(plan, dev)
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    dH = torch.empty((T, d), dtype=H.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        flce.flce_forward(plan, H, W, y, wl.IGNORE_INDEX, ls, loss=loss, lse=lse, ws=ws,
                          stream=stream)
        flce.flce_backward(plan, H, W, y, lse, wl.IGNORE_INDEX, gs, dH=dH, dW=dW, ws=ws,
                           stream=stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.timeline:
        flce.flce_timeline_reset()
        log("one step with workgroup stamps")
        step()
        torch.cuda.synchronize()
        tl = summarize_timeline(flce.flce_timeline_read())
        tl["workload"] = cfg.name
        for k, e in tl.get("kernels", {}).items():
            log(f"  {k:10s} launches {e['launches']:4d} workgroups {e['workgroups']:7d}: busy "
                f"{100 * e['busy']:5.1f}%  head {100 * e['head']:4.1f}%  turnover "
                f"{100 * e['turnover']:4.1f}%  tail {100 * e['tail']:4.1f}%")
        print(json.dumps(tl))
        return
    torch.cuda.reset_peak_memory_stats()
    flce.flce_timing_collect()  # discard anything recorded so far
    flce.flce_timing_enable(True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    flce.flce_timing_enable(False)
    kernels = flce.flce_timing_collect()
    ms = ev0.elapsed_time(ev1) / args.steps
    peak_mem = torch.cuda.max_memory_allocated()
    device_used = free_before - torch.cuda.mem_get_info()[0]
    counted = 8.0 * T * d * V
    value = counted / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    log(f"  {ms:.2f} ms/step (wall {wall / args.steps * 1e3:.2f} ms), {value:.1f} TFLOP/s, "
        f"{100 * value / peak:.1f}% of {peak} TFLOP/s")
    step_kernel_ms = sum(k["total_ms"] for k in kernels.values()) / args.steps
    # The backward skips ignored tokens, but the library counts each launch's
    # flops over its token block's capacity; the algorithmic flops of the
    # contraction kernels per step are 2*T_valid*d*V each (2*T*d*V forward).
    t_valid = int((inp.y != wl.IGNORE_INDEX).sum())
    alg_step = {"fwd_sweep": 2.0 * T * d * V, "bwd_dz": 2.0 * t_valid * d * V,
                "bwd_dhdw": 4.0 * t_valid * d * V}
    for name, k in kernels.items():
        if name in alg_step:
            k["flops"] = alg_step[name] * args.steps
    effective = (2.0 * T * d * V + 6.0 * t_valid * d * V) / (ms / 1e3) / 1e12
    for name, e in kernel_table(kernels, args.steps, ms).items():
        rate = f"{e['tflops']:7.1f} TFLOP/s" if "tflops" in e else f"{e['gbs']:7.1f} GB/s"
        log(f"  {name:10s} launches {e['launches']:5d}  avg {e['avg_ms']:8.3f} ms"
            f"  share {e['share']:6.1%}  {rate}")
    dom_name, dom = max(kernels.items(), key=lambda kv: kv[1]["total_ms"])
    avg_ms = dom["total_ms"] / dom["launches"]
    flops_per_launch = dom["flops"] / dom["launches"]
    achieved = flops_per_launch / (avg_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom_name, "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom_name, cfg.name, plan_key(plan)), "flops_per_launch": flops_per_launch,
                "avg_launch_ms": round(avg_ms, 4), "launches": dom["launches"]}

    shard = shard_leg(flce, wl, H, W, cfg, ws, stream, args.shard_steps) if args.shard_steps > 0 else None
    scoring = scoring_leg(flce, H, W, y, lse, stream) if args.shard_steps > 0 else None
    fused = fused_leg(flce, wl, plan, H, W, y, ws, stream, args.shard_steps) if args.shard_steps > 0 else None
    forms = forms_leg(flce, wl, plan, H, W, y, ws, stream, 2 * args.shard_steps + 1) if args.shard_steps > 0 else None

    lib_gemm = library_gemm_leg() if args.library_gemm else None
    cpu = None
    if args.cpu_rows > 0:
        log(f"cpu baseline: oracle on {args.cpu_rows} rows")
        cpu = cpu_baseline(inp, cfg, args.cpu_rows)
        log(f"  {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads ({cpu['seconds']:.1f} s)")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic" if args.data == "random" else f"synthetic, H and W {args.data}",
        "config": {"workload": cfg.name, "T": T, "d": d, "V": V, "precision": cfg.dtype,
                   "targets": cfg.targets, "ignored_tokens": cfg.n_ignored,
                   "grad_scale": gs, "parallelism": "single GPU"},
        "mfma_peak_frac": round(value / peak, 4),
        # the build's target for this workload: 60% of the dense MFMA peak
        "target_mfma_peak_frac": 0.6,
        "target_met": bool(value / peak >= 0.6),
        # 2*T*d*V + 6*T_valid*d*V per step: the work left once the backward
        # skips ignored tokens (equal to value when none are ignored)
        "effective_tflops": round(effective, 2),
        "valid_tokens": t_valid,
        "ignored_tokens_skipped_in_backward": True,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "memory": {"peak_allocated_bytes": int(peak_mem),
                   # hipMemGetInfo delta: what the step's process holds on the device
                   # (inputs, outputs, workspace, torch's cached blocks and context)
                   "device_used_delta_bytes": int(device_used),
                   "workspace_bytes": int(plan.ws_bytes),
                   "vocab_axis_workspace_bytes": int(plan.dz_ws_bytes),
                   "naive_logits_one_copy_bytes": int(plan.naive_logits_bytes),
                   "naive_logits_and_grad_bytes": int(2 * plan.naive_logits_bytes)},
        "kernels": kernel_table(kernels, args.steps, ms),
        "kernel_ms_per_step": round(step_kernel_ms, 3),
        "shard_mode": shard,
        "token_scoring": scoring,
        "fused_call": fused,
        "target_logit_forms": forms,
        "library_gemm": lib_gemm,
        "plan": {"fwd_splits": plan.fwd_splits, "bwd_block": plan.bwd_block,
                 "bwd_slab": plan.bwd_slab, "n_blocks": plan.n_blocks, "n_slabs": plan.n_slabs},
    }
    # the other workload configurations, each with its oracle host time (all
    # rows for the two small ones, a seeded sample with an extrapolation for
    # the others); the headline's buffers are released first
    others = [] if args.configs == "none" else [int(c) for c in args.configs.split(",") if c]
    if others and not args.shape:
        del H, W, y, ws, loss, lse, dH, dW
        torch.cuda.empty_cache()
        oracle_rows = {0: None, 1: None, 2: 1024, 3: 256, 4: 256}
        out["configs"] = {
            str(c): config_leg(flce, wl, wl.CONFIGS[c], min(args.steps, 10), min(args.warmup, 2),
                               oracle_rows[c] if args.cpu_rows > 0 else 0)
            for c in others if c != cfg.index}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
