"""ctypes binding of libflce.so: argument marshalling only.

Every entry point mirrors the C-ABI of include/flce.h under the same name.
Torch tensors are accepted for device buffers; only their data pointers,
shapes and the current HIP stream are passed on.  No arithmetic of the method
happens here, and there is no fallback: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FLCE_LIB", os.path.join(PKG, "libflce.so"))

FLCE_F32 = 0
FLCE_BF16 = 1
FLCE_OK = 0
FLCE_ERR_INVALID_ARG = -1
FLCE_ERR_UNSUPPORTED = -2
FLCE_ERR_WORKSPACE = -3
FLCE_ERR_HIP = -4
FLCE_REDUCE_SUM = 0
FLCE_REDUCE_MEAN_VALID = 1
FLCE_TARGET_IN_TILE = 0
FLCE_TARGET_GATHER = 1
# bytes of the library's static scratch array (FLCE_SCRATCH_BYTES in flce.h)
FLCE_SCRATCH_BYTES = 268435456

EXPORTED = ["flce_plan", "flce_forward", "flce_backward", "flce_forward_backward",
            "flce_forward_backward_scratch",
            "flce_forward_shard",
            "flce_merge_shards", "flce_backward_shard", "flce_token_logprobs", "flce_timing_enable",
            "flce_timing_collect", "flce_timeline_reset", "flce_timeline_read",
            "flce_status_string", "flce_last_error", "flce_version"]
# libflce_timeline.so: the same library with the per-workgroup timeline
TIMELINE_LIB_PATH = os.path.join(PKG, "libflce_timeline.so")
# flce_wg_record_t.kernel
TIMELINE_KERNELS = {1: "fwd_sweep", 2: "bwd_dz", 3: "bwd_dhdw:dH", 4: "bwd_dhdw:dW"}


class Plan(ctypes.Structure):
    """Mirror of flce_plan_t."""
    _fields_ = [
        ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("V", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
        ("tile_v", ctypes.c_int32), ("tile_t", ctypes.c_int32),
        ("fwd_splits", ctypes.c_int32), ("fwd_tiles_per_split", ctypes.c_int32),
        ("bwd_block", ctypes.c_int64), ("bwd_slab", ctypes.c_int64),
        ("n_blocks", ctypes.c_int64), ("n_slabs", ctypes.c_int64),
        ("fwd_ws_bytes", ctypes.c_uint64), ("dz_ws_bytes", ctypes.c_uint64),
        ("dh_acc_bytes", ctypes.c_uint64), ("bwd_ws_bytes", ctypes.c_uint64),
        ("ws_bytes", ctypes.c_uint64), ("vocab_ws_cap", ctypes.c_uint64),
        ("naive_logits_bytes", ctypes.c_uint64), ("dh_split_bytes", ctypes.c_uint64),
        ("magic", ctypes.c_uint32), ("target_logit", ctypes.c_uint32),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class KernelTime(ctypes.Structure):
    """Mirror of flce_kernel_time_t."""
    _fields_ = [("name", ctypes.c_char * 24), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class WgRecord(ctypes.Structure):
    """Mirror of flce_wg_record_t."""
    _fields_ = [("hw_id", ctypes.c_uint32), ("xcc_id", ctypes.c_uint32),
                ("t_start", ctypes.c_uint64), ("t_end", ctypes.c_uint64),
                ("kernel", ctypes.c_uint32), ("block", ctypes.c_uint32)]


class FlceError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"flce status {status}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Loads libflce.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m linear_cross_entropy_flce_amd.build` "
                          "(or __graft_entry__.build()) first -- there is no fallback path")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Plan)
    vp, i64, f32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64
    lib.flce_plan.argtypes = [i64, i64, i64, ctypes.c_int, u64, P]
    lib.flce_plan.restype = ctypes.c_int
    lib.flce_forward.argtypes = [P, vp, vp, vp, i64, f32, vp, vp, vp, vp, u64, vp]
    lib.flce_forward.restype = ctypes.c_int
    lib.flce_backward.argtypes = [P, vp, vp, vp, vp, i64, f32, vp, vp, ctypes.c_int, vp, u64, vp]
    lib.flce_backward.restype = ctypes.c_int
    lib.flce_forward_backward.argtypes = [P, vp, vp, vp, i64, ctypes.c_int, f32, vp, vp, vp, vp,
                                          vp, ctypes.c_int, vp, vp, u64, vp]
    lib.flce_forward_backward.restype = ctypes.c_int
    lib.flce_forward_backward_scratch.argtypes = [P, vp, vp, vp, i64, ctypes.c_int, f32, vp, vp,
                                                  vp, vp, vp, ctypes.c_int, vp, vp]
    lib.flce_forward_backward_scratch.restype = ctypes.c_int
    lib.flce_forward_shard.argtypes = [P, vp, vp, vp, i64, i64, i64, vp, vp, vp, u64, vp]
    lib.flce_forward_shard.restype = ctypes.c_int
    lib.flce_merge_shards.argtypes = [i64, ctypes.c_int32, vp, vp, vp, i64, i64, f32, vp, vp, vp,
                                      vp]
    lib.flce_merge_shards.restype = ctypes.c_int
    lib.flce_backward_shard.argtypes = [P, vp, vp, vp, vp, i64, i64, i64, f32, vp, vp,
                                        ctypes.c_int, vp, u64, vp]
    lib.flce_backward_shard.restype = ctypes.c_int
    lib.flce_token_logprobs.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, vp, i64, vp, vp, vp]
    lib.flce_token_logprobs.restype = ctypes.c_int
    lib.flce_timing_enable.argtypes = [ctypes.c_int]
    lib.flce_timing_enable.restype = ctypes.c_int
    lib.flce_timing_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int)]
    lib.flce_timing_collect.restype = ctypes.c_int
    lib.flce_timeline_reset.argtypes = []
    lib.flce_timeline_reset.restype = ctypes.c_int
    lib.flce_timeline_read.argtypes = [ctypes.POINTER(WgRecord), ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int)]
    lib.flce_timeline_read.restype = ctypes.c_int
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_last_error.argtypes = []
    lib.flce_last_error.restype = ctypes.c_char_p
    lib.flce_version.argtypes = []
    lib.flce_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != FLCE_OK:
        lib = load()
        raise FlceError(status, lib.flce_status_string(status).decode() + ": " +
                        lib.flce_last_error().decode())


def last_error() -> str:
    return load().flce_last_error().decode()


def version() -> str:
    return load().flce_version().decode()


# ------------------------------------------------------------ marshalling

def _ptr(x) -> int | None:
    """Device pointer of a tensor, an int pointer, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(dtype) -> int:
    import torch
    if dtype in (torch.bfloat16, "bf16", FLCE_BF16):
        return FLCE_BF16
    if dtype in (torch.float32, "f32", FLCE_F32):
        return FLCE_F32
    raise ValueError(f"unsupported dtype {dtype}")


def flce_timing_enable(enable: bool = True) -> None:
    """flce_timing_enable(): bracket every library launch with hipEvents."""
    _check(load().flce_timing_enable(1 if enable else 0))


def flce_timing_collect() -> dict:
    """flce_timing_collect(): {kernel: dict(launches, total_ms, flops, bytes)}; clears."""
    buf = (KernelTime * 16)()
    n = ctypes.c_int(0)
    _check(load().flce_timing_collect(buf, 16, ctypes.byref(n)))
    return {buf[i].name.decode(): dict(launches=buf[i].launches, total_ms=buf[i].total_ms,
                                       flops=buf[i].flops, bytes=buf[i].bytes)
            for i in range(n.value)}


def flce_timeline_reset() -> None:
    """flce_timeline_reset(): raises FlceError (FLCE_ERR_UNSUPPORTED) unless the
    loaded library is libflce_timeline.so."""
    _check(load().flce_timeline_reset())


def flce_timeline_read(max_records: int = 1 << 19):
    """flce_timeline_read(): the records as a list of WgRecord."""
    buf = (WgRecord * max_records)()
    n = ctypes.c_int(0)
    _check(load().flce_timeline_read(buf, max_records, ctypes.byref(n)))
    return buf[:n.value]


def flce_plan(T: int, d: int, V: int, dtype, vocab_ws_cap_bytes: int = 0) -> Plan:
    """flce_plan(): host-only planning.  dtype: torch dtype, 'bf16'/'f32' or code."""
    code = _dtype_code(dtype) if not isinstance(dtype, int) or dtype in (0, 1) else dtype
    p = Plan()
    _check(load().flce_plan(int(T), int(d), int(V), int(code), int(vocab_ws_cap_bytes),
                            ctypes.byref(p)))
    return p


def flce_plan_status(T, d, V, dtype_code: int, cap: int = 0):
    """Raw status of flce_plan (for tests of the error paths)."""
    p = Plan()
    st = load().flce_plan(int(T), int(d), int(V), int(dtype_code), int(cap), ctypes.byref(p))
    return st, p


def workspace(plan: Plan, device="cuda"):
    """A caller-owned workspace of plan.ws_bytes (torch uint8 tensor)."""
    import torch
    return torch.empty(max(int(plan.ws_bytes), 16), dtype=torch.uint8, device=device)


def _check_tensor(name, t, shape, dtype):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _elem_dtype(plan: Plan):
    import torch
    return torch.bfloat16 if plan.dtype == FLCE_BF16 else torch.float32


def flce_forward(plan: Plan, H, W, y, ignore_index: int = -100, scale: float = 1.0, loss=None,
                 lse=None, loss_reduced=None, ws=None, stream=None):
    """flce_forward(): returns (loss, lse, loss_reduced or None) as tensors.

    Outputs not given are allocated with torch on W's device."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    dev = W.device
    et = _elem_dtype(plan)
    _check_tensor("H", H, (T, d), et)
    _check_tensor("W", W, (V, d), et)
    _check_tensor("y", y, (T,), torch.int64)
    if loss is None:
        loss = torch.empty(T, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(T, dtype=torch.float32, device=dev)
    _check_tensor("loss", loss, (T,), torch.float32)
    _check_tensor("lse", lse, (T,), torch.float32)
    if ws is None:
        ws = workspace(plan, dev)
    _check(load().flce_forward(ctypes.byref(plan), _ptr(H), _ptr(W), _ptr(y), int(ignore_index),
                               float(scale), _ptr(loss), _ptr(lse), _ptr(loss_reduced), _ptr(ws),
                               int(ws.numel() * ws.element_size()), _stream(stream)))
    return loss, lse, loss_reduced


def flce_backward(plan: Plan, H, W, y, lse, ignore_index: int = -100, grad_scale: float = 1.0,
                  dH=None, dW=None, accumulate_dW: bool = False, ws=None, stream=None):
    """flce_backward(): returns (dH, dW).  dW is float32 [V, d]."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    dev = W.device
    et = _elem_dtype(plan)
    _check_tensor("H", H, (T, d), et)
    _check_tensor("W", W, (V, d), et)
    _check_tensor("y", y, (T,), torch.int64)
    _check_tensor("lse", lse, (T,), torch.float32)
    if dH is None:
        dH = torch.empty((T, d), dtype=et, device=dev)
    if dW is None:
        if accumulate_dW:
            raise ValueError("accumulate_dW needs an existing dW")
        dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    _check_tensor("dH", dH, (T, d), et)
    _check_tensor("dW", dW, (V, d), torch.float32)
    if ws is None:
        ws = workspace(plan, dev)
    _check(load().flce_backward(ctypes.byref(plan), _ptr(H), _ptr(W), _ptr(y), _ptr(lse),
                                int(ignore_index), float(grad_scale), _ptr(dH), _ptr(dW),
                                1 if accumulate_dW else 0, _ptr(ws),
                                int(ws.numel() * ws.element_size()), _stream(stream)))
    return dH, dW


def flce_forward_shard(plan: Plan, H, W_shard, y, vocab_start: int, vocab_total: int,
                       ignore_index: int = -100, lse_shard=None, zt_shard=None, ws=None,
                       stream=None):
    """flce_forward_shard(): returns (lse_shard, zt_shard) of one vocab shard.

    plan is for the shard (V = its rows); y holds global vocab ids."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    dev = W_shard.device
    et = _elem_dtype(plan)
    _check_tensor("H", H, (T, d), et)
    _check_tensor("W_shard", W_shard, (V, d), et)
    _check_tensor("y", y, (T,), torch.int64)
    if lse_shard is None:
        lse_shard = torch.empty(T, dtype=torch.float32, device=dev)
    if zt_shard is None:
        zt_shard = torch.empty(T, dtype=torch.float32, device=dev)
    _check_tensor("lse_shard", lse_shard, (T,), torch.float32)
    _check_tensor("zt_shard", zt_shard, (T,), torch.float32)
    if ws is None:
        ws = workspace(plan, dev)
    _check(load().flce_forward_shard(ctypes.byref(plan), _ptr(H), _ptr(W_shard), _ptr(y),
                                     int(ignore_index), int(vocab_start), int(vocab_total),
                                     _ptr(lse_shard), _ptr(zt_shard), _ptr(ws),
                                     int(ws.numel() * ws.element_size()), _stream(stream)))
    return lse_shard, zt_shard


def flce_merge_shards(lse_shards, zt_shards, y, vocab_total: int, ignore_index: int = -100,
                      scale: float = 1.0, loss=None, lse=None, loss_reduced=None, stream=None):
    """flce_merge_shards(): lse_shards, zt_shards [n_shards, T] -> (loss, lse, loss_reduced)."""
    import torch
    if lse_shards.dim() != 2:
        raise ValueError("lse_shards must be [n_shards, T]")
    P, T = lse_shards.shape
    dev = lse_shards.device
    _check_tensor("lse_shards", lse_shards, (P, T), torch.float32)
    _check_tensor("zt_shards", zt_shards, (P, T), torch.float32)
    _check_tensor("y", y, (T,), torch.int64)
    if loss is None:
        loss = torch.empty(T, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(T, dtype=torch.float32, device=dev)
    _check_tensor("loss", loss, (T,), torch.float32)
    _check_tensor("lse", lse, (T,), torch.float32)
    _check(load().flce_merge_shards(int(T), int(P), _ptr(lse_shards), _ptr(zt_shards), _ptr(y),
                                    int(ignore_index), int(vocab_total), float(scale), _ptr(loss),
                                    _ptr(lse), _ptr(loss_reduced), _stream(stream)))
    return loss, lse, loss_reduced


def flce_backward_shard(plan: Plan, H, W_shard, y, lse, vocab_start: int, vocab_total: int,
                        ignore_index: int = -100, grad_scale: float = 1.0, dH_partial=None,
                        dW_shard=None, accumulate_dW: bool = False, ws=None, stream=None):
    """flce_backward_shard(): returns (dH_partial, dW_shard); lse is the merged one."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    dev = W_shard.device
    et = _elem_dtype(plan)
    _check_tensor("H", H, (T, d), et)
    _check_tensor("W_shard", W_shard, (V, d), et)
    _check_tensor("y", y, (T,), torch.int64)
    _check_tensor("lse", lse, (T,), torch.float32)
    if dH_partial is None:
        dH_partial = torch.empty((T, d), dtype=et, device=dev)
    if dW_shard is None:
        if accumulate_dW:
            raise ValueError("accumulate_dW needs an existing dW_shard")
        dW_shard = torch.empty((V, d), dtype=torch.float32, device=dev)
    _check_tensor("dH_partial", dH_partial, (T, d), et)
    _check_tensor("dW_shard", dW_shard, (V, d), torch.float32)
    if ws is None:
        ws = workspace(plan, dev)
    _check(load().flce_backward_shard(ctypes.byref(plan), _ptr(H), _ptr(W_shard), _ptr(y),
                                      _ptr(lse), int(ignore_index), int(vocab_start),
                                      int(vocab_total), float(grad_scale), _ptr(dH_partial),
                                      _ptr(dW_shard), 1 if accumulate_dW else 0, _ptr(ws),
                                      int(ws.numel() * ws.element_size()), _stream(stream)))
    return dH_partial, dW_shard


def flce_token_logprobs(H, W, tokens, lse=None, out=None, stream=None):
    """flce_token_logprobs(): out [T, K] = H[t] . W[tokens[t, k]] - lse[t].

    tokens: int64 [T, K] (or [T] for K = 1); lse None gives the logits."""
    import torch
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1] or H.dtype != W.dtype:
        raise ValueError("H [T, d] and W [V, d] of one dtype")
    T, d = H.shape
    V = W.shape[0]
    tok = tokens if tokens.dim() == 2 else tokens.view(-1, 1)
    K = tok.shape[1]
    _check_tensor("H", H, (T, d), H.dtype)
    _check_tensor("W", W, (V, d), H.dtype)
    _check_tensor("tokens", tok, (T, K), torch.int64)
    _check_tensor("lse", lse, (T,), torch.float32)
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=W.device)
    _check_tensor("out", out, (T, K), torch.float32)
    _check(load().flce_token_logprobs(int(T), int(d), int(V), _dtype_code(H.dtype), _ptr(H),
                                      _ptr(W), _ptr(tok), int(K), _ptr(lse), _ptr(out),
                                      _stream(stream)))
    return out if tokens.dim() == 2 else out.view(-1)


_REDUCTIONS = {"sum": FLCE_REDUCE_SUM, "mean_valid": FLCE_REDUCE_MEAN_VALID,
               FLCE_REDUCE_SUM: FLCE_REDUCE_SUM, FLCE_REDUCE_MEAN_VALID: FLCE_REDUCE_MEAN_VALID}


def flce_forward_backward(plan: Plan, H, W, y, ignore_index: int = -100, reduction="sum",
                          scale: float = 1.0, loss=None, lse=None, loss_reduced=None, dH=None,
                          dW=None, accumulate_dW: bool = False, dW_bf16=None, ws=None,
                          stream=None):
    """flce_forward_backward(): returns dict(loss, lse, loss_reduced, dH, dW, dW_bf16).

    reduction: "sum" (g = scale) or "mean_valid" (g = scale / #non-ignored
    tokens, counted on the device)."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    dev = W.device
    et = _elem_dtype(plan)
    if reduction not in _REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    _check_tensor("H", H, (T, d), et)
    _check_tensor("W", W, (V, d), et)
    _check_tensor("y", y, (T,), torch.int64)
    if loss is None:
        loss = torch.empty(T, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(T, dtype=torch.float32, device=dev)
    if loss_reduced is None:
        loss_reduced = torch.empty(1, dtype=torch.float32, device=dev)
    if dH is None:
        dH = torch.empty((T, d), dtype=et, device=dev)
    if dW is None:
        if accumulate_dW:
            raise ValueError("accumulate_dW needs an existing dW")
        dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    _check_tensor("loss", loss, (T,), torch.float32)
    _check_tensor("lse", lse, (T,), torch.float32)
    _check_tensor("loss_reduced", loss_reduced, (1,), torch.float32)
    _check_tensor("dH", dH, (T, d), et)
    _check_tensor("dW", dW, (V, d), torch.float32)
    _check_tensor("dW_bf16", dW_bf16, (V, d), torch.bfloat16)
    if ws is None:
        ws = workspace(plan, dev)
    _check(load().flce_forward_backward(ctypes.byref(plan), _ptr(H), _ptr(W), _ptr(y),
                                        int(ignore_index), _REDUCTIONS[reduction], float(scale),
                                        _ptr(loss), _ptr(lse), _ptr(loss_reduced), _ptr(dH),
                                        _ptr(dW), 1 if accumulate_dW else 0, _ptr(dW_bf16),
                                        _ptr(ws), int(ws.numel() * ws.element_size()),
                                        _stream(stream)))
    return dict(loss=loss, lse=lse, loss_reduced=loss_reduced, dH=dH, dW=dW, dW_bf16=dW_bf16)


def flce_forward_backward_scratch(plan: Plan, H, W, y, ignore_index: int, reduction: str,
                                  scale: float, loss, lse, loss_reduced, dH, dW,
                                  accumulate_dW: bool = False, dW_bf16=None, stream=None):
    """flce_forward_backward_scratch(): flce_forward_backward on the library's
    own scratch array.  Every output is the caller's (nothing is allocated
    here either); loss_reduced and dW_bf16 may be None.  Returns None."""
    import torch
    T, d, V = plan.T, plan.d, plan.V
    et = _elem_dtype(plan)
    if reduction not in _REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    for name, t in (("loss", loss), ("lse", lse), ("dH", dH), ("dW", dW)):
        if t is None:
            raise ValueError(f"{name} must be given: this call allocates nothing")
    _check_tensor("H", H, (T, d), et)
    _check_tensor("W", W, (V, d), et)
    _check_tensor("y", y, (T,), torch.int64)
    _check_tensor("loss", loss, (T,), torch.float32)
    _check_tensor("lse", lse, (T,), torch.float32)
    _check_tensor("loss_reduced", loss_reduced, (1,), torch.float32)
    _check_tensor("dH", dH, (T, d), et)
    _check_tensor("dW", dW, (V, d), torch.float32)
    _check_tensor("dW_bf16", dW_bf16, (V, d), torch.bfloat16)
    _check(load().flce_forward_backward_scratch(
        ctypes.byref(plan), _ptr(H), _ptr(W), _ptr(y), int(ignore_index), _REDUCTIONS[reduction],
        float(scale), _ptr(loss), _ptr(lse), _ptr(loss_reduced), _ptr(dH), _ptr(dW),
        1 if accumulate_dW else 0, _ptr(dW_bf16), _stream(stream)))
