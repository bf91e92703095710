"""Fused linear cross-entropy for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels in libflce.so, reached
through the C-ABI declared in include/flce.h; this package only marshals
arguments (torch supplies device memory and the stream).
"""
from ._lib import (EXPORTED, FLCE_BF16, FLCE_ERR_HIP, FLCE_ERR_INVALID_ARG, FLCE_ERR_UNSUPPORTED,
                   FLCE_ERR_WORKSPACE, FLCE_F32, FLCE_OK, FLCE_REDUCE_MEAN_VALID, FLCE_REDUCE_SUM,
                   FLCE_SCRATCH_BYTES, FLCE_TARGET_GATHER, FLCE_TARGET_IN_TILE,
                   TIMELINE_KERNELS, TIMELINE_LIB_PATH,
                   FlceError, KernelTime, Plan, WgRecord, flce_backward, flce_backward_shard,
                   flce_forward, flce_forward_backward, flce_forward_backward_scratch, flce_forward_shard,
                   flce_merge_shards,
                   flce_plan, flce_plan_status, flce_timeline_read, flce_timeline_reset,
                   flce_timing_collect, flce_timing_enable,
                   flce_token_logprobs, last_error, load, version, workspace)

__all__ = ["EXPORTED", "FLCE_BF16", "FLCE_ERR_HIP", "FLCE_ERR_INVALID_ARG", "FLCE_ERR_UNSUPPORTED",
           "FLCE_ERR_WORKSPACE", "FLCE_F32", "FLCE_OK", "FLCE_REDUCE_MEAN_VALID", "FLCE_REDUCE_SUM",
           "FLCE_SCRATCH_BYTES", "FLCE_TARGET_GATHER", "FLCE_TARGET_IN_TILE",
           "TIMELINE_KERNELS", "TIMELINE_LIB_PATH",
           "FlceError", "KernelTime", "Plan", "WgRecord", "flce_backward", "flce_backward_shard",
           "flce_forward", "flce_forward_backward", "flce_forward_backward_scratch",
           "flce_forward_shard",
           "flce_merge_shards", "flce_plan", "flce_plan_status", "flce_timeline_read",
           "flce_timeline_reset", "flce_timing_collect",
           "flce_timing_enable", "flce_token_logprobs", "last_error", "load", "version",
           "workspace"]
