/*
 * flce.h -- fused linear cross-entropy on AMD Instinct MI355X (gfx950).
 *
 * The operation ("Long-Sequence MoE RL Training: From First Principles to
 * MI300X", section 3, Linear cross-entropy): for hidden states H [T x d] and
 * an LM-head weight W [V x d], the logits are Z = H W^T [T x V].  Each token
 * row is reduced to one cross-entropy value,
 *     lse_i  = log sum_j exp(Z_ij)
 *     loss_i = lse_i - Z_{i, y_i}          (= -log softmax(Z_i)[y_i]),
 * and the backward needs only dZ = softmax(Z) - onehot(y), contracted into
 *     dH = dZ W      and      dW = dZ^T H   (the page writes dW^T = H^T dZ).
 * Z is never materialised: the forward streams vocabulary tiles through a
 * running-max / log-sum-exp recurrence keeping O(block) scalars per token,
 * and the backward recomputes each logit tile, forms its dZ tile and
 * contracts it immediately, so vocab-axis residency is bounded by
 * [token block x vocab slab] instead of [tokens x vocab] (same section; the
 * Megatron-Lite / bumblebee write-up, section 2.3 step 1, streams along the
 * vocab dimension in the same way).
 *
 * Conventions shared by every call:
 *   - Matrices are row-major and dense: H[t*d + k], W[v*d + k], dH[t*d + k],
 *     dW[v*d + k].  Element type of H, W and dH is the plan's dtype
 *     (FLCE_BF16: bfloat16 bits, FLCE_F32: float); dW is always float.
 *   - Targets y are int64 [T].  y_i == ignore_index marks an ignored token:
 *     loss_i = 0 and its dZ row is zero (its lse is still computed).  A
 *     target outside [0, V) that is not ignore_index is a precondition
 *     violation: that token's loss and its dH row are NaN, and so is every
 *     element of dW (its dZ row is NaN, and each dW row sums over all tokens);
 *     its lse, and the loss and dH rows of the other tokens, are unaffected.
 *   - Every pointer argument except the host plan is device memory owned by
 *     the caller.  The library never allocates device memory, never
 *     synchronises the host, and keeps no state between calls other than a
 *     thread-local error string.  All work is ordered on `stream` (a
 *     hipStream_t; NULL means the default stream).
 *   - Requirements: T >= 0, V >= 1, d >= 8 and d % 8 == 0, T, V < 2^31,
 *     d <= 65536, device pointers 16-byte aligned.  H, W and dW may be larger
 *     than 2 GiB.
 *     Violations are reported before anything is launched.
 *   - Results are bitwise reproducible for identical inputs and plan: every
 *     reduction runs in a fixed order, and no floating-point atomics are used.
 *   - Errors are returned as flce_status_t; nothing throws across the ABI.
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flce_dtype { FLCE_F32 = 0, FLCE_BF16 = 1 } flce_dtype_t;

typedef enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad plan */
  FLCE_ERR_UNSUPPORTED = -2, /* shape or alignment outside the requirements */
  FLCE_ERR_WORKSPACE = -3,   /* workspace too small, or cap below the minimum */
  FLCE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} flce_status_t;

/* A launch plan.  Plain data: produced on the host by flce_plan(), read by
 * flce_forward()/flce_backward(); it may be copied freely. */
typedef struct flce_plan {
  int64_t T, d, V;
  int32_t dtype;          /* flce_dtype_t */
  int32_t elem_bytes;     /* 2 (bf16) or 4 (f32) */
  /* forward: tiles of tile_v vocab rows x tile_t tokens; the vocab axis is
   * cut into fwd_splits contiguous ranges reduced independently and merged */
  int32_t tile_v, tile_t;
  int32_t fwd_splits;
  int32_t fwd_tiles_per_split; /* vocab tiles in each split */
  /* backward: token blocks of bwd_block tokens x vocab slabs of bwd_slab */
  int64_t bwd_block, bwd_slab;
  int64_t n_blocks, n_slabs;
  /* workspace (bytes); one buffer of ws_bytes serves both calls */
  uint64_t fwd_ws_bytes;   /* per-split (max, sum) partials + target logits */
  uint64_t dz_ws_bytes;    /* the [bwd_block x bwd_slab] dZ tile buffer */
  uint64_t dh_acc_bytes;   /* fp32 dH accumulator, 0 when there is one slab */
  uint64_t bwd_ws_bytes;   /* dz_ws_bytes + dh_acc_bytes + 2 x bwd_block x d elements (the
                              token block's H as rows and transposed) + the compacted
                              token order (4 bytes per token) and counters
                              + dh_split_bytes */
  uint64_t ws_bytes;       /* max(fwd_ws_bytes, bwd_ws_bytes) + 256: enough for every call,
                              flce_forward_backward's device scalars included */
  uint64_t vocab_ws_cap;   /* the cap the planner honoured */
  /* context: bytes of one materialised [T x V] logits copy in the dtype */
  uint64_t naive_logits_bytes;
  /* fp32 partial tiles that let dH split its vocab (K) loop when a token
   * block has too few tiles to occupy every compute unit (small T or d, or a
   * block thinned by ignored tokens); the device picks the split from the
   * block's token count.  0 when they do not fit under the cap beside the
   * chosen block and slab (dH then never splits). */
  uint64_t dh_split_bytes;
  uint32_t magic;          /* set by flce_plan; checked by the other calls */
  uint32_t target_logit;   /* flce_target_logit_t: how the forward takes each token's
                              target logit; flce_plan sets the default, and a caller
                              may change it in its copy of the plan */
} flce_plan_t;

/* Two forms of the forward's target logit z_{i, y_i}:
 *   FLCE_TARGET_IN_TILE: each vocab tile's epilogue compares its rows with
 *     the tokens' targets and keeps the matching fp32 accumulator value; lse
 *     and z_t then come from the same rounded logits.
 *   FLCE_TARGET_GATHER: the sweep is a pure log-sum-exp (no per-tile target
 *     test) and z_t = H[i] . W[y_i] is one gathered dot product per token
 *     afterwards (Cut Cross-Entropy indexes only the target logit; first
 *     page, section 3).  Its fp32 sum runs in another order than the tile's,
 *     so loss may differ from the other form by fp32 rounding of |z|. */
typedef enum { FLCE_TARGET_IN_TILE = 0, FLCE_TARGET_GATHER = 1 } flce_target_logit_t;

/* flce_plan -- choose tiles, splits, token block and vocab slab.
 * Section 3 of the first page bounds the method's vocab-axis residency by one
 * token block times the vocabulary ([block x vocab], under a gigabyte, down
 * from [tokens x vocab]); section 8 asks for tiles sized to 64-lane waves and
 * LDS.  The plan fixes the [bwd_block x bwd_slab] buffer that bounds this
 * residency, and the MFMA tile shapes the kernels use.
 *   T, d, V : problem size (see requirements above).
 *   dtype   : element type of H, W, dH.
 *   vocab_ws_cap_bytes : upper bound for the backward workspace (the dZ
 *             buffer, the fp32 dH accumulator, the gathered H block and the
 *             token order); 0 selects the default of
 *             950,000,000 bytes, keeping vocab-axis residency below 1 GB.
 *             Caps above 2^31 - 65536 bytes are lowered to that value.
 *   out     : host pointer, filled on success.
 * Host-only integer arithmetic; launches nothing.  Returns
 * FLCE_ERR_INVALID_ARG for a null `out`, negative/zero sizes or an unknown
 * dtype, FLCE_ERR_UNSUPPORTED for d % 8 != 0 or sizes beyond the limits, and
 * FLCE_ERR_WORKSPACE when the cap cannot hold the smallest token block.
 * A vocab slab's rows of W (bwd_slab x d elements) are kept below 2^31 bytes. */
flce_status_t flce_plan(int64_t T, int64_t d, int64_t V, flce_dtype_t dtype,
                        uint64_t vocab_ws_cap_bytes, flce_plan_t* out);

/* flce_forward -- per-token loss and lse (section 3 of the first page).
 *   H [T x d], W [V x d] in the plan's dtype; y [T] int64.
 *   scale   : multiplies the optional reduced loss only (1/N gives a mean).
 *   loss [T], lse [T] : float outputs; loss is the unscaled per-token value.
 *   loss_reduced : NULL, or a device float that receives scale * sum(loss)
 *             (summed in a fixed order, in double precision).
 *   ws, ws_bytes : caller workspace of at least plan->fwd_ws_bytes.
 * The target logit is taken as plan->target_logit says (FLCE_ERR_INVALID_ARG
 * for another value).  T == 0 is valid and writes only loss_reduced (= 0). */
flce_status_t flce_forward(const flce_plan_t* plan, const void* H, const void* W,
                           const int64_t* y, int64_t ignore_index, float scale, float* loss,
                           float* lse, float* loss_reduced, void* ws, uint64_t ws_bytes,
                           void* stream);

/* flce_backward -- dH and dW of grad_scale * sum_i loss_i.
 * Section 3 of the first page: the backward recomputes each logit tile from
 * the still-resident H and W, forms dZ = softmax(Z) - onehot(y) for that tile
 * and contracts it into dH = dZ W and dW^T = H^T dZ; here dZ lives for one
 * [bwd_block x bwd_slab] tile buffer at a time (bf16 for bf16 inputs).
 *   Ignored tokens contribute nothing (their dZ rows are zero), so the
 *   backward compacts the other tokens on the device (ascending order) and
 *   runs its contractions over them only; their dH rows are written as 0.
 *   lse [T]  : the forward's output for the same H, W (its normaliser lets
 *              the recompute form softmax without a running max).
 *   grad_scale : scalar multiplying every dZ element (1/N for a mean).
 *   dH [T x d] : output in the plan's dtype (fp32 accumulation, rounded to
 *              nearest even once at the end for bf16).
 *   dW [V x d] : float; overwritten, or accumulated into when
 *              accumulate_dW != 0 (gradient accumulation across calls).
 *   ws, ws_bytes : caller workspace of at least plan->bwd_ws_bytes.
 * T == 0 is valid: dW is zeroed (or left as is when accumulating). */
flce_status_t flce_backward(const flce_plan_t* plan, const void* H, const void* W,
                            const int64_t* y, const float* lse, int64_t ignore_index,
                            float grad_scale, void* dH, float* dW, int accumulate_dW, void* ws,
                            uint64_t ws_bytes, void* stream);

/* How flce_forward_backward reduces the per-token losses. */
typedef enum {
  FLCE_REDUCE_SUM = 0,        /* loss_reduced = scale * sum(loss), g = scale */
  FLCE_REDUCE_MEAN_VALID = 1  /* divided by the number of tokens with y != ignore_index,
                                 counted on the device (0 tokens: loss_reduced = 0, g = 0) */
} flce_reduction_t;

/* flce_forward_backward -- forward, reduction and backward in one call, for
 * training steps where the gradient scale follows from the reduction: the
 * mean over non-ignored tokens needs their count, which is taken on the GPU
 * and passed to the backward there, with no host round trip.
 *   Arguments as flce_forward and flce_backward; grad scale g as above.
 *   dW [V x d] float: overwritten, or accumulated into when accumulate_dW
 *       != 0 (the fp32 main gradient across micro-batches).
 *   dW_bf16 : NULL, or [V x d] bf16 that receives dW rounded to nearest
 *       even after the call's accumulation.  The dW tiles of the last token
 *       block that holds a non-ignored token write it as they store the final
 *       dW, so it costs no pass over dW of its own (except when T == 0).
 *   ws, ws_bytes : at least plan->ws_bytes.
 * Errors as flce_forward / flce_backward, and FLCE_ERR_INVALID_ARG for an
 * unknown reduction.  Outputs equal flce_forward then flce_backward with the
 * same g, bit for bit. */
flce_status_t flce_forward_backward(const flce_plan_t* plan, const void* H, const void* W,
                                    const int64_t* y, int64_t ignore_index,
                                    flce_reduction_t reduction, float scale, float* loss,
                                    float* lse, float* loss_reduced, void* dH, float* dW,
                                    int accumulate_dW, void* dW_bf16, void* ws, uint64_t ws_bytes,
                                    void* stream);

/* ---- allocation-free variant ---------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * flce_forward_backward_scratch is flce_forward_backward with the library's
 * own static scratch array of FLCE_SCRATCH_BYTES as the workspace: a
 * file-scope device array that every GPU running the library holds until the
 * process ends.  The caller passes inputs and outputs only.  The plan must
 * fit: plan->ws_bytes <= FLCE_SCRATCH_BYTES, which flce_plan() guarantees
 * with vocab_ws_cap_bytes = FLCE_SCRATCH_BYTES - 256 unless the forward's
 * per-token partials alone exceed it (T of several million); otherwise
 * FLCE_ERR_WORKSPACE, before anything is launched.  The first call on a
 * device looks up the array's device address (FLCE_ERR_HIP if that fails)
 * and keeps it; no call allocates, frees or copies memory: it only launches
 * kernels on `stream`.  The array keeps the last call's contents; every byte
 * a call reads is written earlier in the same call.  Calls that overlap on
 * one GPU (other streams, other threads) share the array and race: the
 * caller serialises them.  Kernel timing (flce_timing_enable) does not
 * record these calls.  Results are bit for bit those of
 * flce_forward_backward with the same plan and arguments. */
#define FLCE_SCRATCH_BYTES 268435456ull
flce_status_t flce_forward_backward_scratch(const flce_plan_t* plan, const void* H,
                                            const void* W, const int64_t* y, int64_t ignore_index,
                                            flce_reduction_t reduction, float scale, float* loss,
                                            float* lse, float* loss_reduced, void* dH, float* dW,
                                            int accumulate_dW, void* dW_bf16, void* stream);

/* ---- vocab-parallel shard mode ------------------------------------------
 * The Megatron-Lite / bumblebee write-up (section 2.3, step 1) runs this loss
 * vocab-parallel: each of P tensor-parallel ranks holds a contiguous slice of
 * W's rows.  A shard's forward reduces its own vocab slice to two per-token
 * statistics; gathering them from all P shards and merging gives the same
 * loss and lse as the unsharded forward; the backward of each shard then
 * needs only the merged lse.  The calls below are the per-GPU parts; the
 * exchange between them (an all-gather of 8 * T bytes per shard, and a sum
 * of the P partial dH) is the caller's.
 *
 * A shard plan is flce_plan(T, d, V_local, ...), V_local the shard's rows;
 * the shard is vocab ids [vocab_start, vocab_start + V_local) of a vocabulary
 * of vocab_total ids, and targets y stay global ids.  FLCE_ERR_INVALID_ARG
 * when vocab_total is outside [1, 2^31) or the shard does not lie inside it.
 */

/* flce_forward_shard -- per-token statistics of one vocab shard.
 *   W_shard [V_local x d] : the shard's rows of W, in the plan's dtype.
 *   lse_shard [T] : float, log sum over the shard's ids of exp(logit).
 *   zt_shard  [T] : float, the target logit when y lies in the shard, else
 *                   -inf (also for ignored tokens).
 *   ws, ws_bytes : as flce_forward (plan->fwd_ws_bytes).
 * Other arguments and errors as flce_forward. */
flce_status_t flce_forward_shard(const flce_plan_t* plan, const void* H, const void* W_shard,
                                 const int64_t* y, int64_t ignore_index, int64_t vocab_start,
                                 int64_t vocab_total, float* lse_shard, float* zt_shard, void* ws,
                                 uint64_t ws_bytes, void* stream);

/* flce_merge_shards -- loss and lse from the statistics of n_shards shards.
 *   lse_shards, zt_shards : device floats [n_shards x T] (shard-major, as an
 *             all-gather lays them out), each row from flce_forward_shard.
 *   The merged lse is the log-sum-exp of the shards' lse, in ascending shard
 *   order; the target logit is the one finite zt.  loss as flce_forward:
 *   0 for ignored tokens, NaN for targets outside [0, vocab_total) and for
 *   valid targets that no shard holds; loss_reduced (optional) =
 *   scale * sum(loss) in a fixed order.  Any shard order gives the same
 *   result up to rounding; the same order on every rank gives identical bits.
 * FLCE_ERR_INVALID_ARG for T outside [0, 2^31), n_shards < 1 or above
 * vocab_total, or NULL buffers when T > 0. */
flce_status_t flce_merge_shards(int64_t T, int32_t n_shards, const float* lse_shards,
                                const float* zt_shards, const int64_t* y, int64_t ignore_index,
                                int64_t vocab_total, float scale, float* loss, float* lse,
                                float* loss_reduced, void* stream);

/* flce_backward_shard -- one shard's part of dH and its slice of dW.
 *   lse [T]  : the merged lse over the whole vocabulary.
 *   dH_partial [T x d] : this shard's term dZ_shard * W_shard, in the plan's
 *              dtype; dH is the sum of the P partials.
 *   dW_shard [V_local x d] : float, rows vocab_start.. of dW (overwritten or
 *              accumulated as flce_backward).
 * Tokens whose target lies in another shard contribute their softmax only;
 * the one-hot term lands in the shard that holds the target.  Other
 * arguments, workspace and errors as flce_backward. */
flce_status_t flce_backward_shard(const flce_plan_t* plan, const void* H, const void* W_shard,
                                  const int64_t* y, const float* lse, int64_t ignore_index,
                                  int64_t vocab_start, int64_t vocab_total, float grad_scale,
                                  void* dH_partial, float* dW_shard, int accumulate_dW, void* ws,
                                  uint64_t ws_bytes, void* stream);

/* flce_token_logprobs -- log-probabilities of given tokens.
 *   out[t*K + k] = H[t] . W[tokens[t*K + k]] - lse[t]: the log-softmax of
 *   the logits of the first page's section 3 at the named tokens, given the
 *   lse that flce_forward (or flce_merge_shards) returned for the same H, W.
 *   With lse == NULL, out holds the logits themselves.  Per-token log-probs
 *   of the targets are -loss; this call scores any K tokens per position
 *   (sampled tokens, candidates) with one gathered dot product each, no new
 *   vocabulary sweep.
 *   H [T x d], W [V x d] in dtype; tokens [T x K] int64; out [T x K] float.
 *   Tokens outside [0, V) score NaN.  The dot product is fp32 (exact bf16
 *   products) summed in a fixed order, so it may differ from the forward's
 *   target logit by fp32 rounding.
 * FLCE_ERR_INVALID_ARG for an unknown dtype, negative sizes or NULL buffers
 * (T, K > 0), FLCE_ERR_UNSUPPORTED for d % 8 != 0, sizes beyond the plan's
 * limits or misaligned H/W.  T == 0 or K == 0 launches nothing. */
flce_status_t flce_token_logprobs(int64_t T, int64_t d, int64_t V, flce_dtype_t dtype,
                                  const void* H, const void* W, const int64_t* tokens, int64_t K,
                                  const float* lse, float* out, void* stream);

/* ---- kernel timing (a profiling aid; off by default) --------------------
 * While enabled, every kernel launch made by flce_forward / flce_backward on
 * the calling process is bracketed by two hipEvents recorded on the caller's
 * stream, and tagged with the algorithmic work of that launch.
 * flce_timing_collect() waits for the recorded events, adds each launch's
 * elapsed time to its kernel's entry, fills up to `max_entries` entries
 * (one per kernel name, in a fixed order) and clears the record.  The
 * registry is process-global and mutex-protected; it is the only shared
 * state of the library.  Events are created by the library the first time
 * they are needed and reused; no device memory is allocated. */
typedef struct flce_kernel_time {
  char name[24];     /* kernel name, e.g. "fwd_sweep" */
  int64_t launches;  /* launches recorded since the last collect */
  double total_ms;   /* summed event-to-event time of those launches */
  double flops;      /* algorithmic flops of those launches (2*M*N*K each) */
  double bytes;      /* algorithmic HBM bytes of those launches */
} flce_kernel_time_t;

/* Turns timing on (nonzero) or off (0).  Returns FLCE_OK. */
flce_status_t flce_timing_enable(int enable);

/* Collects and clears the record; *n_out receives the number of entries
 * written.  FLCE_ERR_INVALID_ARG for NULL pointers, FLCE_ERR_HIP when an
 * event query fails. */
flce_status_t flce_timing_collect(flce_kernel_time_t* out, int max_entries, int* n_out);

/* ---- workgroup timeline (a profiling aid of a separate build) ------------
 * Not part of the method; no passage of the pages defines it.  In the library
 * built with -DFLCE_TIMELINE=1 (libflce_timeline.so, compiled by the build
 * step beside libflce.so), every workgroup of the forward sweep, the dZ
 * recompute and the dH/dW launch appends one record: the compute unit it ran
 * on and two stamps of the GPU's constant 100 MHz real-time counter, taken
 * at its start and after its last store was issued.  The record holds up to
 * 524,288 workgroups; later ones are counted but dropped.  In libflce.so both
 * calls return FLCE_ERR_UNSUPPORTED and touch nothing. */
typedef struct {
  uint32_t hw_id;    /* the HW_ID register: CU_ID in bits 11:8, SH_ID bit 12, SE_ID 15:13 */
  uint32_t xcc_id;   /* the XCC_ID register: the XCD in bits 3:0 */
  uint64_t t_start;  /* real-time counter at the workgroup's start */
  uint64_t t_end;    /* ... after its last store was issued */
  uint32_t kernel;   /* 1 forward sweep, 2 dZ recompute, 3 dH and 4 dW workgroups of bwd_dhdw */
  uint32_t block;    /* the workgroup's index in its launch */
} flce_wg_record_t;

/* Clears the record (a synchronous copy to the device).  FLCE_ERR_HIP when
 * the copy fails. */
flce_status_t flce_timeline_reset(void);

/* Waits for the device, then copies up to max_records records in the order
 * the workgroups finished into out (host memory) and writes their number to
 * *n_out.  FLCE_ERR_INVALID_ARG for NULL pointers, FLCE_ERR_HIP when a copy
 * fails. */
flce_status_t flce_timeline_read(flce_wg_record_t* out, int max_records, int* n_out);

/* Static description of a status code. */
const char* flce_status_string(flce_status_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* flce_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* flce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
