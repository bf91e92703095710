// flce_launch.h -- internal interface between the host sequencing (flce_api.cpp)
// and the kernels (flce_kernels.hip).  Not part of the public C-ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace flce {

// Targets of the tokens, as seen by one vocab shard [start, start + V) of a
// vocabulary of `total` ids (start = 0 and total = V when unsharded).
struct Targets {
  const int64_t* y;
  int64_t ignore_index;
  int64_t start;
  int64_t total;
};

struct FwdArgs {
  const void* H;
  const void* W;
  Targets tg;
  int64_t T;
  int d, V;
  int n_ttiles, n_vtiles;
  int splits, tps, grp;
  float* part;  // [splits][T][2] running (max, sum)
  float* zt;    // [T] target logits
};

struct MergeArgs {
  const float* part;
  const float* zt;
  Targets tg;
  int64_t T;
  int V, splits;
  // unsharded: loss [T] and lse [T].  Shard statistics (shard != 0): lse of
  // the shard's vocab into `lse`, the target logit (or -inf when the target
  // is not in the shard or ignored) into `zt_out`; `loss` is unused.
  int shard;
  float* loss;
  float* lse;
  float* zt_out;
};

// Merge of per-shard statistics [n_shards][T] into loss and lse.
struct ShardMergeArgs {
  const float* lse_shards;
  const float* zt_shards;
  Targets tg;
  int64_t T;
  int n_shards;
  float* loss;
  float* lse;
};

// The backward works on the non-ignored tokens only: compacted in ascending
// order, idx[p] is the token at compacted position p (positions [*tv, T)
// hold the ignored tokens).  A token block is compacted positions
// [t_begin, t_begin + t_max); it holds block_count() tokens, which only the
// device knows.
struct TokBlock {
  const int* idx;
  const int* tv;
  int64_t t_begin;
  int t_max;
};

struct DzArgs {
  const void* Hc;  // the block's H rows, compacted: [t_max][d]
  const void* W;
  Targets tg;
  const float* lse;
  int d, V;
  TokBlock blk;
  int64_t v_begin;  // first vocab id of the slab
  int n_vtiles, n_ttiles;
  int64_t ldz;       // dZ row pitch (elements)
  int64_t ldz_cols;  // columns of each dZ row that this call writes
  float grad_scale;
  const float* g_dev;  // when set, the gradient scale is read from here instead
  void* dz;
};

struct DhArgs {
  const void* dz;
  const void* W;
  int64_t ldz;
  int d, V;
  TokBlock blk;
  int64_t v_begin;
  int k_count;  // vocab rows in the slab (K)
  int n_mtiles, n_ntiles;
  int mode;     // 0 first of several, 1 middle, 2 last of several, 3 only
  float* dh_acc;
  void* dH;
  // fp32 partial tiles of a K-split dH, dh_split_slots() tiles of dh_bm x
  // dh_bn; NULL: never split
  float* part;
};

struct DwArgs {
  const void* dz;
  const void* Ht;   // the block's H rows transposed, [d][ldht]
  int64_t ldht;
  int64_t ldz;
  int d;
  TokBlock blk;  // K = block_count()
  int64_t v_begin;
  int v_count;   // N
  int n_mtiles, n_ntiles;  // hidden tiles, vocab tiles
  int accumulate;
  float* dW;
  // When set, the last block holding any token (block 0 when none does) also
  // writes the bf16 copy of its finished dW tiles here ([V][d], round to
  // nearest even), so that the copy needs no pass of its own.
  void* dW_bf16;
};

// One workgroup of the profiling build's timeline (the layout of
// flce_wg_record_t in flce.h).
struct TimelineRecord {
  uint32_t hw_id, xcc_id;
  uint64_t t_start, t_end;
  uint32_t kernel, block;
};
constexpr uint32_t kTimelineFwdSweep = 1, kTimelineDz = 2, kTimelineDh = 3, kTimelineDw = 4;
// hipErrorNotSupported unless built with FLCE_TIMELINE=1
hipError_t timeline_reset();
hipError_t timeline_read(TimelineRecord* out, int max_records, int* n_out);

struct TileInfo {
  // logits: vocab x tokens; dH: tokens x hidden; dW: hidden x vocab
  int logit_bm, logit_bn, dh_bm, dh_bn, dw_bm, dw_bn;
  int dh_bk;  // k (vocab) per dH stage: the unit of its K split
};

TileInfo tile_info(bool bf16);
// The forward sweep.  capture: the target logit is taken from the tile's fp32
// accumulator into a.zt; otherwise the sweep is a pure log-sum-exp and
// launch_target_logit fills a.zt with gathered dot products.
hipError_t launch_fwd_sweep(const FwdArgs& a, bool bf16, bool capture, int grid, hipStream_t s);
hipError_t launch_target_logit(const FwdArgs& a, bool bf16, hipStream_t s);
hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t s);
// Reduced loss and the matching gradient scale (see loss_reduce_kernel).
struct ReduceArgs {
  const float* loss;
  const int64_t* y;  // read only for mean_valid
  int64_t ignore_index;
  int64_t T;
  float scale;
  int mean_valid;
  float* out;    // optional
  float* g_out;  // optional
};
hipError_t launch_loss_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_cast_bf16(const float* src, void* dst, int64_t n, hipStream_t s);
hipError_t launch_bwd_dz(const DzArgs& a, bool bf16, hipStream_t s);
// Sums a split dH's parts and applies the mode (nothing when unsplit); launch
// after launch_bwd_dhdw with the same dH arguments.
hipError_t launch_bwd_dh_reduce(const DhArgs& a, bool bf16, hipStream_t s);
int dh_split_slots();
// dH and dW of one block and slab as a single launch (dH workgroups first);
// launch_bwd_dh_reduce follows when dH splits.
hipError_t launch_bwd_dhdw(const DhArgs& h, const DwArgs& w, bool bf16, hipStream_t s);
// Scoring of given tokens: out[t * K + k] = H[t] . W[tokens[t * K + k]] - lse[t]
// (lse NULL: the logit itself).
struct TokenArgs {
  const void* H;
  const void* W;
  const int64_t* tokens;
  const float* lse;
  int64_t T;
  int d, V, K;
  float* out;
};

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_token_logit(const TokenArgs& a, bool bf16, hipStream_t s);
// Compaction of the non-ignored tokens: idx [T], *tv, with cnt [n] scratch
// (n = compact_chunks(T)).
int64_t compact_chunks(int64_t T);
hipError_t launch_compact(const int64_t* y, int64_t ignore_index, int64_t T, int* cnt, int* idx,
                          int* tv, hipStream_t s);
// dH rows of the ignored tokens (compacted positions [*tv, T)) set to zero.
hipError_t launch_zero_rows(void* dH, const int* idx, const int* tv, int64_t T, int d, bool bf16,
                            hipStream_t s);
// One token block of H gathered: Hc [t_max][d] rows and Ht [d][t_max], zero
// past the block's token count.
hipError_t launch_gather_block(const void* H, const TokBlock& blk, int d, void* Hc, void* Ht,
                               bool bf16, hipStream_t s);
hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t s);
// The library's static device workspace (allocation-free entry point): its
// size, and its device address on the current device (looked up once per
// device, then cached).
uint64_t scratch_bytes();
hipError_t scratch_address(void** out);

}  // namespace flce
