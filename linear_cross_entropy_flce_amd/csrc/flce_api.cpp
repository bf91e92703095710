// flce_api.cpp -- the C-ABI: planning, argument validation and launch order.
//
// Host-only code.  Nothing here allocates device memory or synchronises; every
// launch goes to the caller's stream in a fixed order, so results are
// reproducible bit for bit.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/flce.h"
#include "flce_launch.h"

namespace {

constexpr uint32_t kPlanMagic = 0x464c4345u;  // "FLCE"
constexpr uint64_t kDefaultCap = 950000000ull;
constexpr uint64_t kMaxCap = 0x7fff0000ull;
constexpr int64_t kMaxBlock = 8192;
constexpr int kTargetWorkgroups = 256;  // one per compute unit
constexpr int64_t kComputeUnits = 256;  // MI355X
// Forward: at least this many vocab splits.  An XCD runs 32 workgroups at a
// time, taken as 32 / splits token tiles x splits; 4 x 8 re-reads W half as
// often as 8 x 4 and measured ~1% faster on the 65,536 x 124,160 sweep.
#ifndef FLCE_FWD_MIN_SPLITS
#define FLCE_FWD_MIN_SPLITS 4
#endif
// device scalars of flce_forward_backward (the gradient scale), after the
// larger of the forward and backward workspaces
constexpr uint64_t kScalarBytes = 256;

thread_local char g_err[512] = "";
// set while an allocation-free call runs: its launches are not timed (timing
// would create hipEvents)
thread_local bool g_untimed = false;

flce_status_t fail(flce_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

flce_status_t ok() {
  g_err[0] = 0;
  return FLCE_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

flce_status_t check_plan(const flce_plan_t* p) {
  if (!p) return fail(FLCE_ERR_INVALID_ARG, "plan is NULL");
  if (p->magic != kPlanMagic) return fail(FLCE_ERR_INVALID_ARG, "plan was not made by flce_plan");
  return FLCE_OK;
}

flce_status_t hip_fail(hipError_t e, const char* what) {
  return fail(FLCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------ kernel timing
enum KernelId {
  K_FWD_SWEEP, K_FWD_MERGE, K_LOSS_SUM, K_BWD_DZ, K_BWD_DHDW, K_DH_REDUCE, K_FILL,
  K_SHARD_MERGE, K_TOKEN_LOGIT, K_CAST, K_TRANSPOSE, K_COMPACT, K_TARGET_LOGIT, K_COUNT
};
const char* const kKernelNames[K_COUNT] = {
    "fwd_sweep", "fwd_merge",   "loss_sum",    "bwd_dz",    "bwd_dhdw", "dh_reduce",
    "fill_zero", "shard_merge", "token_logit", "cast_bf16", "gather_h", "compact",
    "target_logit"};

struct TimingRec {
  int kid;
  double flops, bytes;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> pool;
};

Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t pooled_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence at record (no cache writeback and
  // invalidate between the launches being timed)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is enabled.
class Timed {
 public:
  Timed(hipStream_t s, KernelId kid, double flops, double bytes) : s_(s) {
    if (g_untimed) return;
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.enabled) return;
    rec_.kid = kid;
    rec_.flops = flops;
    rec_.bytes = bytes;
    rec_.start = pooled_event(t);
    rec_.stop = pooled_event(t);
    if (rec_.start && rec_.stop && hipEventRecord(rec_.start, s_) == hipSuccess) on_ = true;
  }
  void done() {
    if (!on_) return;
    on_ = false;
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (hipEventRecord(rec_.stop, s_) == hipSuccess) t.recs.push_back(rec_);
  }
  ~Timed() { done(); }

 private:
  hipStream_t s_;
  bool on_ = false;
  TimingRec rec_{};
};

// Modelled time of the backward pass for token block B and vocab slab Vs, in
// units of one 256 x 256 x 256 MFMA block per compute unit.  Every launch
// runs whole rounds of kComputeUnits workgroups, so a grid of n tiles costs
// ceil(n / CU) rounds; the recompute tile also pays its exp/store epilogue,
// the dW tile its fp32 read-modify-write, and each slab a dH accumulator pass.
// With dh_split, a block of at most half a round of dH tiles runs its K loop
// in S parts (the kernels' rule), one round of 1/S of the tile.
double backward_cost(int64_t T, int64_t d, int64_t V, int64_t B, int64_t Vs,
                     const flce::TileInfo& ti, bool dh_split) {
  const double unit = 256.0 * 256.0 * 256.0;
  const int64_t n_dt_h = cdiv(d, ti.dh_bn), n_dt_w = cdiv(d, ti.dw_bm);
  // one (block, slab) launch pair of tc tokens and vc vocab rows
  auto pair = [&](int64_t tc, int64_t vc, bool first_block) {
    const int64_t dz_tiles = cdiv(vc, ti.logit_bm) * cdiv(tc, ti.logit_bn);
    const int64_t dh_tiles = cdiv(tc, ti.dh_bm) * n_dt_h;
    const int64_t dw_tiles = cdiv(vc, ti.dw_bn) * n_dt_w;
    const double dz_tile = (double)ti.logit_bm * ti.logit_bn * d / unit;
    const double dh_tile = (double)ti.dh_bm * ti.dh_bn * vc / unit;
    const double dw_tile = (double)ti.dw_bm * ti.dw_bn * tc / unit;
    double c = cdiv(dz_tiles, kComputeUnits) * dz_tile * 1.10;
    const int64_t dh_parts =
        dh_split && 2 * dh_tiles <= kComputeUnits
            ? std::min<int64_t>(kComputeUnits / dh_tiles, cdiv(vc, ti.dh_bk))
            : 1;
    c += cdiv(dh_tiles, kComputeUnits) * (dh_tile / dh_parts + 0.5);
    c += cdiv(dw_tiles, kComputeUnits) * dw_tile * (first_block ? 1.035 : 1.07);
    return c;
  };
  // a block sweeps full slabs and one possibly shorter last slab
  const int64_t n_full_s = V / Vs, last_s = V - n_full_s * Vs;
  auto block = [&](int64_t tc, bool first_block) {
    double c = (double)n_full_s * pair(tc, Vs, first_block);
    if (last_s > 0) c += pair(tc, last_s, first_block);
    return c;
  };
  // blocks: the first, the other full ones, and a shorter last one; the sum
  // is the same as walking them one by one, in O(1)
  const int64_t n_full_b = T / B, last_b = T - n_full_b * B;
  double cost = 0;
  if (n_full_b > 0) cost += block(B, true) + (double)(n_full_b - 1) * block(B, false);
  if (last_b > 0) cost += block(last_b, n_full_b == 0);
  return cost;
}

}  // namespace

namespace {

// Backward workspace after the dZ buffer and the dH accumulator: the token
// block's H gathered in the compacted order, transposed (Ht, the dW
// contraction's K-contiguous operand) and as rows (Hc, the recompute's), then
// the compacted token order (idx [T]), the per-chunk counts of the
// compaction and the count of non-ignored tokens.
struct BwdTail {
  uint64_t ht, hc, idx, cnt, tv, bytes;  // offsets from the end of dh_acc
};
BwdTail bwd_tail(int64_t T, int64_t B, int64_t d, int64_t esz) {
  BwdTail t;
  t.ht = 0;
  t.hc = (uint64_t)(B * d * esz);
  t.idx = 2 * t.hc;
  t.cnt = t.idx + (uint64_t)round_up(T * 4, 256);
  t.tv = t.cnt + (uint64_t)round_up(flce::compact_chunks(T) * 4, 256);
  t.bytes = t.tv + 256;
  return t;
}

hipError_t launch_loss_sum(const float* loss, int64_t T, float scale, float* out, hipStream_t s) {
  flce::ReduceArgs r{loss, nullptr, 0, T, scale, 0, out, nullptr};
  return flce::launch_loss_reduce(r, s);
}

flce_status_t check_shard(const flce_plan_t& p, int64_t vocab_start, int64_t vocab_total) {
  if (vocab_total < 1 || vocab_total >= ((int64_t)1 << 31))
    return fail(FLCE_ERR_INVALID_ARG, "vocab_total = %lld out of range", (long long)vocab_total);
  if (vocab_start < 0 || vocab_start > vocab_total - p.V)
    return fail(FLCE_ERR_INVALID_ARG, "shard [%lld, %lld) is not inside [0, %lld)",
                (long long)vocab_start, (long long)(vocab_start + p.V), (long long)vocab_total);
  return ok();
}

// The forward for one vocab shard (the whole vocabulary when tg.start = 0
// and tg.total = V).  shard: write the shard statistics (lse of the shard,
// target logit or -inf) into lse and zt_out instead of loss and lse.
flce_status_t forward_impl(const flce_plan_t* plan, const void* H, const void* W,
                           const flce::Targets& tg, float scale, float* loss, float* lse,
                           float* loss_reduced, float* zt_out, bool shard, void* ws,
                           uint64_t ws_bytes, void* stream) {
  flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  const flce_plan_t& p = *plan;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!W) return fail(FLCE_ERR_INVALID_ARG, "W is NULL");
  if (p.T > 0 && (!H || !tg.y || !lse || !ws || (shard ? !zt_out : !loss)))
    return fail(FLCE_ERR_INVALID_ARG, shard ? "H, y, lse_shard, zt_shard and ws must be non-NULL when T > 0"
                                            : "H, y, loss, lse and ws must be non-NULL when T > 0");
  if (misaligned(H) || misaligned(W) || misaligned(ws))
    return fail(FLCE_ERR_UNSUPPORTED, "H, W and ws must be 16-byte aligned");
  if (p.T > 0 && ws_bytes < p.fwd_ws_bytes)
    return fail(FLCE_ERR_WORKSPACE, "forward needs %llu workspace bytes, got %llu",
                (unsigned long long)p.fwd_ws_bytes, (unsigned long long)ws_bytes);
  if (p.target_logit != FLCE_TARGET_IN_TILE && p.target_logit != FLCE_TARGET_GATHER)
    return fail(FLCE_ERR_INVALID_ARG, "unknown target_logit mode %u", (unsigned)p.target_logit);
  const bool bf16 = p.dtype == FLCE_BF16;
  const bool capture = p.target_logit == FLCE_TARGET_IN_TILE;
  hipError_t e;
  if (p.T == 0) {
    if (loss_reduced) {
      Timed tm(s, K_LOSS_SUM, 0, 4);
      e = launch_loss_sum(loss, 0, scale, loss_reduced, s);
      tm.done();
      if (e != hipSuccess) return hip_fail(e, "loss_sum launch");
    }
    return ok();
  }
  float* part = reinterpret_cast<float*>(ws);
  float* zt = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                       round_up((int64_t)p.fwd_splits * p.T * 2 * 4, 256));
  flce::FwdArgs a;
  a.H = H;
  a.W = W;
  a.tg = tg;
  a.T = p.T;
  a.d = (int)p.d;
  a.V = (int)p.V;
  a.n_ttiles = (int)cdiv(p.T, p.tile_t);
  a.n_vtiles = (int)cdiv(p.V, p.tile_v);
  a.splits = p.fwd_splits;
  a.tps = p.fwd_tiles_per_split;
  a.grp = p.fwd_splits >= 32 ? 1 : 32 / p.fwd_splits;
  a.part = part;
  a.zt = zt;
  const int64_t per_group = (int64_t)a.grp * a.splits;
  const int64_t groups = cdiv(a.n_ttiles, a.grp);
  const int64_t grid = 8 * per_group * cdiv(groups, 8);
  const double esz = (double)p.elem_bytes;
  Timed t_sweep(s, K_FWD_SWEEP, 2.0 * p.T * p.d * p.V,
                (p.T + p.V) * p.d * esz + (double)p.fwd_splits * p.T * 8 + p.T * 12.0);
  e = flce::launch_fwd_sweep(a, bf16, capture, (int)grid, s);
  t_sweep.done();
  if (e != hipSuccess) return hip_fail(e, "forward sweep launch");
  if (!capture) {
    // the target logits as gathered dot products (H row + W row per token)
    Timed tm(s, K_TARGET_LOGIT, 0, 2.0 * p.T * p.d * esz + p.T * 12.0);
    e = flce::launch_target_logit(a, bf16, s);
    tm.done();
    if (e != hipSuccess) return hip_fail(e, "target logit launch");
  }
  flce::MergeArgs m;
  m.part = part;
  m.zt = zt;
  m.tg = tg;
  m.T = p.T;
  m.V = (int)p.V;
  m.splits = p.fwd_splits;
  m.shard = shard ? 1 : 0;
  m.loss = loss;
  m.lse = lse;
  m.zt_out = zt_out;
  Timed t_merge(s, K_FWD_MERGE, 0, (double)p.fwd_splits * p.T * 8 + p.T * 20.0);
  e = flce::launch_fwd_merge(m, s);
  t_merge.done();
  if (e != hipSuccess) return hip_fail(e, "forward merge launch");
  if (loss_reduced) {
    Timed tm(s, K_LOSS_SUM, 0, p.T * 4.0 + 4);
    e = launch_loss_sum(loss, p.T, scale, loss_reduced, s);
    tm.done();
    if (e != hipSuccess) return hip_fail(e, "loss_sum launch");
  }
  return ok();
}

// The backward for one vocab shard (the whole vocabulary when tg.start = 0
// and tg.total = V); lse is over the whole vocabulary.
flce_status_t backward_impl(const flce_plan_t* plan, const void* H, const void* W,
                            const flce::Targets& tg, const float* lse, float grad_scale,
                            const float* g_dev, void* dH, float* dW, int accumulate_dW,
                            void* dW_bf16, void* ws, uint64_t ws_bytes, void* stream) {
  flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  const flce_plan_t& p = *plan;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!W || !dW) return fail(FLCE_ERR_INVALID_ARG, "W and dW must be non-NULL");
  if (p.T > 0 && (!H || !tg.y || !lse || !dH || !ws))
    return fail(FLCE_ERR_INVALID_ARG, "H, y, lse, dH and ws must be non-NULL when T > 0");
  if (misaligned(H) || misaligned(W) || misaligned(dH) || misaligned(dW) || misaligned(ws))
    return fail(FLCE_ERR_UNSUPPORTED, "H, W, dH, dW and ws must be 16-byte aligned");
  if (p.T > 0 && ws_bytes < p.bwd_ws_bytes)
    return fail(FLCE_ERR_WORKSPACE, "backward needs %llu workspace bytes, got %llu",
                (unsigned long long)p.bwd_ws_bytes, (unsigned long long)ws_bytes);
  const bool bf16 = p.dtype == FLCE_BF16;
  const flce::TileInfo ti = flce::tile_info(bf16);
  hipError_t e;
  if (p.T == 0) {
    if (!accumulate_dW) {
      Timed tm(s, K_FILL, 0, p.V * p.d * 4.0);
      e = flce::launch_fill_zero(dW, p.V * p.d, s);
      tm.done();
      if (e != hipSuccess) return hip_fail(e, "dW fill launch");
    }
    if (dW_bf16) {
      // no dW tile runs: the copy takes a pass of its own
      Timed tm(s, K_CAST, 0, p.V * p.d * 6.0);
      e = flce::launch_cast_bf16(dW, dW_bf16, p.V * p.d, s);
      tm.done();
      if (e != hipSuccess) return hip_fail(e, "dW cast launch");
    }
    return ok();
  }
  void* dz = ws;
  float* dh_acc = p.dh_acc_bytes ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                                            p.dz_ws_bytes)
                                 : nullptr;
  char* tail = reinterpret_cast<char*>(ws) + p.dz_ws_bytes + p.dh_acc_bytes;
  const BwdTail tl = bwd_tail(p.T, p.bwd_block, p.d, p.elem_bytes);
  void* ht = tail + tl.ht;
  void* hc = tail + tl.hc;
  int* idx = reinterpret_cast<int*>(tail + tl.idx);
  int* tv = reinterpret_cast<int*>(tail + tl.tv);
  float* dh_part = p.dh_split_bytes ? reinterpret_cast<float*>(tail + tl.bytes) : nullptr;
  {
    // the non-ignored tokens in ascending order; dH rows of the others are 0
    Timed tm(s, K_COMPACT, 0, p.T * 8.0 * 2 + p.T * 8.0);
    e = flce::launch_compact(tg.y, tg.ignore_index, p.T, reinterpret_cast<int*>(tail + tl.cnt),
                             idx, tv, s);
    if (e == hipSuccess) e = flce::launch_zero_rows(dH, idx, tv, p.T, (int)p.d, bf16, s);
    tm.done();
    if (e != hipSuccess) return hip_fail(e, "token compaction launch");
  }
  for (int64_t b = 0; b < p.n_blocks; ++b) {
    const int64_t t_begin = b * p.bwd_block;
    // at most this many tokens (the device knows how many are not ignored)
    const int t_count = (int)(p.T - t_begin < p.bwd_block ? p.T - t_begin : p.bwd_block);
    const flce::TokBlock blk{idx, tv, t_begin, (int)p.bwd_block};
    {
      Timed tm(s, K_TRANSPOSE, 0, 3.0 * p.bwd_block * p.d * p.elem_bytes);
      e = flce::launch_gather_block(H, blk, (int)p.d, hc, ht, bf16, s);
      tm.done();
      if (e != hipSuccess) return hip_fail(e, "H gather launch");
    }
    for (int64_t sl = 0; sl < p.n_slabs; ++sl) {
      const int64_t v_begin = sl * p.bwd_slab;
      const int v_count = (int)(p.V - v_begin < p.bwd_slab ? p.V - v_begin : p.bwd_slab);

      flce::DzArgs z;
      z.Hc = hc;
      z.W = W;
      z.tg = tg;
      z.lse = lse;
      z.d = (int)p.d;
      z.V = (int)p.V;
      z.blk = blk;
      z.v_begin = v_begin;
      z.n_vtiles = (int)cdiv(v_count, ti.logit_bm);
      z.n_ttiles = (int)cdiv(t_count, ti.logit_bn);
      z.ldz = p.bwd_slab;
      z.ldz_cols = (int64_t)z.n_vtiles * ti.logit_bm;
      z.grad_scale = grad_scale;
      z.g_dev = g_dev;
      z.dz = dz;
      const double esz = (double)p.elem_bytes;
      const double tc = t_count, vc = v_count, dd = (double)p.d;
      Timed t_dz(s, K_BWD_DZ, 2.0 * tc * dd * vc, (tc + vc) * dd * esz + tc * 12 + tc * vc * esz);
      e = flce::launch_bwd_dz(z, bf16, s);
      t_dz.done();
      if (e != hipSuccess) return hip_fail(e, "dZ launch");

      flce::DhArgs h;
      h.dz = dz;
      h.W = W;
      h.ldz = p.bwd_slab;
      h.d = (int)p.d;
      h.V = (int)p.V;
      h.blk = blk;
      h.v_begin = v_begin;
      h.k_count = v_count;
      h.n_mtiles = (int)cdiv(t_count, ti.dh_bm);
      h.n_ntiles = (int)cdiv(p.d, ti.dh_bn);
      if (p.n_slabs == 1) h.mode = 3;
      else if (sl == 0) h.mode = 0;
      else if (sl + 1 < p.n_slabs) h.mode = 1;
      else h.mode = 2;
      h.dh_acc = dh_acc;
      h.dH = dH;
      h.part = dh_part;
      flce::DwArgs w;
      w.dz = dz;
      w.Ht = ht;
      w.ldht = p.bwd_block;
      w.ldz = p.bwd_slab;
      w.d = (int)p.d;
      w.blk = blk;
      w.v_begin = v_begin;
      w.v_count = v_count;
      w.n_mtiles = (int)cdiv(p.d, ti.dw_bm);
      w.n_ntiles = (int)cdiv(v_count, ti.dw_bn);
      w.accumulate = (b > 0 || accumulate_dW) ? 1 : 0;
      w.dW = dW;
      w.dW_bf16 = dW_bf16;
      // dH and dW in one launch (both only read this slab's dZ)
      Timed t_hw(s, K_BWD_DHDW, 4.0 * tc * dd * vc,
                 2.0 * tc * vc * esz + vc * dd * esz +
                     tc * dd * (h.mode == 1 || h.mode == 2 ? 4.0 : 0.0) +
                     tc * dd * (h.mode >= 2 ? esz : 4.0) + tc * dd * esz +
                     vc * dd * (w.accumulate ? 8.0 : 4.0));
      e = flce::launch_bwd_dhdw(h, w, bf16, s);
      t_hw.done();
      if (e != hipSuccess) return hip_fail(e, "dH/dW launch");
      if (dh_part) {
        // sums the parts when the device split dH's K loop (reads them all
        // once, then the mode's accumulator and dH traffic)
        Timed t_red(s, K_DH_REDUCE, 0, tc * dd * 4.0 * 2);
        e = flce::launch_bwd_dh_reduce(h, bf16, s);
        t_red.done();
        if (e != hipSuccess) return hip_fail(e, "dH reduce launch");
      }
    }
  }
  return ok();
}

}  // namespace

extern "C" {

flce_status_t flce_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.enabled = enable != 0;
  return ok();
}

flce_status_t flce_timing_collect(flce_kernel_time_t* out, int max_entries, int* n_out) {
  if (!out || !n_out) return fail(FLCE_ERR_INVALID_ARG, "out and n_out must be non-NULL");
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  flce_kernel_time_t acc[K_COUNT];
  memset(acc, 0, sizeof acc);
  flce_status_t st = FLCE_OK;
  for (const TimingRec& r : t.recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && st == FLCE_OK) st = hip_fail(e, "timing event");
    acc[r.kid].launches += 1;
    acc[r.kid].total_ms += ms;
    acc[r.kid].flops += r.flops;
    acc[r.kid].bytes += r.bytes;
    t.pool.push_back(r.start);
    t.pool.push_back(r.stop);
  }
  t.recs.clear();
  int n = 0;
  for (int k = 0; k < K_COUNT && n < max_entries; ++k) {
    if (acc[k].launches == 0) continue;
    out[n] = acc[k];
    snprintf(out[n].name, sizeof out[n].name, "%s", kKernelNames[k]);
    ++n;
  }
  *n_out = n;
  return st == FLCE_OK ? ok() : st;
}


flce_status_t flce_timeline_reset(void) {
  const hipError_t e = flce::timeline_reset();
  if (e == hipErrorNotSupported)
    return fail(FLCE_ERR_UNSUPPORTED, "this library was built without the workgroup timeline");
  if (e != hipSuccess) return hip_fail(e, "timeline reset");
  return ok();
}

flce_status_t flce_timeline_read(flce_wg_record_t* out, int max_records, int* n_out) {
  if (!out || !n_out) return fail(FLCE_ERR_INVALID_ARG, "out and n_out must be non-NULL");
  static_assert(sizeof(flce_wg_record_t) == sizeof(flce::TimelineRecord) &&
                    offsetof(flce_wg_record_t, t_start) == offsetof(flce::TimelineRecord, t_start) &&
                    offsetof(flce_wg_record_t, kernel) == offsetof(flce::TimelineRecord, kernel),
                "one record layout");
  const hipError_t e =
      flce::timeline_read(reinterpret_cast<flce::TimelineRecord*>(out), max_records, n_out);
  if (e == hipErrorNotSupported)
    return fail(FLCE_ERR_UNSUPPORTED, "this library was built without the workgroup timeline");
  if (e != hipSuccess) return hip_fail(e, "timeline read");
  return ok();
}

const char* flce_version(void) { return "0.1.0"; }

const char* flce_last_error(void) { return g_err; }

const char* flce_status_string(flce_status_t s) {
  switch (s) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARG: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case FLCE_ERR_WORKSPACE: return "workspace too small";
    case FLCE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

flce_status_t flce_plan(int64_t T, int64_t d, int64_t V, flce_dtype_t dtype, uint64_t cap,
                        flce_plan_t* out) {
  if (!out) return fail(FLCE_ERR_INVALID_ARG, "out is NULL");
  if (dtype != FLCE_F32 && dtype != FLCE_BF16)
    return fail(FLCE_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (T < 0) return fail(FLCE_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
  if (d <= 0) return fail(FLCE_ERR_INVALID_ARG, "d = %lld <= 0", (long long)d);
  if (V <= 0) return fail(FLCE_ERR_INVALID_ARG, "V = %lld <= 0", (long long)V);
  if (d % 8 != 0) return fail(FLCE_ERR_UNSUPPORTED, "d = %lld is not a multiple of 8", (long long)d);
  if (d > 65536) return fail(FLCE_ERR_UNSUPPORTED, "d = %lld > 65536", (long long)d);
  if (T >= (1ll << 31) || V >= (1ll << 31))
    return fail(FLCE_ERR_UNSUPPORTED, "T and V must be below 2^31");

  const bool bf16 = dtype == FLCE_BF16;
  const int64_t esz = bf16 ? 2 : 4;
  const flce::TileInfo ti = flce::tile_info(bf16);
  // The kernels address their operands through buffer resources with 32-bit
  // byte offsets, each based at the first row of the tile (or, for dH's W
  // operand, of the vocab slab) it reads, so H and W may exceed 2 GiB; a
  // slab's W rows must stay below 2^31 bytes.
  const int64_t slab_rows_max = ((1ll << 31) - 1) / (d * esz) / ti.logit_bm * ti.logit_bm;
  if (slab_rows_max < ti.logit_bm)
    return fail(FLCE_ERR_UNSUPPORTED, "d = %lld is too large for a %d-row vocab tile",
                (long long)d, ti.logit_bm);
  if (cap == 0) cap = kDefaultCap;
  // tile offsets into the workspace are 32-bit: keep it below 2 GiB
  if (cap > kMaxCap) cap = kMaxCap;

  flce_plan_t p;
  memset(&p, 0, sizeof p);
  p.T = T;
  p.d = d;
  p.V = V;
  p.dtype = (int32_t)dtype;
  p.elem_bytes = (int32_t)esz;
  p.tile_v = ti.logit_bm;
  p.tile_t = ti.logit_bn;

  // ---- forward: split the vocab tiles so that there are at least
  // kTargetWorkgroups workgroups, and at least FLCE_FWD_MIN_SPLITS splits.
  const int64_t n_tt = cdiv(T, ti.logit_bn);
  const int64_t n_vt = cdiv(V, ti.logit_bm);
  int64_t splits = cdiv(kTargetWorkgroups, n_tt > 0 ? n_tt : 1);
  if (splits < FLCE_FWD_MIN_SPLITS) splits = FLCE_FWD_MIN_SPLITS;
  if (splits > n_vt) splits = n_vt;
  const int64_t tps = cdiv(n_vt, splits);
  splits = cdiv(n_vt, tps);
  p.fwd_splits = (int32_t)splits;
  p.fwd_tiles_per_split = (int32_t)tps;
  p.fwd_ws_bytes = (uint64_t)round_up(splits * T * 2 * 4, 256) + (uint64_t)round_up(T * 4, 256);

  // ---- backward: the largest token block B (<= 8192, tile multiple) for
  // which some vocab slab fits under the cap, then the slab width that
  // minimises the modelled time (backward_cost): a dZ buffer of B x Vs plus
  // the fp32 dH accumulator when the vocab needs several slabs.
  //
  // dH's tile grid is (B / dh_bm) x (d / dh_bn).  When a full block has at
  // most half as many tiles as the GPU has compute units, dH will split its
  // K loop, so the partial tiles it needs are part of `need` in a first
  // search; a second search without them serves caps too small for both.
  const int64_t Tr = round_up(T > 0 ? T : 1, ti.logit_bn);
  const int64_t Vfull = round_up(V, ti.logit_bm);
  const int64_t dh_nt = cdiv(d, ti.dh_bn);
  const uint64_t split = (uint64_t)flce::dh_split_slots() * ti.dh_bm * ti.dh_bn * 4;
  int64_t best_B = 0, best_Vs = 0, best_slabs = 0;
  uint64_t best_split = 0;
  for (int pass = 0; pass < 2 && best_B == 0; ++pass) {
    for (int64_t B = (Tr < kMaxBlock ? Tr : kMaxBlock); B >= ti.logit_bn && best_B == 0;
         B -= ti.logit_bn) {
      const uint64_t reserve =
          pass == 0 && 2 * cdiv(B, ti.dh_bm) * dh_nt <= flce::dh_split_slots() ? split : 0;
      double best_cost = 0;
      for (int64_t Vs = ti.logit_bm; Vs <= Vfull && Vs <= slab_rows_max; Vs += ti.logit_bm) {
        const int64_t slabs = cdiv(V, Vs);
        const uint64_t need = (uint64_t)(B * Vs * esz) +
                              (slabs > 1 ? (uint64_t)(B * d * 4) : 0) +
                              bwd_tail(T, B, d, esz).bytes + reserve;
        if (need > cap) break;  // need grows with Vs
        const double c = backward_cost(T > 0 ? T : 1, d, V, B, Vs, ti, reserve > 0);
        if (best_B == 0 || c < best_cost * (1 - 1e-9)) {
          best_cost = c;
          best_B = B;
          best_Vs = Vs;
          best_slabs = slabs;
          best_split = reserve;
        }
      }
    }
  }
  if (best_B == 0)
    return fail(FLCE_ERR_WORKSPACE,
                "cap of %llu bytes cannot hold the smallest %d-token block x %d-vocab slab",
                (unsigned long long)cap, ti.logit_bn, ti.logit_bm);
  p.bwd_block = best_B;
  p.bwd_slab = best_Vs;
  p.n_blocks = T > 0 ? cdiv(T, best_B) : 0;
  p.n_slabs = best_slabs;
  p.dz_ws_bytes = (uint64_t)(best_B * best_Vs * esz);
  p.dh_acc_bytes = best_slabs > 1 ? (uint64_t)(best_B * d * 4) : 0;
  const uint64_t bwd_base = p.dz_ws_bytes + p.dh_acc_bytes + bwd_tail(T, best_B, d, esz).bytes;
  // Without a planned split, the partial tiles still help blocks that
  // ignored tokens thin out; they are kept where they fit beside the chosen
  // block and slab.
  p.dh_split_bytes = best_split ? best_split : (bwd_base + split <= cap ? split : 0);
  p.bwd_ws_bytes = bwd_base + p.dh_split_bytes;
  p.ws_bytes = (p.fwd_ws_bytes > p.bwd_ws_bytes ? p.fwd_ws_bytes : p.bwd_ws_bytes) + kScalarBytes;
  p.vocab_ws_cap = cap;
  p.naive_logits_bytes = (uint64_t)T * (uint64_t)V * (uint64_t)esz;
  p.magic = kPlanMagic;
  *out = p;
  return ok();
}

flce_status_t flce_forward(const flce_plan_t* plan, const void* H, const void* W, const int64_t* y,
                           int64_t ignore_index, float scale, float* loss, float* lse,
                           float* loss_reduced, void* ws, uint64_t ws_bytes, void* stream) {
  const flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  const flce::Targets tg{y, ignore_index, 0, plan->V};
  return forward_impl(plan, H, W, tg, scale, loss, lse, loss_reduced, nullptr, false, ws, ws_bytes,
                      stream);
}

flce_status_t flce_backward(const flce_plan_t* plan, const void* H, const void* W, const int64_t* y,
                            const float* lse, int64_t ignore_index, float grad_scale, void* dH,
                            float* dW, int accumulate_dW, void* ws, uint64_t ws_bytes,
                            void* stream) {
  const flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  const flce::Targets tg{y, ignore_index, 0, plan->V};
  return backward_impl(plan, H, W, tg, lse, grad_scale, nullptr, dH, dW, accumulate_dW, nullptr,
                       ws, ws_bytes, stream);
}

flce_status_t flce_forward_backward(const flce_plan_t* plan, const void* H, const void* W,
                                    const int64_t* y, int64_t ignore_index,
                                    flce_reduction_t reduction, float scale, float* loss,
                                    float* lse, float* loss_reduced, void* dH, float* dW,
                                    int accumulate_dW, void* dW_bf16, void* ws, uint64_t ws_bytes,
                                    void* stream) {
  flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  const flce_plan_t& p = *plan;
  if (reduction != FLCE_REDUCE_SUM && reduction != FLCE_REDUCE_MEAN_VALID)
    return fail(FLCE_ERR_INVALID_ARG, "unknown reduction %d", (int)reduction);
  if (!W || !dW) return fail(FLCE_ERR_INVALID_ARG, "W and dW must be non-NULL");
  if (p.T > 0 && (!H || !y || !loss || !lse || !dH || !ws))
    return fail(FLCE_ERR_INVALID_ARG, "H, y, loss, lse, dH and ws must be non-NULL when T > 0");
  if (misaligned(H) || misaligned(W) || misaligned(dH) || misaligned(dW) || misaligned(ws) ||
      misaligned(dW_bf16))
    return fail(FLCE_ERR_UNSUPPORTED, "H, W, dH, dW, dW_bf16 and ws must be 16-byte aligned");
  if (p.T > 0 && ws_bytes < p.ws_bytes)
    return fail(FLCE_ERR_WORKSPACE, "forward_backward needs %llu workspace bytes, got %llu",
                (unsigned long long)p.ws_bytes, (unsigned long long)ws_bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const flce::Targets tg{y, ignore_index, 0, p.V};
  float* g_dev = nullptr;
  if (p.T > 0) {
    st = forward_impl(plan, H, W, tg, scale, loss, lse, nullptr, nullptr, false, ws, ws_bytes,
                      stream);
    if (st != FLCE_OK) return st;
    g_dev = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (p.ws_bytes - kScalarBytes));
    flce::ReduceArgs r{loss, y, ignore_index, p.T, scale,
                       reduction == FLCE_REDUCE_MEAN_VALID ? 1 : 0, loss_reduced, g_dev};
    Timed tm(s, K_LOSS_SUM, 0, p.T * (reduction == FLCE_REDUCE_MEAN_VALID ? 12.0 : 4.0) + 8);
    e = flce::launch_loss_reduce(r, s);
    tm.done();
    if (e != hipSuccess) return hip_fail(e, "loss reduce launch");
  } else if (loss_reduced) {
    e = launch_loss_sum(loss, 0, scale, loss_reduced, s);
    if (e != hipSuccess) return hip_fail(e, "loss_sum launch");
  }
  // the last block with tokens writes the bf16 copy of dW from its dW tiles
  return backward_impl(plan, H, W, tg, lse, scale, g_dev, dH, dW, accumulate_dW, dW_bf16, ws,
                       ws_bytes, stream);
}

flce_status_t flce_forward_backward_scratch(const flce_plan_t* plan, const void* H,
                                            const void* W, const int64_t* y, int64_t ignore_index,
                                            flce_reduction_t reduction, float scale, float* loss,
                                            float* lse, float* loss_reduced, void* dH, float* dW,
                                            int accumulate_dW, void* dW_bf16, void* stream) {
  flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  const uint64_t cap = flce::scratch_bytes();
  if (plan->ws_bytes > cap)
    return fail(FLCE_ERR_WORKSPACE,
                "the plan needs %llu workspace bytes; the scratch array holds %llu (plan with "
                "vocab_ws_cap_bytes <= %llu)",
                (unsigned long long)plan->ws_bytes, (unsigned long long)cap,
                (unsigned long long)(cap - kScalarBytes));
  void* ws = nullptr;
  const hipError_t e = flce::scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "scratch array address");
  g_untimed = true;
  st = flce_forward_backward(plan, H, W, y, ignore_index, reduction, scale, loss, lse,
                             loss_reduced, dH, dW, accumulate_dW, dW_bf16, ws, cap, stream);
  g_untimed = false;
  return st;
}

flce_status_t flce_forward_shard(const flce_plan_t* plan, const void* H, const void* W_shard,
                                 const int64_t* y, int64_t ignore_index, int64_t vocab_start,
                                 int64_t vocab_total, float* lse_shard, float* zt_shard, void* ws,
                                 uint64_t ws_bytes, void* stream) {
  flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  st = check_shard(*plan, vocab_start, vocab_total);
  if (st != FLCE_OK) return st;
  const flce::Targets tg{y, ignore_index, vocab_start, vocab_total};
  return forward_impl(plan, H, W_shard, tg, 1.f, nullptr, lse_shard, nullptr, zt_shard, true, ws,
                      ws_bytes, stream);
}

flce_status_t flce_merge_shards(int64_t T, int32_t n_shards, const float* lse_shards,
                                const float* zt_shards, const int64_t* y, int64_t ignore_index,
                                int64_t vocab_total, float scale, float* loss, float* lse,
                                float* loss_reduced, void* stream) {
  if (T < 0 || T >= ((int64_t)1 << 31)) return fail(FLCE_ERR_INVALID_ARG, "T = %lld out of range", (long long)T);
  if (n_shards < 1) return fail(FLCE_ERR_INVALID_ARG, "n_shards = %d must be >= 1", (int)n_shards);
  if (vocab_total < 1 || vocab_total >= ((int64_t)1 << 31))
    return fail(FLCE_ERR_INVALID_ARG, "vocab_total = %lld out of range", (long long)vocab_total);
  if ((int64_t)n_shards > vocab_total)
    return fail(FLCE_ERR_INVALID_ARG, "%d shards of a %lld-id vocabulary", (int)n_shards,
                (long long)vocab_total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T > 0 && (!lse_shards || !zt_shards || !y || !loss || !lse))
    return fail(FLCE_ERR_INVALID_ARG, "lse_shards, zt_shards, y, loss and lse must be non-NULL when T > 0");
  hipError_t e;
  if (T > 0) {
    flce::ShardMergeArgs m;
    m.lse_shards = lse_shards;
    m.zt_shards = zt_shards;
    m.tg = flce::Targets{y, ignore_index, 0, vocab_total};
    m.T = T;
    m.n_shards = n_shards;
    m.loss = loss;
    m.lse = lse;
    Timed tm(s, K_SHARD_MERGE, 0, (double)n_shards * T * 8 + T * 16.0);
    e = flce::launch_shard_merge(m, s);
    tm.done();
    if (e != hipSuccess) return hip_fail(e, "shard merge launch");
  }
  if (loss_reduced) {
    Timed tm(s, K_LOSS_SUM, 0, T * 4.0 + 4);
    e = launch_loss_sum(loss, T, scale, loss_reduced, s);
    tm.done();
    if (e != hipSuccess) return hip_fail(e, "loss_sum launch");
  }
  return ok();
}

flce_status_t flce_backward_shard(const flce_plan_t* plan, const void* H, const void* W_shard,
                                  const int64_t* y, const float* lse, int64_t ignore_index,
                                  int64_t vocab_start, int64_t vocab_total, float grad_scale,
                                  void* dH_partial, float* dW_shard, int accumulate_dW, void* ws,
                                  uint64_t ws_bytes, void* stream) {
  flce_status_t st = check_plan(plan);
  if (st != FLCE_OK) return st;
  st = check_shard(*plan, vocab_start, vocab_total);
  if (st != FLCE_OK) return st;
  const flce::Targets tg{y, ignore_index, vocab_start, vocab_total};
  return backward_impl(plan, H, W_shard, tg, lse, grad_scale, nullptr, dH_partial, dW_shard,
                       accumulate_dW, nullptr, ws, ws_bytes, stream);
}

flce_status_t flce_token_logprobs(int64_t T, int64_t d, int64_t V, flce_dtype_t dtype,
                                  const void* H, const void* W, const int64_t* tokens, int64_t K,
                                  const float* lse, float* out, void* stream) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16)
    return fail(FLCE_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (T < 0 || V < 1 || d < 1 || K < 0)
    return fail(FLCE_ERR_INVALID_ARG, "sizes T=%lld d=%lld V=%lld K=%lld out of range", (long long)T,
                (long long)d, (long long)V, (long long)K);
  if (d % 8 != 0) return fail(FLCE_ERR_UNSUPPORTED, "d = %lld is not a multiple of 8", (long long)d);
  if (T >= ((int64_t)1 << 31) || V >= ((int64_t)1 << 31) || d > 65536 || K >= ((int64_t)1 << 31) ||
      (K > 0 && T > (((int64_t)1 << 62) / K)))
    return fail(FLCE_ERR_UNSUPPORTED, "sizes beyond the limits");
  if (T == 0 || K == 0) return ok();
  if (!H || !W || !tokens || !out)
    return fail(FLCE_ERR_INVALID_ARG, "H, W, tokens and out must be non-NULL");
  if (misaligned(H) || misaligned(W))
    return fail(FLCE_ERR_UNSUPPORTED, "H and W must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  flce::TokenArgs a;
  a.H = H;
  a.W = W;
  a.tokens = tokens;
  a.lse = lse;
  a.T = T;
  a.d = (int)d;
  a.V = (int)V;
  a.K = (int)K;
  a.out = out;
  const double esz = dtype == FLCE_BF16 ? 2.0 : 4.0;
  Timed tm(s, K_TOKEN_LOGIT, 2.0 * T * K * d,
           (double)T * d * esz * (1.0 + K) + T * K * 12.0 + (lse ? T * 4.0 : 0.0));
  const hipError_t e = flce::launch_token_logit(a, dtype == FLCE_BF16, s);
  tm.done();
  if (e != hipSuccess) return hip_fail(e, "token logit launch");
  return ok();
}

}  // extern "C"
