// flce_host_check.cpp -- the library's host code (planning, validation and
// launch sequencing in flce_api.cpp), built for the CPU with AddressSanitizer
// and UndefinedBehaviorSanitizer against stand-ins for the GPU side: the kernel
// launchers of flce_launch.h and the few HIP runtime calls the host code makes.
//
// Device buffers are fake addresses that are never dereferenced.  Every
// stand-in launcher checks that each buffer the launch would touch lies inside
// one of the buffers the caller passed (its extent computed from the launch
// arguments), counts the launch, and returns hipSuccess.  The driver reads
// cases "T d V dtype cap" from stdin; for each it prints the plan, runs every
// entry point on it, and checks the validation paths (which must return their
// status before any launch).  Any violation aborts with a message.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../linear_cross_entropy_flce_amd/csrc/flce_launch.h"
#include "flce.h"

namespace {

struct Buf {
  std::string name;
  uintptr_t base;
  uint64_t bytes;
};
std::vector<Buf> g_bufs;
int64_t g_T = 0;        // tokens of the call under test
int g_launches = 0;     // launches since the last reset
int g_dz = 0, g_dhdw = 0, g_sweep = 0, g_target = 0, g_merge = 0;

[[noreturn]] void die(const char* fmt, const char* a, unsigned long long b,
                      unsigned long long c) {
  fprintf(stderr, "HOST CHECK FAILED: ");
  fprintf(stderr, fmt, a, b, c);
  fprintf(stderr, "\n");
  abort();
}

// The extent [p, p + bytes) must lie inside one registered buffer.
void in_buf(const void* p, double bytes_d, const char* what) {
  if (bytes_d <= 0) return;
  const uint64_t bytes = (uint64_t)bytes_d;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (!p) die("%s: NULL for %llu bytes%llu", what, bytes, 0);
  if (a % 16) die("%s: %llx is not 16-byte aligned%llu", what, a, 0);
  for (const Buf& b : g_bufs)
    if (a >= b.base && a - b.base <= b.bytes && bytes <= b.bytes - (a - b.base)) return;
  die("%s: [%llx, +%llu) outside every buffer", what, a, bytes);
}

void launched() { ++g_launches; }

}  // namespace

// ------------------------------------------------------------ HIP stand-ins
extern "C" {
const char* hipGetErrorString(hipError_t) { return "stand-in"; }
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  static char events[1 << 16];
  static size_t next = 0;
  *e = reinterpret_cast<hipEvent_t>(events + (next++ % sizeof events));
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.01f;
  return hipSuccess;
}
}

// -------------------------------------------------- kernel launcher stand-ins
namespace flce {

TileInfo tile_info(bool bf16) {
  // the tile shapes of flce_kernels.hip; a drift would change the plans, which
  // the test compares against the real library's
  TileInfo t;
  const int b = bf16 ? 256 : 128;
  t.logit_bm = t.logit_bn = t.dh_bm = t.dh_bn = t.dw_bm = t.dw_bn = b;
  t.dh_bk = bf16 ? 64 : 32;
  return t;
}
int64_t compact_chunks(int64_t T) { return (T + 4095) / 4096; }
// the static scratch array: a fake buffer registered per case by the driver
uintptr_t g_scratch = 0;
uint64_t scratch_bytes() { return FLCE_SCRATCH_BYTES; }
hipError_t scratch_address(void** out) {
  *out = reinterpret_cast<void*>(g_scratch);
  return hipSuccess;
}
int dh_split_slots() { return 256; }
// the default build: no workgroup timeline
hipError_t timeline_reset() { return hipErrorNotSupported; }
hipError_t timeline_read(TimelineRecord*, int, int* n_out) {
  *n_out = 0;
  return hipErrorNotSupported;
}

static double esz(bool bf16) { return bf16 ? 2.0 : 4.0; }

hipError_t launch_fwd_sweep(const FwdArgs& a, bool bf16, bool, int grid, hipStream_t) {
  if (grid <= 0 || a.splits < 1 || a.tps < 1 || a.grp < 1) die("sweep: grid %s%llu %llu", "", grid, a.splits);
  if ((int64_t)a.splits * a.tps < a.n_vtiles) die("sweep: %s%llu splits miss tiles of %llu", "", a.splits, a.n_vtiles);
  in_buf(a.H, (double)a.T * a.d * esz(bf16), "sweep H");
  in_buf(a.W, (double)a.V * a.d * esz(bf16), "sweep W");
  in_buf(a.tg.y, a.T * 8.0, "sweep y");
  in_buf(a.part, (double)a.splits * a.T * 8.0, "sweep partials");
  in_buf(a.zt, a.T * 4.0, "sweep zt");
  ++g_sweep;
  launched();
  return hipSuccess;
}
hipError_t launch_target_logit(const FwdArgs& a, bool bf16, hipStream_t) {
  in_buf(a.H, (double)a.T * a.d * esz(bf16), "target H");
  in_buf(a.W, (double)a.V * a.d * esz(bf16), "target W");
  in_buf(a.tg.y, a.T * 8.0, "target y");
  in_buf(a.zt, a.T * 4.0, "target zt");
  ++g_target;
  launched();
  return hipSuccess;
}
hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t) {
  in_buf(a.part, (double)a.splits * a.T * 8.0, "merge partials");
  in_buf(a.zt, a.T * 4.0, "merge zt");
  in_buf(a.lse, a.T * 4.0, "merge lse");
  in_buf(a.shard ? a.zt_out : a.loss, a.T * 4.0, "merge out");
  ++g_merge;
  launched();
  return hipSuccess;
}
hipError_t launch_loss_reduce(const ReduceArgs& a, hipStream_t) {
  in_buf(a.loss, a.T * 4.0, "reduce loss");
  if (a.mean_valid) in_buf(a.y, a.T * 8.0, "reduce y");
  if (a.out) in_buf(a.out, 4, "reduce out");
  if (a.g_out) in_buf(a.g_out, 4, "reduce g");
  launched();
  return hipSuccess;
}
hipError_t launch_cast_bf16(const float* src, void* dst, int64_t n, hipStream_t) {
  in_buf(src, n * 4.0, "cast src");
  in_buf(dst, n * 2.0, "cast dst");
  launched();
  return hipSuccess;
}
hipError_t launch_bwd_dz(const DzArgs& a, bool bf16, hipStream_t) {
  const TileInfo ti = tile_info(bf16);
  if (a.ldz_cols > a.ldz) die("dz: %scols %llu > pitch %llu", "", a.ldz_cols, a.ldz);
  if (a.v_begin + (int64_t)a.n_vtiles * ti.logit_bm - ti.logit_bm >= a.V)
    die("dz: %sslab tiles %llu past V %llu", "", a.n_vtiles, a.V);
  in_buf(a.Hc, (double)a.blk.t_max * a.d * esz(bf16), "dz Hc");
  in_buf(a.W, (double)a.V * a.d * esz(bf16), "dz W");
  in_buf(a.lse, g_T * 4.0, "dz lse");
  in_buf(a.tg.y, g_T * 8.0, "dz y");
  in_buf(a.blk.idx, g_T * 4.0, "dz idx");
  in_buf(a.blk.tv, 4, "dz tv");
  in_buf(a.dz, (double)a.blk.t_max * a.ldz * esz(bf16), "dz buffer");
  if (a.g_dev) in_buf(a.g_dev, 4, "dz g");
  if (a.blk.t_begin < 0 || a.blk.t_begin >= g_T) die("dz: %sblock start %llu of %llu", "", a.blk.t_begin, g_T);
  ++g_dz;
  launched();
  return hipSuccess;
}
hipError_t launch_bwd_dhdw(const DhArgs& h, const DwArgs& w, bool bf16, hipStream_t) {
  const TileInfo ti = tile_info(bf16);
  const double e = esz(bf16);
  if ((double)h.k_count * h.d * e >= 2147483648.0) die("dh: %sslab of %llu rows x %llu past 2^31 bytes", "", h.k_count, h.d);
  in_buf(h.dz, (double)h.blk.t_max * h.ldz * e, "dh dz");
  in_buf(h.W, (double)h.V * h.d * e, "dh W");
  in_buf((const char*)h.W + h.v_begin * h.d * (int64_t)e, (double)h.k_count * h.d * e, "dh W slab");
  if (h.mode != 3) in_buf(h.dh_acc, (double)h.blk.t_max * h.d * 4.0, "dh accumulator");
  in_buf(h.dH, (double)g_T * h.d * e, "dh dH");
  if (h.part) in_buf(h.part, (double)dh_split_slots() * ti.dh_bm * ti.dh_bn * 4.0, "dh partials");
  in_buf(w.dz, (double)w.blk.t_max * w.ldz * e, "dw dz");
  in_buf(w.Ht, (double)w.d * w.ldht * e, "dw Ht");
  in_buf((const float*)w.dW + w.v_begin * w.d, (double)w.v_count * w.d * 4.0, "dw dW");
  ++g_dhdw;
  launched();
  return hipSuccess;
}
hipError_t launch_bwd_dh_reduce(const DhArgs& h, bool bf16, hipStream_t) {
  const TileInfo ti = tile_info(bf16);
  in_buf(h.part, (double)dh_split_slots() * ti.dh_bm * ti.dh_bn * 4.0, "reduce partials");
  in_buf(h.dH, (double)g_T * h.d * esz(bf16), "reduce dH");
  launched();
  return hipSuccess;
}
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t) {
  in_buf(p, n * 4.0, "fill");
  launched();
  return hipSuccess;
}
hipError_t launch_token_logit(const TokenArgs& a, bool bf16, hipStream_t) {
  in_buf(a.H, (double)a.T * a.d * esz(bf16), "token H");
  in_buf(a.W, (double)a.V * a.d * esz(bf16), "token W");
  in_buf(a.tokens, (double)a.T * a.K * 8.0, "token ids");
  if (a.lse) in_buf(a.lse, a.T * 4.0, "token lse");
  in_buf(a.out, (double)a.T * a.K * 4.0, "token out");
  launched();
  return hipSuccess;
}
hipError_t launch_compact(const int64_t* y, int64_t, int64_t T, int* cnt, int* idx, int* tv,
                          hipStream_t) {
  in_buf(y, T * 8.0, "compact y");
  in_buf(cnt, compact_chunks(T) * 4.0, "compact counts");
  in_buf(idx, T * 4.0, "compact idx");
  in_buf(tv, 4, "compact total");
  launched();
  return hipSuccess;
}
hipError_t launch_zero_rows(void* dH, const int* idx, const int* tv, int64_t T, int d, bool bf16,
                            hipStream_t) {
  in_buf(dH, (double)T * d * esz(bf16), "zero dH");
  in_buf(idx, T * 4.0, "zero idx");
  in_buf(tv, 4, "zero total");
  launched();
  return hipSuccess;
}
hipError_t launch_gather_block(const void* H, const TokBlock& blk, int d, void* Hc, void* Ht,
                               bool bf16, hipStream_t) {
  in_buf(H, (double)g_T * d * esz(bf16), "gather H");
  in_buf(Hc, (double)blk.t_max * d * esz(bf16), "gather Hc");
  in_buf(Ht, (double)blk.t_max * d * esz(bf16), "gather Ht");
  launched();
  return hipSuccess;
}
hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t) {
  in_buf(a.lse_shards, (double)a.n_shards * a.T * 4.0, "shard lse");
  in_buf(a.zt_shards, (double)a.n_shards * a.T * 4.0, "shard zt");
  in_buf(a.tg.y, a.T * 8.0, "shard y");
  in_buf(a.loss, a.T * 4.0, "shard loss");
  in_buf(a.lse, a.T * 4.0, "shard merged lse");
  launched();
  return hipSuccess;
}

}  // namespace flce

// --------------------------------------------------------------------- driver
namespace {

int g_fail = 0;

void expect(bool ok, const char* what, long long a = 0, long long b = 0) {
  if (!ok) {
    fprintf(stderr, "EXPECTATION FAILED: %s (%lld, %lld): %s\n", what, a, b, flce_last_error());
    ++g_fail;
  }
}

// A fake device buffer 16 TiB apart from the others.
const void* buf(const char* name, double bytes) {
  const uintptr_t base = (uintptr_t)(g_bufs.size() + 1) << 44;
  g_bufs.push_back(Buf{name, base, (uint64_t)(bytes > 0 ? bytes : 0)});
  return reinterpret_cast<const void*>(base);
}

template <typename T>
T* p(const void* v) {
  return const_cast<T*>(reinterpret_cast<const T*>(v));
}

void reset() { g_launches = g_dz = g_dhdw = g_sweep = g_target = g_merge = 0; }

// Every validation failure returns before anything is launched.
void expect_status(flce_status_t got, flce_status_t want, const char* what) {
  expect(got == want, what, got, want);
  if (want != FLCE_OK) {
    expect(g_launches == 0, "a rejected call launched something", g_launches, 0);
    expect(flce_last_error()[0] != 0, "a rejected call left no message");
  }
  reset();
}

void run_case(int64_t T, int64_t d, int64_t V, int dt, unsigned long long cap) {
  flce_plan_t plan;
  const flce_status_t st = flce_plan(T, d, V, (flce_dtype_t)dt, cap, &plan);
  if (st != FLCE_OK) {
    printf("PLAN %lld %lld %lld %d %llu status %d\n", (long long)T, (long long)d, (long long)V, dt,
           cap, (int)st);
    expect(flce_last_error()[0] != 0, "planner failure without a message");
    return;
  }
  printf("PLAN %lld %lld %lld %d %llu status 0 splits %d tps %d block %lld slab %lld nb %lld ns %lld "
         "fws %llu bws %llu ws %llu split %llu\n",
         (long long)T, (long long)d, (long long)V, dt, cap, plan.fwd_splits,
         plan.fwd_tiles_per_split, (long long)plan.bwd_block, (long long)plan.bwd_slab,
         (long long)plan.n_blocks, (long long)plan.n_slabs, (unsigned long long)plan.fwd_ws_bytes,
         (unsigned long long)plan.bwd_ws_bytes, (unsigned long long)plan.ws_bytes,
         (unsigned long long)plan.dh_split_bytes);
  expect(plan.ws_bytes >= plan.fwd_ws_bytes && plan.ws_bytes >= plan.bwd_ws_bytes,
         "ws_bytes below a part");
  expect(plan.bwd_ws_bytes <= plan.vocab_ws_cap, "backward workspace above the cap");
  expect(plan.n_slabs * plan.bwd_slab >= V && (plan.n_slabs - 1) * plan.bwd_slab < V,
         "slabs do not tile V");
  expect(T == 0 || (plan.n_blocks * plan.bwd_block >= T && (plan.n_blocks - 1) * plan.bwd_block < T),
         "blocks do not tile T");

  g_bufs.clear();
  g_T = T;
  const double e = dt == FLCE_BF16 ? 2.0 : 4.0;
  const int64_t K = 3;
  const void* H = buf("H", T * d * e);
  const void* W = buf("W", V * d * e);
  const void* y = buf("y", T * 8.0);
  const void* loss = buf("loss", T * 4.0);
  const void* lse = buf("lse", T * 4.0);
  const void* red = buf("loss_reduced", 4);
  const void* dH = buf("dH", T * d * e);
  const void* dW = buf("dW", V * d * 4.0);
  const void* dWb = buf("dW_bf16", V * d * 2.0);
  const void* ws = buf("ws", (double)plan.ws_bytes);
  const void* tok = buf("tokens", T * K * 8.0);
  const void* out = buf("scores", T * K * 4.0);
  const void* lse2 = buf("lse_shards", 2.0 * T * 4);
  const void* zt2 = buf("zt_shards", 2.0 * T * 4);
  const uint64_t wsb = plan.ws_bytes;
  flce::g_scratch = reinterpret_cast<uintptr_t>(buf("scratch", (double)FLCE_SCRATCH_BYTES));
  reset();

  // ---- every entry point on the plan
  for (uint32_t mode : {0u, 1u}) {
    flce_plan_t pm = plan;
    pm.target_logit = mode;
    expect_status(flce_forward(&pm, H, W, p<int64_t>(y), -100, 0.5f, p<float>(loss), p<float>(lse),
                               p<float>(red), p<void>(ws), wsb, nullptr),
                  FLCE_OK, "forward");
  }
  for (int acc : {0, 1}) {
    flce_status_t s = flce_backward(&plan, H, W, p<int64_t>(y), p<float>(lse), -100, 0.5f,
                                    p<void>(dH), p<float>(dW), acc, p<void>(ws), wsb, nullptr);
    expect(T == 0 || g_dz == plan.n_blocks * plan.n_slabs, "dZ launches", g_dz,
           plan.n_blocks * plan.n_slabs);
    expect(T == 0 || g_dhdw == plan.n_blocks * plan.n_slabs, "dH/dW launches", g_dhdw,
           plan.n_blocks * plan.n_slabs);
    expect_status(s, FLCE_OK, "backward");
  }
  for (flce_reduction_t r : {FLCE_REDUCE_SUM, FLCE_REDUCE_MEAN_VALID})
    for (const void* b16 : {(const void*)nullptr, dWb})
      expect_status(flce_forward_backward(&plan, H, W, p<int64_t>(y), -100, r, 1.f, p<float>(loss),
                                          p<float>(lse), p<float>(red), p<void>(dH), p<float>(dW),
                                          0, p<void>(b16), p<void>(ws), wsb, nullptr),
                    FLCE_OK, "forward_backward");
  // the allocation-free variant: the plan fits the scratch array, or the
  // call is refused before any launch
  expect_status(flce_forward_backward_scratch(&plan, H, W, p<int64_t>(y), -100,
                                              FLCE_REDUCE_MEAN_VALID, 1.f, p<float>(loss),
                                              p<float>(lse), p<float>(red), p<void>(dH),
                                              p<float>(dW), 1, p<void>(dWb), nullptr),
                plan.ws_bytes <= FLCE_SCRATCH_BYTES ? FLCE_OK : FLCE_ERR_WORKSPACE,
                "forward_backward_scratch");
  // this plan as a shard [vs, vs + V) of a vocabulary of vt ids
  const int64_t vt = V + 9 < ((int64_t)1 << 31) ? V + 9 : ((int64_t)1 << 31) - 1;
  const int64_t vs = (vt - V) / 2;
  expect_status(flce_forward_shard(&plan, H, W, p<int64_t>(y), -100, vs, vt, p<float>(lse2),
                                   p<float>(zt2), p<void>(ws), wsb, nullptr),
                FLCE_OK, "forward_shard");
  expect_status(flce_merge_shards(T, 2, p<float>(lse2), p<float>(zt2), p<int64_t>(y), -100, vt,
                                  1.f, p<float>(loss), p<float>(lse), p<float>(red), nullptr),
                FLCE_OK, "merge_shards");
  expect_status(flce_backward_shard(&plan, H, W, p<int64_t>(y), p<float>(lse), -100, vs, vt, 1.f,
                                    p<void>(dH), p<float>(dW), 1, p<void>(ws), wsb, nullptr),
                FLCE_OK, "backward_shard");
  expect_status(flce_token_logprobs(T, d, V, (flce_dtype_t)dt, H, W, p<int64_t>(tok), K,
                                    p<float>(lse), p<float>(out), nullptr),
                FLCE_OK, "token_logprobs");

  // ---- validation paths
  if (T > 0) {
    const void* Hm = reinterpret_cast<const char*>(H) + 8;
    expect_status(flce_forward(&plan, Hm, W, p<int64_t>(y), -100, 1.f, p<float>(loss),
                               p<float>(lse), nullptr, p<void>(ws), wsb, nullptr),
                  FLCE_ERR_UNSUPPORTED, "misaligned H");
    expect_status(flce_forward(&plan, H, W, p<int64_t>(y), -100, 1.f, p<float>(loss),
                               p<float>(lse), nullptr, p<void>(ws), plan.fwd_ws_bytes - 1, nullptr),
                  FLCE_ERR_WORKSPACE, "small forward workspace");
    expect_status(flce_backward(&plan, H, W, p<int64_t>(y), p<float>(lse), -100, 1.f, p<void>(dH),
                                p<float>(dW), 0, p<void>(ws), plan.bwd_ws_bytes - 1, nullptr),
                  FLCE_ERR_WORKSPACE, "small backward workspace");
    expect_status(flce_forward_backward(&plan, H, W, p<int64_t>(y), -100, FLCE_REDUCE_SUM, 1.f,
                                        p<float>(loss), p<float>(lse), nullptr, p<void>(dH),
                                        p<float>(dW), 0, nullptr, p<void>(ws), wsb - 1, nullptr),
                  FLCE_ERR_WORKSPACE, "small fused workspace");
    expect_status(flce_backward(&plan, nullptr, W, p<int64_t>(y), p<float>(lse), -100, 1.f,
                                p<void>(dH), p<float>(dW), 0, p<void>(ws), wsb, nullptr),
                  FLCE_ERR_INVALID_ARG, "NULL H");
    expect_status(flce_token_logprobs(T, d, V, (flce_dtype_t)dt, H, W, nullptr, K, p<float>(lse),
                                      p<float>(out), nullptr),
                  FLCE_ERR_INVALID_ARG, "NULL tokens");
  }
  flce_plan_t bad = plan;
  bad.magic ^= 1u;
  expect_status(flce_forward(&bad, H, W, p<int64_t>(y), -100, 1.f, p<float>(loss), p<float>(lse),
                             nullptr, p<void>(ws), wsb, nullptr),
                FLCE_ERR_INVALID_ARG, "foreign plan");
  bad = plan;
  bad.target_logit = 7;
  expect_status(flce_forward(&bad, H, W, p<int64_t>(y), -100, 1.f, p<float>(loss), p<float>(lse),
                             nullptr, p<void>(ws), wsb, nullptr),
                FLCE_ERR_INVALID_ARG, "unknown target_logit");
  expect_status(flce_forward(nullptr, H, W, p<int64_t>(y), -100, 1.f, p<float>(loss),
                             p<float>(lse), nullptr, p<void>(ws), wsb, nullptr),
                FLCE_ERR_INVALID_ARG, "NULL plan");
  expect_status(flce_forward_backward(&plan, H, W, p<int64_t>(y), -100, (flce_reduction_t)5, 1.f,
                                      p<float>(loss), p<float>(lse), nullptr, p<void>(dH),
                                      p<float>(dW), 0, nullptr, p<void>(ws), wsb, nullptr),
                FLCE_ERR_INVALID_ARG, "unknown reduction");
  expect_status(flce_forward_shard(&plan, H, W, p<int64_t>(y), -100, vt - V + 1, vt, p<float>(lse2),
                                   p<float>(zt2), p<void>(ws), wsb, nullptr),
                FLCE_ERR_INVALID_ARG, "shard past the vocabulary");
  expect_status(flce_merge_shards(T, 0, p<float>(lse2), p<float>(zt2), p<int64_t>(y), -100, V,
                                  1.f, p<float>(loss), p<float>(lse), nullptr, nullptr),
                FLCE_ERR_INVALID_ARG, "no shards");
}

}  // namespace

int main() {
  long long T, d, V;
  int dt;
  unsigned long long cap;
  int n = 0;
  while (scanf("%lld %lld %lld %d %llu", &T, &d, &V, &dt, &cap) == 5) {
    run_case(T, d, V, dt, cap);
    ++n;
  }
  // the planner's own argument checks
  flce_plan_t pl;
  expect(flce_plan(10, 128, 1000, FLCE_BF16, 0, nullptr) == FLCE_ERR_INVALID_ARG, "NULL out");
  expect(flce_plan(10, 128, 1000, (flce_dtype_t)9, 0, &pl) == FLCE_ERR_INVALID_ARG, "bad dtype");
  // the timeline calls of a library built without it
  flce_wg_record_t recs[2];
  int got = -1;
  expect(flce_timeline_reset() == FLCE_ERR_UNSUPPORTED, "timeline reset");
  expect(flce_timeline_read(recs, 2, &got) == FLCE_ERR_UNSUPPORTED && got == 0, "timeline read");
  expect(flce_timeline_read(nullptr, 2, &got) == FLCE_ERR_INVALID_ARG, "timeline read NULL");
  printf("CASES %d FAILURES %d\n", n, g_fail);
  return g_fail ? 1 : 0;
}
