// flce_kernels.hip -- the fused linear cross-entropy kernels for gfx950.
//
// Orientation: every logit tile is computed transposed, Z^T = W H^T, with the
// vocab axis as the MFMA M dimension and tokens as N.  A lane then holds 16
// vocab rows of one token column per 32x32 block, so the per-token softmax
// statistics reduce inside the lane's own registers; the two half-waves
// (rows 4*(lane/32)..) and the waves stacked along M are merged only once, at
// the end of a workgroup's sweep.
//
// Kernels (the method is section 3 of "Long-Sequence MoE RL Training: From
// First Principles to MI300X"):
//   fwd_sweep    logits tile + running max / log-sum-exp over the workgroup's
//                vocab range, target logit captured from the fp32 accumulator;
//                writes per-split (max, sum) partials and z_target.
//   fwd_merge    merges the splits in ascending order: lse, loss (or, for a
//                vocab shard, the shard's lse and target logit).
//   shard_merge  lse and loss from several shards' statistics.
//   loss_reduce  fixed-order double-precision sum (and count) for the reduced loss.
//   compact_*    the backward's token order: non-ignored tokens first, ascending.
//   zero_rows    dH rows of the ignored tokens.
//   gather_block one token block of H in that order, as rows and transposed.
//   bwd_dz       recomputed logits tile -> dZ = g * (exp(z - lse) - onehot),
//                stored (bf16 or fp32) to the [block x slab] workspace.
//   bwd_dhdw     one launch of both contractions of a block and slab (dH
//                workgroups first, so a partial last round of dH's long tiles
//                fills with dW's short ones):
//                dH_block (+)= dZ W_slab   (fp32 accumulate, cast at the end;
//                the slab's K loop cut into parts when the block has too few
//                tiles to occupy the GPU), and
//                dW_slab^T (+)= H_block^T dZ (fp32, deterministic block order);
//                the last block holding tokens also writes the optional bf16
//                copy of dW from the same tiles.
//   bwd_dh_reduce  sums dH's parts in order and applies the accumulator mode.
//   token_logit  gathered h . w minus lse for given tokens (scoring), up to
//                eight gathered rows per pass.
//   cast_bf16    the bf16 copy of dW when no dW tile runs (T = 0).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "flce_launch.h"
#include "flce_tile.hpp"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Argument of exp2 for exp(z - m).  bf16 inputs: one FMA, z * log2(e) + nb with
// nb = -m * log2(e); its rounding error (|z| * 2^-24 relative to the exponent)
// is far below bf16 input precision.  fp32 inputs: subtract first, so the
// exponent error stays at the rounding of (z - m).
template <int ESZ>
__device__ __forceinline__ float exp2_arg(float z, float m, float nb) {
  if constexpr (ESZ == 2) return fmaf(z, kLog2e, nb);
  else return (z - m) * kLog2e;
}
// Same for g * exp(z - lse) with log2|g| folded in (bias = log2|g| - lse * log2(e),
// or +-inf / NaN for ignored / invalid targets, which the fp32 form keeps).
template <int ESZ>
__device__ __forceinline__ float dz_arg(float z, float lse, float log2g, float bias) {
  if constexpr (ESZ == 2) return fmaf(z, kLog2e, bias);
  else return (bias != bias || bias == kNegInf) ? bias : fmaf(z - lse, kLog2e, log2g);
}

// Tile shapes: 256 x 256 per workgroup in 2 x 4 waves of 128 x 64 (bf16);
// 128 x 128 in 2 x 2 waves of 64 x 64 for fp32.  Each kernel picks its
// global -> LDS path (DMA ring of NS stages with 64-byte k rows, or the
// register-staged double buffer with 128-byte k rows) by measurement.
#ifndef FLCE_LOGIT_NS
#define FLCE_LOGIT_NS 2
#endif
#ifndef FLCE_DH_NS
#define FLCE_DH_NS 2
#endif
#ifndef FLCE_DW_NS
#define FLCE_DW_NS 2
#endif
#ifndef FLCE_BIG_WN
#define FLCE_BIG_WN 4
#endif
#ifndef FLCE_LOGIT_KB
#define FLCE_LOGIT_KB 128
#endif
#ifndef FLCE_DH_KB
#define FLCE_DH_KB 128
#endif
#ifndef FLCE_DW_KB
#define FLCE_DW_KB 128
#endif
#ifndef FLCE_LOGIT_DMA
#define FLCE_LOGIT_DMA 0
#endif
#ifndef FLCE_DH_DMA
#define FLCE_DH_DMA 0
#endif
#ifndef FLCE_DW_DMA
#define FLCE_DW_DMA 0
#endif
template <typename E, bool A_KC, bool B_KC, int NS, int KB, bool DMA>
using BigTile = Tile<256, 256, 2, FLCE_BIG_WN, E, A_KC, B_KC, KB, NS, DMA || NS != 2>;
template <typename E, bool A_KC, bool B_KC, int NS>
using SmallTile = Tile<128, 128, 2, 2, E, A_KC, B_KC, NS == 2 ? 128 : 64, NS, NS != 2>;

// Logits (A = W rows, B = H rows, both K-contiguous).
template <typename E>
struct LogitCfg;
template <>
struct LogitCfg<__bf16> {
  using T = BigTile<__bf16, true, true, FLCE_LOGIT_NS, FLCE_LOGIT_KB, FLCE_LOGIT_DMA>;
};
template <>
struct LogitCfg<float> {
  using T = SmallTile<float, true, true, FLCE_LOGIT_NS>;
};

// dH, computed as its transpose dH^T = W[slab]^T dZ^T: M = hidden, N = tokens,
// K = slab vocab (A = W MN-contiguous, B = dZ K-contiguous), so that each
// lane's accumulator quads are four consecutive hidden units of one token row
// (16-byte accumulator and dH accesses, one token lookup per column).  The
// bf16 tile's 8 waves are 4 x 2 (64 hidden x 128 tokens each): measured as
// fast as the untransposed 2 x 4 product, where 2 x 4 with A MN-contiguous
// was 2% slower.
template <typename E>
struct DhCfg;
template <>
struct DhCfg<__bf16> {
  using T = Tile<256, 256, 4, 2, __bf16, false, true, FLCE_DH_KB, FLCE_DH_NS,
                 FLCE_DH_DMA || FLCE_DH_NS != 2>;
};
template <>
struct DhCfg<float> {
  using T = SmallTile<float, false, true, FLCE_DH_NS>;
};
template <typename E>
struct DwCfg;
// dW^T = Ht[block] dZ: A = the token block's H, transposed into the workspace
// (K-contiguous); B = dZ (MN-contiguous).
template <>
struct DwCfg<__bf16> {
  using T = BigTile<__bf16, true, false, FLCE_DW_NS, FLCE_DW_KB, FLCE_DW_DMA>;
};
template <>
struct DwCfg<float> {
  using T = SmallTile<float, true, false, FLCE_DW_NS>;
};

// Tokens in a block of the compacted order (0 when it lies past the last
// non-ignored token).
__device__ __forceinline__ int block_count(const TokBlock& b) {
  const int64_t n = (int64_t)*b.tv - b.t_begin;
  return n <= 0 ? 0 : (n < b.t_max ? (int)n : b.t_max);
}

// ------------------------------------------------------ workgroup timeline
// Profiling build only (-DFLCE_TIMELINE=1, libflce_timeline.so): each
// workgroup of the forward sweep, the dZ recompute and the dH/dW launch
// records the compute unit it ran on (HW_ID and XCC_ID registers) and
// wall-clock stamps (the 100 MHz real-time counter) at its start and after
// its last store was issued, so that a launch's compute-unit time can be
// split into workgroups, the gaps between them and the launch's tail.  In
// the default build the stamps compile to nothing.
#ifndef FLCE_TIMELINE
#define FLCE_TIMELINE 0
#endif
#if FLCE_TIMELINE
constexpr unsigned kTimelineCap = 1u << 19;
__device__ TimelineRecord g_timeline[kTimelineCap];
__device__ unsigned int g_timeline_n;
#endif

__device__ __forceinline__ uint64_t timeline_start() {
#if FLCE_TIMELINE
  return wall_clock64();
#else
  return 0;
#endif
}

__device__ __forceinline__ void timeline_end(uint32_t kernel, uint64_t t_start) {
#if FLCE_TIMELINE
  if (threadIdx.x == 0) {
    const uint64_t t_end = wall_clock64();
    const unsigned slot = atomicAdd(&g_timeline_n, 1u);
    if (slot < kTimelineCap) {
      TimelineRecord r;
      r.hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID, 32 bits
      r.xcc_id = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID, 32 bits
      r.t_start = t_start;
      r.t_end = t_end;
      r.kernel = kernel;
      r.block = blockIdx.x;
      g_timeline[slot] = r;
    }
  }
#else
  (void)kernel;
  (void)t_start;
#endif
}

// The last block that holds a non-ignored token (block 0 when there is none):
// the one whose dW is final for the whole call.
__device__ __forceinline__ bool last_filled_block(const TokBlock& b) {
  const int64_t tv = *b.tv;
  return tv == 0 ? b.t_begin == 0 : (b.t_begin < tv && tv <= b.t_begin + b.t_max);
}

__device__ __forceinline__ uint32_t clamp_bytes(int64_t b) {
  return (uint32_t)(b < 0 ? 0 : (b > 0x7fffffffLL ? 0x7fffffffLL : b));
}

// Target of token t: its row in this vocab shard, in [0, V); or -1 when the
// token is ignored, -2 when the target is outside [0, total) (invalid), -3
// when it is valid but belongs to another shard.
constexpr int kIgnored = -1, kInvalid = -2, kElsewhere = -3;
__device__ __forceinline__ int target_code(const Targets& g, int64_t t, int V) {
  const int64_t v = g.y[t];
  if (v == g.ignore_index) return kIgnored;
  if (v < 0 || v >= g.total) return kInvalid;
  const int64_t r = v - g.start;
  return r >= 0 && r < V ? (int)r : kElsewhere;
}

// ============================================================== forward sweep
//
// Workgroup (token tile tt, split s) sweeps vocab tiles
// [s * tps, min((s+1) * tps, n_vtiles)).  The linear workgroup id is mapped so
// that the 32 workgroups an XCD holds at once are `grp` token tiles x `spl`
// splits: they share H panels within a token tile and W panels across the
// token tiles, in that XCD's L2.
template <typename E, bool CAPTURE>
__global__ void __launch_bounds__(LogitCfg<E>::T::NT, 1)
    fwd_sweep_kernel(FwdArgs a) {
  using TL = typename LogitCfg<E>::T;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int ESZ = TL::ESZ;
  const uint64_t tl_t0 = timeline_start();

  // ---- workgroup -> (token tile, split)
  const int bid = blockIdx.x;
  const int x = bid & 7, q = bid >> 3;
  const int per_group = a.grp * a.splits;
  const int gi = (q / per_group) * 8 + x;
  const int within = q % per_group;
  const int split = within / a.grp;
  const int tt = gi * a.grp + within % a.grp;
  if (tt >= a.n_ttiles) return;
  const int vt_begin = split * a.tps;
  const int vt_end = min(vt_begin + a.tps, a.n_vtiles);
  if (vt_begin >= vt_end) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int64_t t0 = (int64_t)tt * TL::BN;

  // B operand: H rows of this token tile (K-contiguous).  Each operand tile
  // gets a buffer resource based at its own first row, so H and W may exceed
  // the 2^31 bytes that 32-bit buffer offsets reach: only a tile (at most
  // 256 rows x 65,536 elements) has to lie below that.
  Operand B;
  B.rows = (int)min<int64_t>(TL::BN, a.T - t0);
  B.rs = make_rsrc(reinterpret_cast<const char*>(a.H) + t0 * a.d * ESZ,
                   (uint32_t)((int64_t)B.rows * a.d * ESZ));
  B.off = 0;
  B.ld_bytes = (uint32_t)(a.d * ESZ);
  B.cols = a.d;

  // Per-lane state for its NI token columns: running max and sum over the
  // vocab rows this lane holds, and the target (row index) of each column.
  float m_run[TL::NI], s_run[TL::NI];
  int tgt[TL::NI];
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    m_run[j] = kNegInf;
    s_run[j] = 0.f;
    const int64_t t = t0 + TL::col_of(wn, j);
    tgt[j] = CAPTURE && t < a.T ? target_code(a.tg, t, a.V) : kIgnored;
  }

  TL tile;
  Operand A;
  A.off = 0;
  A.ld_bytes = (uint32_t)(a.d * ESZ);
  A.cols = a.d;
  for (int vt = vt_begin; vt < vt_end; ++vt) {
    const int64_t v0 = (int64_t)vt * TL::BM;
    A.rows = (int)min<int64_t>(TL::BM, a.V - v0);
    A.rs = make_rsrc(reinterpret_cast<const char*>(a.W) + v0 * a.d * ESZ,
                     (uint32_t)((int64_t)A.rows * a.d * ESZ));
    tile.zero();
    tile.mainloop(A, B, a.d, lds);

    // rows past V (last tile only) do not take part; `lim` is the number of
    // valid rows counted from this lane's first row
    if (v0 + TL::BM > a.V) {
      const int lim = a.V - (int)v0 - wm * TL::WTM - 4 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (i * 32 + 8 * (r >> 2) + (r & 3) >= lim)
#pragma unroll
            for (int j = 0; j < TL::NI; ++j) tile.acc[i][j][r] = kNegInf;
    }

    const int wrow0 = (int)v0 + wm * TL::WTM;  // first vocab id of this wave's rows
#pragma unroll
    for (int j = 0; j < TL::NI; ++j) {
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, tile.acc[i][j][r]);
      const float m_new = fmaxf(m_run[j], mx);
      if (m_new != kNegInf) {
        const float nb = -m_new * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += fast_exp2(exp2_arg<TL::ESZ>(tile.acc[i][j][r], m_new, nb));
        s_run[j] = s_run[j] * fast_exp2((m_run[j] - m_new) * kLog2e) + sum;
        m_run[j] = m_new;
      }
      // target logit, taken from the fp32 accumulator (rare: one tile per
      // token); without CAPTURE the sweep is a pure log-sum-exp and the
      // target logits come from a gathered dot product afterwards
      const int rt = tgt[j] - wrow0 - 4 * (lane >> 5);
      if (CAPTURE && tgt[j] >= wrow0 && tgt[j] < wrow0 + TL::WTM) {
        float zt = 0.f;
        bool hit = false;
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rt == i * 32 + 8 * (r >> 2) + (r & 3)) {
              zt = tile.acc[i][j][r];
              hit = true;
            }
        if (hit) a.zt[t0 + TL::col_of(wn, j)] = zt;
      }
    }
  }

  // ---- merge the two half-waves (same columns, interleaved rows)
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    const float mo = __shfl_xor(m_run[j], 32);
    const float so = __shfl_xor(s_run[j], 32);
    const float mn = fmaxf(m_run[j], mo);
    if (mn != kNegInf) {
      s_run[j] = s_run[j] * fast_exp2((m_run[j] - mn) * kLog2e) + so * fast_exp2((mo - mn) * kLog2e);
      m_run[j] = mn;
    }
  }
  // ---- merge the waves stacked along M through LDS, in ascending wm order
  float* red = reinterpret_cast<float*>(lds);  // [WM][BN][2]
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < TL::NI; ++j) {
      const int c = TL::col_of(wn, j);
      red[(wm * TL::BN + c) * 2 + 0] = m_run[j];
      red[(wm * TL::BN + c) * 2 + 1] = s_run[j];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < TL::BN; c += TL::NT) {
    const int64_t t = t0 + c;
    if (t >= a.T) continue;
    float M = kNegInf, S = 0.f;
    for (int w = 0; w < TL::WM; ++w) {
      const float mw = red[(w * TL::BN + c) * 2 + 0];
      const float sw = red[(w * TL::BN + c) * 2 + 1];
      const float mn = fmaxf(M, mw);
      if (mn != kNegInf) {
        S = S * fast_exp2((M - mn) * kLog2e) + sw * fast_exp2((mw - mn) * kLog2e);
        M = mn;
      }
    }
    a.part[((int64_t)split * a.T + t) * 2 + 0] = M;
    a.part[((int64_t)split * a.T + t) * 2 + 1] = S;
  }
  timeline_end(kTimelineFwdSweep, tl_t0);
}

// ============================================================== forward merge
__global__ void __launch_bounds__(256) fwd_merge_kernel(MergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  float M = kNegInf, S = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float ms = a.part[((int64_t)s * a.T + t) * 2 + 0];
    const float ss = a.part[((int64_t)s * a.T + t) * 2 + 1];
    const float mn = fmaxf(M, ms);
    if (mn != kNegInf) {
      S = S * expf(M - mn) + ss * expf(ms - mn);
      M = mn;
    }
  }
  const float lse = M + logf(S);
  a.lse[t] = lse;
  const int code = target_code(a.tg, t, a.V);
  if (a.shard) {
    a.zt_out[t] = code >= 0 ? a.zt[t] : kNegInf;
    return;
  }
  float loss;
  if (code == kIgnored) loss = 0.f;
  else if (code < 0) loss = __builtin_nanf("");  // invalid (no other shards here)
  else loss = lse - a.zt[t];
  a.loss[t] = loss;
}

// =============================================================== shard merge
// Per token: lse = log-sum-exp of the shards' lse in ascending shard order;
// the target logit is the one shard value that is not -inf.  A valid token
// whose target no shard holds gets a NaN loss.
__global__ void __launch_bounds__(256) shard_merge_kernel(ShardMergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  float M = kNegInf, zt = kNegInf;
  for (int p = 0; p < a.n_shards; ++p) {
    M = fmaxf(M, a.lse_shards[(int64_t)p * a.T + t]);
    zt = fmaxf(zt, a.zt_shards[(int64_t)p * a.T + t]);
  }
  float S = 0.f;
  for (int p = 0; p < a.n_shards; ++p) S += expf(a.lse_shards[(int64_t)p * a.T + t] - M);
  const float lse = M + logf(S);
  a.lse[t] = lse;
  const int64_t v = a.tg.y[t];
  float loss;
  if (v == a.tg.ignore_index) loss = 0.f;
  else if (v < 0 || v >= a.tg.total || zt == kNegInf) loss = __builtin_nanf("");
  else loss = lse - zt;
  a.loss[t] = loss;
}

// Fixed-order reduction: thread x sums loss[x + 1024 k] in double into eight
// interleaved partial sums (k mod 8), so that eight independent loads per
// thread are in flight, then adds them in a fixed tree; for a mean over the
// non-ignored tokens it also counts them; then a tree over the 1024 threads.
// One workgroup; deterministic for a given T.  Writes the reduced loss
// scale * sum (/ count) and the gradient scale of that reduction,
// scale (/ count); a mean over no tokens is 0 with gradient scale 0.
__global__ void __launch_bounds__(1024) loss_reduce_kernel(ReduceArgs a) {
  __shared__ double buf[1024];
  __shared__ int64_t cnt[1024];
  constexpr int U = 8;
  double p[U];
#pragma unroll
  for (int u = 0; u < U; ++u) p[u] = 0.0;
  int64_t c = 0;
  int64_t i = threadIdx.x;
  for (; i + (U - 1) * 1024 < a.T; i += U * 1024) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = a.loss[i + u * 1024];
    if (a.mean_valid) {
#pragma unroll
      for (int u = 0; u < U; ++u) c += a.y[i + u * 1024] != a.ignore_index ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) p[u] += (double)v[u];
  }
  for (int u = 0; i < a.T; i += 1024, ++u) {  // fewer than U left for this thread
    p[u] += (double)a.loss[i];
    if (a.mean_valid) c += a.y[i] != a.ignore_index ? 1 : 0;
  }
  const double s = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  buf[threadIdx.x] = s;
  cnt[threadIdx.x] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      buf[threadIdx.x] += buf[threadIdx.x + w];
      cnt[threadIdx.x] += cnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double scale = (double)a.scale;
    if (a.mean_valid) scale = cnt[0] > 0 ? scale / (double)cnt[0] : 0.0;
    if (a.out) *a.out = (float)(buf[0] * scale);
    if (a.g_out) *a.g_out = (float)scale;
  }
}

// dst = bf16(src), round to nearest even, 8 elements per thread and step.
__global__ void __launch_bounds__(256) cast_bf16_kernel(const float* src, __bf16* dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += stride) {
    if (i + 8 <= n) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src + i);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(src + i + 4);
      const bf16x8_t v = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                          (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
      *reinterpret_cast<bf16x8_t*>(dst + i) = v;
    } else {
      for (int64_t k = i; k < n; ++k) dst[k] = (__bf16)src[k];
    }
  }
}

// ================================================================ backward dZ
template <typename E>
__device__ __forceinline__ void store4(E* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  bf16x4_t v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  *reinterpret_cast<bf16x4_t*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
}

// Writes a finished bf16 dZ tile (vocab x token in the accumulators) to the
// token-major workspace through LDS, so that each store instruction covers
// whole 512-byte token rows instead of 32 scattered 8-byte pieces.  LDS holds
// the tile as [token][vocab] with its 8-byte granules XOR-swizzled by the
// token (granule g of row c sits at g ^ (c % 32)), which keeps both the
// 8-byte writes (32 tokens, one granule) and the 16-byte row reads free of
// bank conflicts.  Needs BN * BM * 2 bytes of LDS; the caller's mainloop has
// ended with a barrier.
template <typename TL>
__device__ __forceinline__ void store_dz_tile(const TL& tile, char* lds, __bf16* dz, int64_t ldz,
                                              int64_t vl0, int64_t ldz_cols, int64_t tl0,
                                              int64_t t_count, int wm, int wn) {
  static_assert(TL::BM == 256 && TL::ESZ == 2, "token rows of 512 bytes");
  static_assert(TL::BN * TL::BM * 2 <= TL::LDS_BYTES, "tile fits the mainloop's LDS");
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    const int c = TL::col_of(wn, j);
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int g = TL::row_of(wm, i, rq * 4) >> 2;
        bf16x4_t v = {(__bf16)tile.acc[i][j][rq * 4], (__bf16)tile.acc[i][j][rq * 4 + 1],
                      (__bf16)tile.acc[i][j][rq * 4 + 2], (__bf16)tile.acc[i][j][rq * 4 + 3]};
        *reinterpret_cast<bf16x4_t*>(lds + c * 512 + ((g ^ (c & 31)) << 3)) = v;
      }
  }
  __syncthreads();
  constexpr int kChunks = TL::BN * 32 / TL::NT;  // 16-byte chunks per thread
#pragma unroll
  for (int it = 0; it < kChunks; ++it) {
    const int idx = it * TL::NT + (int)threadIdx.x;
    const int c = idx >> 5, m = idx & 31, x = c & 31;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + c * 512 + ((m ^ (x >> 1)) << 4));
    if (x & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
    const int64_t vl = vl0 + 8 * m;
    if (tl0 + c < t_count && vl < ldz_cols)
      *reinterpret_cast<u32x4_t*>(dz + (tl0 + c) * ldz + vl) = v;
  }
}

// One 256 x 256 (vocab x token) tile of the block/slab: recompute logits,
// form dZ, write it token-major: dz[t_local * ldz + v_local].  Vocab rows past
// V inside the slab's last tile are written as zeros so the contractions can
// read whole 16-byte chunks.
template <typename E>
__device__ __forceinline__ void dz_tile(const DzArgs& a, int tm, int tn, char* lds) {
  using TL = typename LogitCfg<E>::T;
  constexpr int ESZ = TL::ESZ;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int64_t v0 = a.v_begin + (int64_t)tm * TL::BM;  // global vocab id of tile row 0
  const int64_t tl0 = (int64_t)tn * TL::BN;             // token within the block
  const int t_count = block_count(a.blk);
  if (tl0 >= t_count) return;

  Operand A, B;
  A.rows = (int)max<int64_t>(0, min<int64_t>(TL::BM, a.V - v0));
  A.rs = make_rsrc(reinterpret_cast<const char*>(a.W) + v0 * a.d * ESZ,
                   (uint32_t)((int64_t)A.rows * a.d * ESZ));  // W may pass 2^31 bytes
  A.off = 0;
  A.ld_bytes = (uint32_t)(a.d * ESZ);
  A.cols = a.d;
  B.rs = make_rsrc(a.Hc, clamp_bytes((int64_t)a.blk.t_max * a.d * ESZ));
  B.off = (uint32_t)(tl0 * a.d * ESZ);
  B.ld_bytes = (uint32_t)(a.d * ESZ);
  B.rows = (int)min<int64_t>(TL::BN, t_count - tl0);
  B.cols = a.d;

  TL tile;
  tile.zero();
  if (A.rows > 0) tile.mainloop(A, B, a.d, lds);

  // dZ = g * exp(z - lse) - g * [row == target]: with |g| folded into the
  // exponent, each element costs one FMA and one exp2:
  //   g * exp(z - lse) = sign(g) * exp2(z * log2(e) + (log2|g| - lse * log2(e))).
  // Ignored tokens get a -inf bias (exactly 0), invalid targets a NaN bias.
  const float g = a.g_dev ? *a.g_dev : a.grad_scale;
  const float gsign = g < 0.f ? -1.f : 1.f;
  const float log2g = g == 0.f ? kNegInf : __log2f(fabsf(g));
  const bool tail = v0 + TL::BM > a.V;  // last vocab tile: rows past V are zero
  const int lim = a.V - (int)v0 - wm * TL::WTM - 4 * (lane >> 5);
  E* dz = reinterpret_cast<E*>(a.dz);
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    const int c = TL::col_of(wn, j);
    const int64_t tl = tl0 + c;
    const bool col_ok = tl < t_count;
    const int64_t t = a.blk.idx[a.blk.t_begin + (col_ok ? tl : 0)];  // the token itself
    const int code = target_code(a.tg, t, a.V);
    const float lse_t = a.lse[t];
    const float bias = code == kIgnored ? kNegInf
                       : code == kInvalid ? __builtin_nanf("")
                                    : log2g - lse_t * kLog2e;
    // the sign of g is uniform: two copies of the loop keep it out of the
    // per-element work
    if (gsign > 0.f) {
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tile.acc[i][j][r] = fast_exp2(dz_arg<TL::ESZ>(tile.acc[i][j][r], lse_t, log2g, bias));
    } else {
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tile.acc[i][j][r] = -fast_exp2(dz_arg<TL::ESZ>(tile.acc[i][j][r], lse_t, log2g, bias));
    }
    // the one-hot term (rare: only the wave holding the target row)
    const int wrow0 = (int)v0 + wm * TL::WTM;
    if (code >= wrow0 && code < wrow0 + TL::WTM) {
      const int rt = code - wrow0 - 4 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rt == i * 32 + 8 * (r >> 2) + (r & 3)) tile.acc[i][j][r] -= g;
    }
    if (tail) {
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (i * 32 + 8 * (r >> 2) + (r & 3) >= lim) tile.acc[i][j][r] = 0.f;
    }
    if constexpr (ESZ == 4) {
      if (!col_ok) continue;
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int row0 = TL::row_of(wm, i, rq * 4);
          const int64_t vl = v0 - a.v_begin + row0;  // vocab within the slab
          if (vl < a.ldz_cols)
            store4<E>(dz + tl * a.ldz + vl, tile.acc[i][j][rq * 4], tile.acc[i][j][rq * 4 + 1],
                      tile.acc[i][j][rq * 4 + 2], tile.acc[i][j][rq * 4 + 3]);
        }
    }
  }
  if constexpr (ESZ == 2) store_dz_tile<TL>(tile, lds, dz, a.ldz, v0 - a.v_begin, a.ldz_cols,
                                            tl0, t_count, wm, wn);
}

template <typename E>
__global__ void __launch_bounds__(LogitCfg<E>::T::NT, 1) bwd_dz_kernel(DzArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const uint64_t tl_t0 = timeline_start();
  int tm, tn;
  if (!xcd_tile(blockIdx.x, a.n_vtiles, a.n_ttiles, 4, tm, tn)) return;
  dz_tile<E>(a, tm, tn, lds);
  timeline_end(kTimelineDz, tl_t0);
}

// ================================================================ backward dH
// dH[block] (+)= dZ[block, slab] * W[slab].  M = tokens, N = hidden, K = slab.
// mode: 0 = first slab of several (write fp32 acc), 1 = middle (acc += ),
// 2 = last of several (acc + partial -> dH in E), 3 = only slab (-> dH in E).
// (The K loop over a whole slab is long, so the epilogue's read of the
// partial costs little here; dW, with a short K loop, preloads instead.)
//
// The tile grid is (block tokens / BM) x (d / BN): 256 tiles for 8,192 tokens
// at d = 2,048, but fewer for smaller blocks, smaller d, or a block thinned
// by ignored tokens, which would leave compute units idle for the whole long
// K loop.  With a partial buffer (a.part) the kernel then cuts the slab's K
// range into S = kDhSplitSlots / tiles contiguous parts (whole k stages), one
// workgroup each, and stores each part's fp32 tile; bwd_dh_reduce_kernel sums
// the S parts in ascending order and applies the mode.  S is computed on the
// device from the block's token count, identically in both kernels.
constexpr int kDhSplitSlots = 256;  // partial tiles the buffer holds; also the CU count

template <typename TL>
__device__ __forceinline__ int dh_splits(const DhArgs& a, int act_m) {
  if (!a.part) return 1;
  const int tiles = act_m * a.n_ntiles;
  if (tiles <= 0) return 1;
  const int stages = (a.k_count + TL::BK - 1) / TL::BK;  // each part keeps at least one
  return max(1, min(kDhSplitSlots / tiles, stages));
}

// Part `sp` of S of the tile (tm, tn), as stored by the dH kernel: row-major
// [token column][hidden row] fp32, i.e. dH's own orientation, so that the
// reduce pass reads every part and writes the accumulator / dH rows
// contiguously; the dH kernel's stores are 16-byte quads of four hidden units.
template <typename TL>
__device__ __forceinline__ float* dh_part(const DhArgs& a, int act_m, int sp, int tm, int tn) {
  return a.part + ((int64_t)(sp * act_m + tm) * a.n_ntiles + tn) * (TL::BM * TL::BN);
}

// Applies the mode to four consecutive hidden units of token row tl of the
// block: v (+)= accumulator, then the accumulator or the token's dH row.
template <typename E>
__device__ __forceinline__ void dh_quad(const DhArgs& a, f32x4_t v, int64_t tl, int64_t n,
                                        int64_t t_row) {
  f32x4_t* accp = reinterpret_cast<f32x4_t*>(a.dh_acc + tl * a.d + n);
  if (a.mode == 1 || a.mode == 2) v += *accp;
  if (a.mode == 0 || a.mode == 1) {
    *accp = v;
  } else {
    E* out = reinterpret_cast<E*>(a.dH) + t_row * a.d + n;
    if constexpr (sizeof(E) == 2) {
      *reinterpret_cast<bf16x4_t*>(out) = bf16x4_t{(E)v[0], (E)v[1], (E)v[2], (E)v[3]};
    } else {
      *reinterpret_cast<f32x4_t*>(out) = v;
    }
  }
}

// The mode epilogue of one finished tile (hidden rows n0.. of the transposed
// tile, token columns tl0..): per token column one lookup of the token's own
// row, then 16-byte accesses of four consecutive hidden units.
template <typename E, typename TL>
__device__ __forceinline__ void dh_store(const DhArgs& a, const TL& tile, int64_t tl0, int64_t n0,
                                         int t_count) {
  const int wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    const int64_t tl = tl0 + TL::col_of(wn, j);  // token within the block
    if (tl >= t_count) continue;
    const int64_t t_row = a.mode >= 2 ? (int64_t)a.blk.idx[a.blk.t_begin + tl] : 0;
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // d is a multiple of 8 and n of 4: the four units are all in range or none
        const int64_t n = n0 + TL::row_of(wm, i, 4 * q);
        if (n >= a.d) continue;
        dh_quad<E>(a, f32x4_t{tile.acc[i][j][4 * q], tile.acc[i][j][4 * q + 1],
                              tile.acc[i][j][4 * q + 2], tile.acc[i][j][4 * q + 3]},
                   tl, n, t_row);
      }
  }
}

// One dH workgroup; `bid` is its index among the dH workgroups of the launch.
template <typename E>
__device__ __forceinline__ void dh_body(const DhArgs& a, int bid, char* lds) {
  using TL = typename DhCfg<E>::T;
  constexpr int ESZ = TL::ESZ;
  const int t_count = block_count(a.blk);
  const int act_m = (t_count + TL::BN - 1) / TL::BN;  // token tiles
  const int S = dh_splits<TL>(a, act_m);
  // split-major virtual token tiles: the workgroups an XCD runs together
  // share one part's W panels
  int tv, tn;
  if (!xcd_tile(bid, act_m * S, a.n_ntiles, 4, tv, tn)) return;
  const int sp = tv / act_m, tm = tv % act_m;
  const int64_t tl0 = (int64_t)tm * TL::BN;  // token within block
  const int64_t n0 = (int64_t)tn * TL::BM;   // hidden index
  const int stages = (a.k_count + TL::BK - 1) / TL::BK;
  const int k_lo = (int)((int64_t)stages * sp / S) * TL::BK;
  const int k_hi = min(a.k_count, (int)((int64_t)stages * (sp + 1) / S) * TL::BK);
  const int K = k_hi - k_lo;  // >= 1: S <= stages

  Operand A, B;
  // W rows of this part of the slab, based at the part's first row: the
  // planner keeps a slab's rows (K x d elements) below 2^31 bytes, so W
  // itself may be larger
  A.rs = make_rsrc(reinterpret_cast<const char*>(a.W) + (a.v_begin + k_lo) * a.d * ESZ,
                   clamp_bytes((int64_t)K * a.d * ESZ));
  A.off = (uint32_t)(n0 * ESZ);
  A.ld_bytes = (uint32_t)(a.d * ESZ);
  A.rows = K;
  A.cols = (int)min<int64_t>(TL::BM, a.d - n0);
  B.rs = make_rsrc(a.dz, clamp_bytes((int64_t)t_count * a.ldz * ESZ));
  B.off = (uint32_t)((tl0 * a.ldz + k_lo) * ESZ);
  B.ld_bytes = (uint32_t)(a.ldz * ESZ);
  B.rows = (int)min<int64_t>(TL::BN, t_count - tl0);
  B.cols = K;

  TL tile;
  tile.zero();
  __builtin_assume(K > 0);
  tile.mainloop(A, B, K, lds);

  if (S == 1) {
    dh_store<E>(a, tile, tl0, n0, t_count);
    return;
  }
  float* pt = dh_part<TL>(a, act_m, sp, tm, tn);
  const int wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    float* row = pt + TL::col_of(wn, j) * TL::BM;
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(row + TL::row_of(wm, i, 4 * q)) =
            f32x4_t{tile.acc[i][j][4 * q], tile.acc[i][j][4 * q + 1], tile.acc[i][j][4 * q + 2],
                    tile.acc[i][j][4 * q + 3]};
  }
}

// Sum of a split dH's parts in ascending part order, then the mode epilogue,
// as an elementwise pass over 16-byte quads (four consecutive hidden units of
// one token row): consecutive threads take consecutive quads of a token row,
// so the parts and the accumulator / dH rows are all accessed contiguously.
// Nothing to do when the dH kernel ran unsplit (S = 1).
template <typename E>
__global__ void __launch_bounds__(256) bwd_dh_reduce_kernel(DhArgs a) {
  using TL = typename DhCfg<E>::T;  // transposed tile: M = hidden, N = tokens
  const int t_count = block_count(a.blk);
  const int act_m = (t_count + TL::BN - 1) / TL::BN;
  const int S = dh_splits<TL>(a, act_m);
  if (S == 1) return;
  constexpr int kQuads = TL::BM * TL::BN / 4;  // quads per tile
  const int64_t n_units = (int64_t)act_m * a.n_ntiles * kQuads;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * 256) {
    const int tile = (int)(u / kQuads);
    const int e = (int)(u % kQuads) * 4;           // element of the row-major part
    const int c = e / TL::BM, m = e % TL::BM;      // token column, hidden row
    const int tm = tile / a.n_ntiles, tn = tile % a.n_ntiles;
    const int64_t tl = (int64_t)tm * TL::BN + c;
    const int64_t n = (int64_t)tn * TL::BM + m;
    // d is a multiple of 8 and n of 4: the four units are all in range or none
    if (tl >= t_count || n >= a.d) continue;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < S; ++sp)
      v += *reinterpret_cast<const f32x4_t*>(dh_part<TL>(a, act_m, sp, tm, tn) + e);
    const int64_t t_row = a.mode >= 2 ? (int64_t)a.blk.idx[a.blk.t_begin + tl] : 0;
    dh_quad<E>(a, v, tl, n, t_row);
  }
}

// ================================================================ backward dW
// dW[slab] (+)= dZ[block, slab]^T * H[block], computed as its transpose
// H[block]^T * dZ[block, slab]: M = hidden, N = slab vocab, K = block tokens,
// so that each lane's accumulator quads are four consecutive hidden units of
// one dW row (16-byte loads and stores).  accumulate: 0 = overwrite, 1 = add
// to dW (the MFMA accumulators start from the stored dW tile, so the
// epilogue only stores).
// One dW workgroup; `bid` is its index among the dW workgroups of the launch.
template <typename E>
__device__ __forceinline__ void dw_body(const DwArgs& a, int bid, char* lds) {
  using TL = typename DwCfg<E>::T;
  constexpr int ESZ = TL::ESZ;
  int tm, tn;
  if (!xcd_tile(bid, a.n_mtiles, a.n_ntiles, 8, tm, tn)) return;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int64_t n0 = (int64_t)tm * TL::BM;   // hidden
  const int64_t vl0 = (int64_t)tn * TL::BN;  // vocab within slab

  const int t_count = block_count(a.blk);  // K
  // the bf16 copy comes from the block whose dW is final
  __bf16* dwb = a.dW_bf16 != nullptr && last_filled_block(a.blk)
                    ? reinterpret_cast<__bf16*>(a.dW_bf16) + (a.v_begin + vl0) * a.d + n0
                    : nullptr;
  // nothing to add; an empty block that still owes the copy rewrites its
  // tile of dW unchanged below
  if (t_count == 0 && a.accumulate && dwb == nullptr) return;

  Operand A, B;
  A.rs = make_rsrc(a.Ht, clamp_bytes((int64_t)a.d * a.ldht * ESZ));
  A.off = (uint32_t)(n0 * a.ldht * ESZ);
  A.ld_bytes = (uint32_t)(a.ldht * ESZ);
  A.rows = (int)min<int64_t>(TL::BM, a.d - n0);
  A.cols = t_count;
  B.rs = make_rsrc(a.dz, clamp_bytes((int64_t)t_count * a.ldz * ESZ));
  B.off = (uint32_t)(vl0 * ESZ);
  B.ld_bytes = (uint32_t)(a.ldz * ESZ);
  B.rows = t_count;
  B.cols = (int)min<int64_t>(TL::BN, a.ldz - vl0);

  const int n_rows = (int)min<int64_t>(TL::BM, a.d - n0);  // a multiple of 8
  const int v_cols = (int)min<int64_t>(TL::BN, a.v_count - vl0);
  float* dw = a.dW + (a.v_begin + vl0) * a.d + n0;  // dW row = tile column
  TL tile;
  // token blocks after the first (or a caller's running sum) continue from dW
  if (a.accumulate)
    tile.load_acc_t(dw, a.d, n_rows, v_cols);
  else
    tile.zero();
  // An empty block (every token ignored) only overwrites with zeros.  Past
  // this branch the K loop runs at least once, which the compiler must know:
  // otherwise it keeps a spilled copy of the preloaded tile for a loop that
  // runs zero times.
  if (t_count > 0) {
    __builtin_assume(t_count > 0);
    tile.mainloop(A, B, t_count, lds);
  }

  // each lane holds four consecutive hidden units of one vocab row per quad
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    const int c = TL::col_of(wn, j);
    if (c >= v_cols) continue;
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = TL::row_of(wm, i, 4 * q);
        if (row < n_rows) {
          const f32x4_t v = {tile.acc[i][j][4 * q], tile.acc[i][j][4 * q + 1],
                             tile.acc[i][j][4 * q + 2], tile.acc[i][j][4 * q + 3]};
          *reinterpret_cast<f32x4_t*>(dw + (int64_t)c * a.d + row) = v;
          if (dwb != nullptr)
            *reinterpret_cast<bf16x4_t*>(dwb + (int64_t)c * a.d + row) =
                bf16x4_t{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        }
      }
  }
}

// dH and dW of one block and slab in a single launch: both only read the
// slab's dZ and write different outputs.  The dH workgroups come first, so the
// compute units that a partial last round of the long dH tiles leaves idle
// take the short dW tiles instead of waiting for the next launch.
template <typename E>
__global__ void __launch_bounds__(DhCfg<E>::T::NT, 1) bwd_dhdw_kernel(DhArgs h, DwArgs w,
                                                                     int dh_grid) {
  static_assert(DhCfg<E>::T::NT == DwCfg<E>::T::NT &&
                DhCfg<E>::T::LDS_BYTES == DwCfg<E>::T::LDS_BYTES, "one launch shape");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const uint64_t tl_t0 = timeline_start();
  if ((int)blockIdx.x < dh_grid) {
    dh_body<E>(h, blockIdx.x, lds);
    timeline_end(kTimelineDh, tl_t0);
  } else {
    dw_body<E>(w, blockIdx.x - dh_grid, lds);
    timeline_end(kTimelineDw, tl_t0);
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* p, int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = i0; i < n; i += stride) {
    if (i + 4 <= n) {
      *reinterpret_cast<f32x4_t*>(p + i) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
      for (int64_t k = i; k < n; ++k) p[k] = 0.f;
    }
  }
}

// ================================================================ compaction
// The backward skips ignored tokens: their dZ rows are zero, so they add
// nothing to dH or dW.  Three passes give a deterministic order: counts per
// chunk of kChunk tokens, an exclusive scan of the counts, then each chunk
// writes its non-ignored tokens (ascending) from its offset and its ignored
// ones after all non-ignored tokens.
constexpr int kChunk = 4096;  // tokens per workgroup: 256 threads x 16

__global__ void __launch_bounds__(256) compact_count_kernel(const int64_t* y, int64_t ignore,
                                                            int64_t T, int* cnt) {
  __shared__ int red[256];
  const int64_t t0 = (int64_t)blockIdx.x * kChunk + threadIdx.x * 16;
  int c = 0;
  for (int k = 0; k < 16; ++k) c += (t0 + k < T && y[t0 + k] != ignore) ? 1 : 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) cnt[blockIdx.x] = red[0];
}

// One workgroup: exclusive scan of n counts in place, the total into *tv.
__global__ void __launch_bounds__(1024) compact_scan_kernel(int* cnt, int64_t n, int* tv) {
  __shared__ int buf[1024];
  int carry = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int v = i < n ? cnt[i] : 0;
    buf[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
      const int add = (int)threadIdx.x >= o ? buf[threadIdx.x - o] : 0;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < n) cnt[i] = carry + buf[threadIdx.x] - v;
    carry += buf[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) *tv = carry;
}

__global__ void __launch_bounds__(256) compact_scatter_kernel(const int64_t* y, int64_t ignore,
                                                              int64_t T, const int* off,
                                                              const int* tv, int* idx) {
  __shared__ int buf[256];
  const int64_t t0 = (int64_t)blockIdx.x * kChunk + threadIdx.x * 16;
  unsigned valid = 0;
  int c = 0;
  for (int k = 0; k < 16; ++k)
    if (t0 + k < T && y[t0 + k] != ignore) {
      valid |= 1u << k;
      ++c;
    }
  buf[threadIdx.x] = c;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int add = (int)threadIdx.x >= o ? buf[threadIdx.x - o] : 0;
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  int64_t vpos = (int64_t)off[blockIdx.x] + buf[threadIdx.x] - c;  // valid tokens before t0
  int64_t ipos = *tv + (t0 - vpos);                                // ignored tokens before t0
  for (int k = 0; k < 16; ++k) {
    if (t0 + k >= T) break;
    if (valid >> k & 1u) idx[vpos++] = (int)(t0 + k);
    else idx[ipos++] = (int)(t0 + k);
  }
}

// Zeros the dH rows of the ignored tokens, 16 bytes per item.
template <typename E>
__global__ void __launch_bounds__(256) zero_rows_kernel(E* dH, const int* idx, const int* tv,
                                                        int64_t T, int d) {
  constexpr int CW = 16 / (int)sizeof(E);
  const int cpr = d / CW;
  const int64_t n = (T - *tv) * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t row = idx[*tv + i / cpr];
    *reinterpret_cast<u32x4_t*>(dH + row * d + (i % cpr) * CW) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// A token block of H gathered from the compacted order: Hc[r] = H[idx[t_begin
// + r]] and Ht[c][r] = Hc[r][c] for r < t_max (zero rows past the block's
// token count); 64 x 64 tiles through LDS, 16-byte loads and stores.
template <typename E>
__global__ void __launch_bounds__(256) gather_block_kernel(const E* H, TokBlock blk, int d, E* Hc,
                                                           E* Ht) {
  constexpr int CW = 16 / (int)sizeof(E);
  constexpr int CPR = 64 / CW;  // 16-byte chunks per tile row
  __shared__ E tile[64][64 + CW];
  const int count = block_count(blk);
  const int r0 = blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, ch = i % CPR;
    const int gc = c0 + ch * CW;
    if (r0 + r >= blk.t_max || gc >= d) continue;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r0 + r < count) {
      const int64_t t = blk.idx[blk.t_begin + r0 + r];
      v = *reinterpret_cast<const u32x4_t*>(H + t * d + gc);
    }
    *reinterpret_cast<u32x4_t*>(Hc + (int64_t)(r0 + r) * d + gc) = v;
    const E* e = reinterpret_cast<const E*>(&v);
#pragma unroll
    for (int k = 0; k < CW; ++k) tile[r][ch * CW + k] = e[k];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int c = i / CPR, ch = i % CPR;
    const int gc = c0 + c;
    const int gr = r0 + ch * CW;
    if (gc >= d || gr >= blk.t_max) continue;
    u32x4_t v;
    E* e = reinterpret_cast<E*>(&v);
#pragma unroll
    for (int k = 0; k < CW; ++k) e[k] = tile[ch * CW + k][c];
    *reinterpret_cast<u32x4_t*>(Ht + (int64_t)gc * blk.t_max + gr) = v;
  }
}

// ============================================================= token scoring
// One wave per token position: the lanes stride over 16-byte chunks of H[t]
// and of the token's W row (both rows read contiguously, 1 KB per wave
// instruction), multiply in fp32 (exact for bf16 inputs), and a fixed xor
// tree sums the wave.  Tokens outside [0, V) score NaN.
__device__ __forceinline__ float dot16(const u32x4_t& h, const u32x4_t& w, float acc, __bf16*) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(__builtin_bit_cast(float, h[q] << 16), __builtin_bit_cast(float, w[q] << 16), acc);
    acc = fmaf(__builtin_bit_cast(float, h[q] & 0xffff0000u),
               __builtin_bit_cast(float, w[q] & 0xffff0000u), acc);
  }
  return acc;
}
__device__ __forceinline__ float dot16(const u32x4_t& h, const u32x4_t& w, float acc, float*) {
  // whole-vector casts: a bit_cast of one element of a vector lvalue reads
  // element 0 with this compiler
  const f32x4_t hf = __builtin_bit_cast(f32x4_t, h), wf = __builtin_bit_cast(f32x4_t, w);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(hf[q], wf[q], acc);
  return acc;
}

// N gathered rows of one position at once: the loads of all N rows' chunks
// and of the position's H chunk are issued together, so a wave keeps
// (N + 1) x 16 bytes per lane per chunk step in flight instead of walking
// the rows one after another.  Each (lane, row) accumulates its chunks in
// ascending order, as for a single row; rows past `nk` or with an id outside
// the vocabulary read H's row instead and are not written.
template <typename E, int N>
__device__ __forceinline__ void token_logit_rows(const TokenArgs& a, int64_t t, int k0, int nk,
                                                 const char* h, float lse, int lane) {
  constexpr int CW = 16 / (int)sizeof(E);
  const int nc = a.d / CW;
  const char* w[N];
  bool ok[N];
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const int64_t v = r < nk ? a.tokens[t * a.K + k0 + r] : -1;
    ok[r] = v >= 0 && v < a.V;
    w[r] = ok[r] ? reinterpret_cast<const char*>(a.W) + v * a.d * (int64_t)sizeof(E) : h;
  }
  float acc[N];
#pragma unroll
  for (int r = 0; r < N; ++r) acc[r] = 0.f;
#pragma unroll 4
  for (int c = lane; c < nc; c += 64) {
    const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(h + (int64_t)c * 16);
    u32x4_t wv[N];
#pragma unroll
    for (int r = 0; r < N; ++r) wv[r] = *reinterpret_cast<const u32x4_t*>(w[r] + (int64_t)c * 16);
#pragma unroll
    for (int r = 0; r < N; ++r) acc[r] = dot16(hv, wv[r], acc[r], (E*)nullptr);
  }
#pragma unroll
  for (int r = 0; r < N; ++r) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[r] += __shfl_xor(acc[r], o);
    if (lane == 0 && r < nk) a.out[t * a.K + k0 + r] = ok[r] ? acc[r] - lse : __builtin_nanf("");
  }
}

template <typename E>
__global__ void __launch_bounds__(256) token_logit_kernel(TokenArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const char* h = reinterpret_cast<const char*>(a.H) + t * a.d * (int64_t)sizeof(E);
  const float lse = a.lse ? a.lse[t] : 0.f;
  for (int k0 = 0; k0 < a.K; k0 += 8) {
    const int nk = min(8, a.K - k0);
    if (nk == 1) token_logit_rows<E, 1>(a, t, k0, nk, h, lse, lane);
    else if (nk == 2) token_logit_rows<E, 2>(a, t, k0, nk, h, lse, lane);
    else if (nk <= 4) token_logit_rows<E, 4>(a, t, k0, nk, h, lse, lane);
    else token_logit_rows<E, 8>(a, t, k0, nk, h, lse, lane);
  }
}

// Target logits of the forward when its sweep is a pure log-sum-exp: one
// wave per token, zt[t] = H[t] . W[y_t - start] (fp32 products of the stored
// values, each lane's chunks in ascending order, then a fixed xor tree) for
// targets inside this vocab range; -inf for every other token (ignored,
// invalid, or held by another shard), which the merge never reads as a logit.
template <typename E>
__global__ void __launch_bounds__(256) target_logit_kernel(FwdArgs a) {
  constexpr int CW = 16 / (int)sizeof(E);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const int code = target_code(a.tg, t, a.V);
  if (code < 0) {
    if (lane == 0) a.zt[t] = kNegInf;
    return;
  }
  const char* h = reinterpret_cast<const char*>(a.H) + t * a.d * (int64_t)sizeof(E);
  const char* w = reinterpret_cast<const char*>(a.W) + (int64_t)code * a.d * (int64_t)sizeof(E);
  const int nc = a.d / CW;
  float acc = 0.f;
#pragma unroll 4
  for (int c = lane; c < nc; c += 64) {
    const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(h + (int64_t)c * 16);
    const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(w + (int64_t)c * 16);
    acc = dot16(hv, wv, acc, (E*)nullptr);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) a.zt[t] = acc;
}

// ================================================================== launchers
template <typename K, typename Args>
static hipError_t launch(K kernel, int grid, int threads, int lds, hipStream_t s, const Args& args) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, s, args);
  return hipGetLastError();
}

template <typename K>
static hipError_t set_lds(K kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <typename E, bool CAPTURE>
static hipError_t launch_sweep(const FwdArgs& a, int grid, hipStream_t s) {
  using TL = typename LogitCfg<E>::T;
  hipError_t e = set_lds(fwd_sweep_kernel<E, CAPTURE>, TL::LDS_BYTES);
  if (e != hipSuccess) return e;
  return launch(fwd_sweep_kernel<E, CAPTURE>, grid, TL::NT, TL::LDS_BYTES, s, a);
}

hipError_t launch_fwd_sweep(const FwdArgs& a, bool bf16, bool capture, int grid, hipStream_t s) {
  if (bf16) return capture ? launch_sweep<__bf16, true>(a, grid, s) : launch_sweep<__bf16, false>(a, grid, s);
  return capture ? launch_sweep<float, true>(a, grid, s) : launch_sweep<float, false>(a, grid, s);
}

hipError_t launch_target_logit(const FwdArgs& a, bool bf16, hipStream_t s) {
  const int grid = (int)((a.T + 3) / 4);
  if (bf16) return launch(target_logit_kernel<__bf16>, grid, 256, 0, s, a);
  return launch(target_logit_kernel<float>, grid, 256, 0, s, a);
}

hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t s) {
  return launch(fwd_merge_kernel, (int)((a.T + 255) / 256), 256, 0, s, a);
}

hipError_t launch_loss_reduce(const ReduceArgs& a, hipStream_t s) {
  return launch(loss_reduce_kernel, 1, 1024, 0, s, a);
}

hipError_t launch_cast_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n / 8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src,
                     reinterpret_cast<__bf16*>(dst), n);
  return hipGetLastError();
}

int64_t compact_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

hipError_t launch_compact(const int64_t* y, int64_t ignore_index, int64_t T, int* cnt, int* idx,
                          int* tv, hipStream_t s) {
  const int64_t n = compact_chunks(T);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_count_kernel, dim3((unsigned)n), dim3(256), 0, s, y, ignore_index, T,
                     cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, n, tv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_scatter_kernel, dim3((unsigned)n), dim3(256), 0, s, y, ignore_index,
                     T, (const int*)cnt, (const int*)tv, idx);
  return hipGetLastError();
}

hipError_t launch_zero_rows(void* dH, const int* idx, const int* tv, int64_t T, int d, bool bf16,
                            hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t items = T * (int64_t)(d / (bf16 ? 8 : 4));
  int64_t blocks = (items + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (bf16)
    hipLaunchKernelGGL(zero_rows_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<__bf16*>(dH), idx, tv, T, d);
  else
    hipLaunchKernelGGL(zero_rows_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<float*>(dH), idx, tv, T, d);
  return hipGetLastError();
}

hipError_t launch_gather_block(const void* H, const TokBlock& blk, int d, void* Hc, void* Ht,
                               bool bf16, hipStream_t s) {
  if (blk.t_max <= 0 || d <= 0) return hipSuccess;
  const dim3 grid((unsigned)((d + 63) / 64), (unsigned)((blk.t_max + 63) / 64));
  if (bf16)
    hipLaunchKernelGGL(gather_block_kernel<__bf16>, grid, dim3(256), 0, s,
                       reinterpret_cast<const __bf16*>(H), blk, d, reinterpret_cast<__bf16*>(Hc),
                       reinterpret_cast<__bf16*>(Ht));
  else
    hipLaunchKernelGGL(gather_block_kernel<float>, grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(H), blk, d, reinterpret_cast<float*>(Hc),
                       reinterpret_cast<float*>(Ht));
  return hipGetLastError();
}

hipError_t launch_token_logit(const TokenArgs& a, bool bf16, hipStream_t s) {
  const int grid = (int)((a.T + 3) / 4);
  if (bf16) return launch(token_logit_kernel<__bf16>, grid, 256, 0, s, a);
  return launch(token_logit_kernel<float>, grid, 256, 0, s, a);
}

hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t s) {
  return launch(shard_merge_kernel, (int)((a.T + 255) / 256), 256, 0, s, a);
}

hipError_t launch_bwd_dz(const DzArgs& a, bool bf16, hipStream_t s) {
  const int grid = xcd_grid(a.n_vtiles, a.n_ttiles);
  if (bf16) {
    using TL = LogitCfg<__bf16>::T;
    hipError_t e = set_lds(bwd_dz_kernel<__bf16>, TL::LDS_BYTES);
    if (e != hipSuccess) return e;
    return launch(bwd_dz_kernel<__bf16>, grid, TL::NT, TL::LDS_BYTES, s, a);
  }
  using TL = LogitCfg<float>::T;
  hipError_t e = set_lds(bwd_dz_kernel<float>, TL::LDS_BYTES);
  if (e != hipSuccess) return e;
  return launch(bwd_dz_kernel<float>, grid, TL::NT, TL::LDS_BYTES, s, a);
}

template <typename E>
static int dh_grid(const DhArgs& a) {
  int tiles = a.n_mtiles * a.n_ntiles;
  if (a.part && tiles < kDhSplitSlots) tiles = kDhSplitSlots;
  return xcd_grid(tiles, 1);
}

template <typename E>
static hipError_t launch_dhdw(const DhArgs& h, const DwArgs& w, hipStream_t s) {
  using TL = typename DhCfg<E>::T;
  hipError_t e = set_lds(bwd_dhdw_kernel<E>, TL::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int gh = dh_grid<E>(h);
  const int gw = xcd_grid(w.n_mtiles, w.n_ntiles);
  if (gh + gw <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dhdw_kernel<E>, dim3(gh + gw), dim3(TL::NT), TL::LDS_BYTES, s, h, w, gh);
  return hipGetLastError();
}

hipError_t launch_bwd_dhdw(const DhArgs& h, const DwArgs& w, bool bf16, hipStream_t s) {
  return bf16 ? launch_dhdw<__bf16>(h, w, s) : launch_dhdw<float>(h, w, s);
}

template <typename E>
static hipError_t launch_dh_reduce(const DhArgs& a, hipStream_t s) {
  using TL = typename DhCfg<E>::T;
  // grid-stride over the full block's tiles (the device's count is smaller
  // or equal); 8 workgroups of 256 threads per compute unit at most
  const int64_t units = (int64_t)a.n_mtiles * a.n_ntiles * (TL::BM * TL::BN / 4);
  const int64_t blocks = (units + 255) / 256;
  return launch(bwd_dh_reduce_kernel<E>, (int)(blocks < 2048 ? blocks : 2048), 256, 0, s, a);
}

hipError_t launch_bwd_dh_reduce(const DhArgs& a, bool bf16, hipStream_t s) {
  if (!a.part) return hipSuccess;
  return bf16 ? launch_dh_reduce<__bf16>(a, s) : launch_dh_reduce<float>(a, s);
}

int dh_split_slots() { return kDhSplitSlots; }

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// ========================================================= workgroup timeline
hipError_t timeline_reset() {
#if FLCE_TIMELINE
  const unsigned zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_timeline_n), &zero, sizeof zero);
#else
  return hipErrorNotSupported;
#endif
}

hipError_t timeline_read(TimelineRecord* out, int max_records, int* n_out) {
#if FLCE_TIMELINE
  *n_out = 0;
  hipError_t e = hipDeviceSynchronize();
  unsigned n = 0;
  if (e == hipSuccess) e = hipMemcpyFromSymbol(&n, HIP_SYMBOL(g_timeline_n), sizeof n);
  if (e != hipSuccess) return e;
  if (n > kTimelineCap) n = kTimelineCap;  // the count runs on past a full buffer
  if (max_records < 0) max_records = 0;
  if (n > (unsigned)max_records) n = (unsigned)max_records;
  if (n > 0) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_timeline), (size_t)n * sizeof(TimelineRecord));
  if (e == hipSuccess) *n_out = (int)n;
  return e;
#else
  (void)out;
  (void)max_records;
  *n_out = 0;
  return hipErrorNotSupported;
#endif
}

// ============================================================= scratch array
// The workspace of the allocation-free entry point (for callers that cannot
// allocate device memory).  Static device memory: every GPU that runs the
// library holds its own copy until the process ends.  In host code the
// array's name is only a stand-in for the device symbol, never an address:
// scratch_address() looks the device address up once per device, with that
// device current, and every use goes through that address.
constexpr uint64_t kScratchBytes = 256ull << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

uint64_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

TileInfo tile_info(bool bf16) {
  TileInfo t;
  if (bf16) {
    t.logit_bm = LogitCfg<__bf16>::T::BM;
    t.logit_bn = LogitCfg<__bf16>::T::BN;
    t.dh_bm = DhCfg<__bf16>::T::BN;  // tokens (the transposed tile's N)
    t.dh_bn = DhCfg<__bf16>::T::BM;  // hidden
    t.dw_bm = DwCfg<__bf16>::T::BM;
    t.dw_bn = DwCfg<__bf16>::T::BN;
    t.dh_bk = DhCfg<__bf16>::T::BK;
  } else {
    t.logit_bm = LogitCfg<float>::T::BM;
    t.logit_bn = LogitCfg<float>::T::BN;
    t.dh_bm = DhCfg<float>::T::BN;
    t.dh_bn = DhCfg<float>::T::BM;
    t.dw_bm = DwCfg<float>::T::BM;
    t.dw_bn = DwCfg<float>::T::BN;
    t.dh_bk = DhCfg<float>::T::BK;
  }
  return t;
}

}  // namespace flce
