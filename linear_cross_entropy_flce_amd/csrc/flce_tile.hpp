// flce_tile.hpp -- MFMA tile engine for gfx950 (CDNA4), shared by every kernel.
//
// C[BM x BN] += A[BM x K] * B[K x BN] for one workgroup tile, with bf16 or fp32
// operands and fp32 accumulation in MFMA accumulators.
//
// Operand storage (in HBM) is either
//   K-contiguous  ("KC"): element (r, k) at base + r*ld + k, or
//   MN-contiguous ("MC"): element (r, k) at base + k*ld + r,
// where r is the tile's M (for A) or N (for B) index.  The library needs both:
// the forward and the logit recompute contract H and W over the hidden axis
// (both KC), while dH = dZ W contracts W over the vocab axis and
// dW = dZ^T H contracts H and dZ over the token axis (MC).
//
// Global -> LDS: each thread moves 16-byte chunks through registers, one
// k-tile ahead of the MFMA work (LDS double buffer, one barrier per k-tile).
//   KC tiles are stored [row][128 bytes of k] with the 16-byte chunk index
//   XOR-swizzled by (row & 7) so that the 32 lanes reading one MFMA fragment
//   column hit distinct banks.
//   MC tiles are stored [k][row] with a 64-byte row pad, and fragments are read
//   with ds_read_b64_tr_b16 (bf16), the gfx950 LDS transpose read: within each
//   16-lane group, lanes 4s..4s+3 fetch 16 consecutive elements of one LDS row
//   and lane j receives element j of each of those four rows.  Two such reads
//   give a lane the 8 consecutive k values an MFMA operand needs.
//
// MFMA: v_mfma_f32_32x32x16_bf16 (bf16) or four v_mfma_f32_32x32x2_f32 (fp32).
// Lane l supplies row (l % 32) and the k values 8*(l/32)..+7 (bf16; fp32:
// 4*(l/32)..+3, one per MFMA); accumulator register r of lane l holds
// C[8*(r/4) + 4*(l/32) + (r%4)][l % 32] of each 32x32 block.  Any fixed k
// order works as long as A and B agree, which both read paths guarantee.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FLCE_LDS_PTR(T) __attribute__((address_space(3))) T*

// Buffer resource word 3 for gfx9-family buffer loads (raw, 32-bit format).
constexpr int kBufferFlags = 0x00020000;
// An offset beyond every resource's num_records: the load returns zeros.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          kBufferFlags);
}

__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
}

// A runtime description of one operand of one workgroup tile.
struct Operand {
  const char* base;   // KC: row 0 of the tile, k = 0.  MC: k = 0, first tile column.
  uint32_t ld_bytes;  // distance between consecutive rows in memory, in bytes
  uint32_t bytes;     // bytes readable from base (guards every load)
  int rows;           // KC: valid tile rows (M or N) from base.  MC: valid k rows (K).
  int cols;           // KC: K in elements.                        MC: valid tile columns.
};

template <typename E>
struct ElemTraits;
template <>
struct ElemTraits<__bf16> {
  static constexpr int kBytes = 2;
};
template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
};

template <int BM_, int BN_, int WM_, int WN_, typename E, bool A_KC, bool B_KC>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;       // threads per workgroup
  static constexpr int ESZ = ElemTraits<E>::kBytes;
  static constexpr int CW = 16 / ESZ;           // elements per 16-byte chunk
  static constexpr int BK = 128 / ESZ;          // k per LDS stage (128 bytes)
  static constexpr int KSTEP = 2 * CW;          // k per fragment step
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int A_PITCH = BM * ESZ + 64;  // MC LDS row pitch (bytes)
  static constexpr int B_PITCH = BN * ESZ + 64;
  static constexpr int A_BYTES = A_KC ? BM * 128 : BK * A_PITCH;
  static constexpr int B_BYTES = B_KC ? BN * 128 : BK * B_PITCH;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int A_LD = BM * BK / CW / NT;  // 16-byte loads per thread per stage
  static constexpr int B_LD = BN * BK / CW / NT;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32-aligned");
  static_assert((BM * BK / CW) % NT == 0 && (BN * BK / CW) % NT == 0, "loads must divide");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  f32x16_t acc[MI][NI];
  u32x4_t ra[A_LD], rb[B_LD];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // ---------------------------------------------------------------- global
  template <bool KC, int ROWS, int NLD>
  __device__ __forceinline__ static void gload(const Operand& op, __amdgpu_buffer_rsrc_t rs,
                                               int k0, u32x4_t* r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + NT * i;
      uint32_t off;
      if constexpr (KC) {
        const int row = c >> 3, kc = c & 7;
        const int k = k0 + kc * CW;
        off = (row < op.rows && k < op.cols) ? (uint32_t)row * op.ld_bytes + (uint32_t)k * ESZ
                                             : kOOB;
      } else {
        constexpr int CPR = ROWS * ESZ / 16;  // chunks per LDS row
        const int kr = c / CPR, cc = c % CPR;
        const int k = k0 + kr;
        off = (k < op.rows && cc * CW < op.cols) ? (uint32_t)k * op.ld_bytes + (uint32_t)cc * 16
                                                 : kOOB;
      }
      r[i] = buffer_load16(rs, off);
    }
  }

  template <bool KC, int ROWS, int PITCH, int NLD>
  __device__ __forceinline__ static void lstore(char* lds, const u32x4_t* r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + NT * i;
      int off;
      if constexpr (KC) {
        const int row = c >> 3, kc = c & 7;
        off = row * 128 + ((kc ^ (row & 7)) << 4);
      } else {
        constexpr int CPR = ROWS * ESZ / 16;
        off = (c / CPR) * PITCH + (c % CPR) * 16;
      }
      *reinterpret_cast<u32x4_t*>(lds + off) = r[i];
    }
  }

  // --------------------------------------------------------------- fragments
  // KC: lane reads its row's 16-byte chunk (2*ks + half) of the 128-byte k row.
  __device__ __forceinline__ static u32x4_t frag_kc(const char* lds, int row0, int ks) {
    const int lane = threadIdx.x & 63;
    const int row = row0 + (lane & 31);
    const int chunk = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const u32x4_t*>(lds + row * 128 + ((chunk ^ (row & 7)) << 4));
  }

  // MC, bf16: two transpose reads give k = 16*ks + 8*half + 0..7 of column row0 + lane%32.
  template <int PITCH>
  __device__ __forceinline__ static u32x4_t frag_mc_bf16(const char* lds, int row0, int ks) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i = lane & 15;
    const int col = row0 + 16 * (g & 1) + 4 * (i & 3);
    const int k = ks * 16 + 8 * (g >> 1) + (i >> 2);
    const char* p0 = lds + k * PITCH + col * 2;
    const char* p1 = p0 + 4 * PITCH;
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FLCE_LDS_PTR(i16x4_t))(p0));
    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FLCE_LDS_PTR(i16x4_t))(p1));
    u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
    u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }

  // MC, fp32: four scalar reads give k = 8*ks + 4*half + 0..3 of column row0 + lane%32.
  template <int PITCH>
  __device__ __forceinline__ static u32x4_t frag_mc_f32(const char* lds, int row0, int ks) {
    const int lane = threadIdx.x & 63;
    const int col = row0 + (lane & 31);
    const int k = ks * 8 + 4 * (lane >> 5);
    const char* p = lds + k * PITCH + col * 4;
    u32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint32_t*>(p + q * PITCH);
    return v;
  }

  __device__ __forceinline__ static void mma(f32x16_t& c, u32x4_t a, u32x4_t b) {
    if constexpr (ESZ == 2) {
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
      // bit-cast whole vectors: a bit cast of a vector element (a[q]) reads
      // element 0 with this compiler
      const f32x4_t af = __builtin_bit_cast(f32x4_t, a);
      const f32x4_t bf = __builtin_bit_cast(f32x4_t, b);
#pragma unroll
      for (int q = 0; q < 4; ++q) c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[q], bf[q], c, 0, 0, 0);
    }
  }

  __device__ __forceinline__ void compute_stage(const char* la, const char* lb, int wm, int wn) {
#pragma unroll
    for (int ks = 0; ks < BK / KSTEP; ++ks) {
      u32x4_t fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r0 = wm * WTM + i * 32;
        if constexpr (A_KC) fa[i] = frag_kc(la, r0, ks);
        else if constexpr (ESZ == 2) fa[i] = frag_mc_bf16<A_PITCH>(la, r0, ks);
        else fa[i] = frag_mc_f32<A_PITCH>(la, r0, ks);
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r0 = wn * WTN + j * 32;
        if constexpr (B_KC) fb[j] = frag_kc(lb, r0, ks);
        else if constexpr (ESZ == 2) fb[j] = frag_mc_bf16<B_PITCH>(lb, r0, ks);
        else fb[j] = frag_mc_f32<B_PITCH>(lb, r0, ks);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
  }

  // Full K loop for one tile: acc += A * B.  `lds` holds LDS_BYTES.  Ends with a
  // barrier, so the caller may reuse LDS (or start another tile) right away.
  __device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int K, char* lds) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(A.base, A.bytes);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(B.base, B.bytes);
    const int nk = (K + BK - 1) / BK;
    if (nk <= 0) return;
    gload<A_KC, BM, A_LD>(A, rsa, 0, ra);
    gload<B_KC, BN, B_LD>(B, rsb, 0, rb);
    lstore<A_KC, BM, A_PITCH, A_LD>(lds, ra);
    lstore<B_KC, BN, B_PITCH, B_LD>(lds + A_BYTES, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = lds + (kt & 1) * STAGE;
      char* nxt = lds + ((kt + 1) & 1) * STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        gload<A_KC, BM, A_LD>(A, rsa, (kt + 1) * BK, ra);
        gload<B_KC, BN, B_LD>(B, rsb, (kt + 1) * BK, rb);
      }
      compute_stage(cur, cur + A_BYTES, wm, wn);
      if (more) {
        lstore<A_KC, BM, A_PITCH, A_LD>(nxt, ra);
        lstore<B_KC, BN, B_PITCH, B_LD>(nxt + A_BYTES, rb);
      }
      __syncthreads();
    }
  }

  // Row (within the workgroup tile) of accumulator register r of block (i, *).
  __device__ __forceinline__ static int row_of(int wm, int i, int r) {
    const int lane = threadIdx.x & 63;
    return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ __forceinline__ static int col_of(int wn, int j) {
    const int lane = threadIdx.x & 63;
    return wn * WTN + j * 32 + (lane & 31);
  }
};

// Workgroup -> tile mapping that keeps the workgroups co-resident on one XCD
// (consecutive workgroup ids are dealt round-robin over the 8 XCDs, each with
// its own L2) on a compact block of tiles: XCD x takes a contiguous range of
// tile ids, and ids are rastered in column strips `group` tiles tall, so the
// ~32 workgroups an XCD runs at once share a few A and B panels in its L2.
// Returns false for the few padding workgroups past the last tile.
__device__ __forceinline__ bool xcd_tile(int bid, int nm, int nn, int group, int& tm, int& tn) {
  const int total = nm * nn;
  const int per = (total + 7) / 8;
  const int id = (bid & 7) * per + (bid >> 3);
  if (id >= total) return false;
  const int span = group * nn;
  const int g = id / span, w = id % span;
  const int m0 = g * group;
  const int gs = min(nm - m0, group);
  tm = m0 + w % gs;
  tn = w / gs;
  return true;
}

__host__ __device__ inline int xcd_grid(int nm, int nn) { return ((nm * nn + 7) / 8) * 8; }

}  // namespace flce
