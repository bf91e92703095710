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
// Global -> LDS, three loaders (one barrier per stage each):
//   - register-staged double buffer (DMA = false, NS = 2; what every kernel
//     uses): buffer_load_dwordx4 into VGPRs 1.5 stages ahead, ds_write into
//     the other LDS stage, with an explicit MFMA / LDS / global-load
//     interleave in the branch-free steady state;
//   - two-stage direct DMA (buffer_load_dwordx4 ... lds, no VGPR staging);
//   - a DMA ring of NS > 2 stages running NS - 1 stages ahead.
// LDS layouts, the same for all three:
//   KC tiles are stored [row][KB bytes of k] with the 16-byte chunk index
//   XOR-swizzled so that the lanes reading one MFMA fragment column hit
//   distinct banks.
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

// A runtime description of one operand of one workgroup tile.  `rs` covers the
// rows the tile reads (based at the tile's first row, or at the first row of
// the vocab slab part it contracts over), always below 2 GiB, so 32-bit byte
// offsets reach all of it and kOOB stays beyond every resource; `off` is the
// byte offset of the tile origin inside it.
struct Operand {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off;       // KC: row 0 of the tile, k = 0.  MC: k = 0, first tile column.
  uint32_t ld_bytes;  // distance between consecutive rows in memory, in bytes
  int rows;           // KC: valid tile rows (M or N).  MC: valid k rows (K).
  int cols;           // KC: K in elements.             MC: valid tile columns.
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

template <int BM_, int BN_, int WM_, int WN_, typename E, bool A_KC, bool B_KC, int KB_ = 64,
          int NS_ = 3, bool DMA_ = true>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN;             // waves per workgroup
  static constexpr int NT = NW * 64;             // threads per workgroup
  static constexpr int ESZ = ElemTraits<E>::kBytes;
  static constexpr int CW = 16 / ESZ;            // elements per 16-byte chunk
  static constexpr int KB = KB_;                 // bytes of k per KC row per stage
  static constexpr int NS = NS_;                 // LDS ring stages (2 without DMA)
  static constexpr bool DMA = DMA_;              // global -> LDS by DMA, else through VGPRs
  static constexpr bool kAKC = A_KC, kBKC = B_KC;  // operand layouts
  static constexpr int BK = KB / ESZ;            // k per stage
  static constexpr int KSTEP = 2 * CW;           // k per fragment step
  static constexpr int KS = BK / KSTEP;          // fragment steps per stage
  static constexpr int CPR = KB / 16;            // 16-byte chunks per KC row
  static constexpr int RPB = 1024 / KB;          // KC rows per 1 KB DMA block
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int A_PITCH = BM * ESZ + 64;  // MC LDS row pitch (bytes)
  static constexpr int B_PITCH = BN * ESZ + 64;
  static constexpr int A_NB = A_KC ? BM * KB / 1024 : (BK * A_PITCH + 1023) / 1024;  // DMA blocks
  static constexpr int B_NB = B_KC ? BN * KB / 1024 : (BK * B_PITCH + 1023) / 1024;
  static constexpr int A_BYTES = A_NB * 1024;
  static constexpr int B_BYTES = B_NB * 1024;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NS * STAGE;
  static constexpr int A_J = (A_NB + NW - 1) / NW;  // DMA instructions per wave (upper bound)
  static constexpr int B_J = (B_NB + NW - 1) / NW;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32-aligned");
  static_assert(KS >= 1 && BK % KSTEP == 0, "stage must hold whole fragment steps");
  static_assert(KB == 64 || KB == 128, "KC rows of 64 or 128 bytes");
  static_assert(DMA ? NS >= 2 : NS == 2, "DMA ring of >= 2 stages, or a register-staged double buffer");
  static constexpr int A_LD = BM * BK / CW / NT;  // 16-byte loads per thread per stage (no DMA)
  static constexpr int B_LD = BN * BK / CW / NT;
  static_assert(DMA || ((BM * BK / CW) % NT == 0 && (BN * BK / CW) % NT == 0), "loads must divide");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  f32x16_t acc[MI][NI];

  // acc = C[tile] for a matrix stored transposed: tile element (row, col) is
  // c[col * ldc + row], with `rows` x `cols` of the tile valid and `rows` a
  // multiple of 4.  Each lane's four consecutive rows are one 16-byte load;
  // the row offsets of the (i, quad) blocks are immediates on one per-column
  // address register.  The buffer resource ends at the last valid element, so
  // columns past `cols` read as 0.
  __device__ __forceinline__ void load_acc_t(const float* c, int64_t ldc, int rows, int cols) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t bytes = rows > 0 && cols > 0 ? ((int64_t)(cols - 1) * ldc + rows) * 4 : 0;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(c, (uint32_t)(bytes > 0x7fffffff ? 0x7fffffff : bytes));
    const uint32_t ld4 = (uint32_t)ldc * 4u;
    const int row0 = wm * WTM + 4 * (lane >> 5);  // this lane's first row
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const uint32_t vo = (uint32_t)col_of(wn, j) * ld4 + (uint32_t)row0 * 4u;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dr = i * 32 + 8 * q;
          const uint32_t off = rows >= BM || row0 + dr < rows ? vo + (uint32_t)dr * 4u : kOOB;
          const f32x4_t v = __builtin_bit_cast(f32x4_t, buffer_load16(rs, off));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = v[e];
        }
    }
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // Chunk swizzle of the KC layout: the 16 rows read by 16 lanes at one
  // logical chunk land in 16 distinct 16-byte bank groups of the 64 x 4-byte
  // LDS banks (256 / KB rows share one bank window).
  __device__ __forceinline__ static int swz(int row) { return (row / (256 / KB)) % CPR; }

  // ------------------------------------------------------ global -> LDS (DMA)
  // One buffer_load_dwordx4 ... lds moves 64 x 16 bytes into a contiguous
  // 1 KB block of LDS (lane l -> byte 16 l).  Each lane picks the global chunk
  // that belongs at its slot, so the swizzled / padded layouts come for free.
  // Blocks are dealt round-robin over the waves.
  struct Dma {
    uint32_t off[A_J + B_J];  // byte offset from the operand base at k0 = 0
    int krel[A_J + B_J];      // KC: k of the chunk;  MC: k row within the stage
    bool ok[A_J + B_J];       // the slot is inside the operand (row / column bounds)
  };

  template <bool KC, int ROWS, int PITCH, int NB, int J>
  __device__ __forceinline__ static void dma_setup(const Operand& op, int wave, uint32_t* off,
                                                   int* krel, bool* ok) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int b = wave + NW * j;
      if constexpr (KC) {
        const int row = b * RPB + lane / CPR;
        const int kc = (lane % CPR) ^ swz(row);
        off[j] = op.off + (uint32_t)row * op.ld_bytes + (uint32_t)kc * 16;
        krel[j] = kc * CW;
        ok[j] = b < NB && row < op.rows;
      } else {
        const int o = b * 1024 + 16 * lane;
        const int kr = o / PITCH, cb = o % PITCH;
        off[j] = op.off + (uint32_t)kr * op.ld_bytes + (uint32_t)cb;
        krel[j] = kr;
        ok[j] = b < NB && kr < BK && cb < ROWS * ESZ && (cb / 16) * CW < op.cols;
      }
    }
  }

  template <bool KC, int NB, int J>
  __device__ __forceinline__ static void dma_issue(const Operand& op, int wave, int k0, char* dst,
                                                   const uint32_t* off, const int* krel,
                                                   const bool* ok) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int b = wave + NW * j;
      if (J * NW == NB || b < NB) {
        bool v;
        uint32_t o;
        if constexpr (KC) {
          v = ok[j] && k0 + krel[j] < op.cols;
          o = off[j] + (uint32_t)k0 * ESZ;
        } else {
          v = ok[j] && k0 + krel[j] < op.rows;
          o = off[j] + (uint32_t)k0 * op.ld_bytes;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            op.rs, (__attribute__((address_space(3))) void*)(dst + b * 1024), 16, v ? o : kOOB, 0,
            0, 0);
      }
    }
  }

  // ------------------------------------------- global -> VGPR -> LDS staging
  // Thread c of the workgroup moves chunk c, c + NT, ... of the stage: KC rows
  // are CPR chunks wide, MC rows ROWS * ESZ / 16 chunks.
  template <bool KC, int ROWS, int NLD>
  __device__ __forceinline__ static void gload(const Operand& op, int k0, u32x4_t* r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + NT * i;
      uint32_t off;
      if constexpr (KC) {
        const int row = c / CPR, kc = c % CPR;
        const int k = k0 + kc * CW;
        off = (row < op.rows && k < op.cols)
                  ? op.off + (uint32_t)row * op.ld_bytes + (uint32_t)k * ESZ
                  : kOOB;
      } else {
        constexpr int RC = ROWS * ESZ / 16;
        const int kr = c / RC, cc = c % RC;
        const int k = k0 + kr;
        off = (k < op.rows && cc * CW < op.cols)
                  ? op.off + (uint32_t)k * op.ld_bytes + (uint32_t)cc * 16
                  : kOOB;
      }
      r[i] = buffer_load16(op.rs, off);
    }
  }

  // Per-thread part of gload's offsets, fixed for the whole K loop: the
  // tile-relative byte offset of each of this thread's chunks at k0 = 0, or
  // kOOB when the chunk's row (KC) / column (MC) lies outside the operand.
  // The stage's k then enters as the instruction's scalar offset, so a full
  // stage costs no vector arithmetic; `kk` keeps each chunk's k (KC: element
  // offset in the row, MC: row in the stage) for the partial last stage.
  template <bool KC, int ROWS, int NLD>
  __device__ __forceinline__ static void gprep(const Operand& op, uint32_t* voff, int* kk) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + NT * i;
      if constexpr (KC) {
        const int row = c / CPR, kc = c % CPR;
        voff[i] = row < op.rows ? op.off + (uint32_t)row * op.ld_bytes + (uint32_t)kc * 16 : kOOB;
        kk[i] = kc * CW;
      } else {
        constexpr int RC = ROWS * ESZ / 16;
        const int kr = c / RC, cc = c % RC;
        voff[i] = cc * CW < op.cols ? op.off + (uint32_t)kr * op.ld_bytes + (uint32_t)cc * 16 : kOOB;
        kk[i] = kr;
      }
    }
  }

  // Loads of the stage starting at k0.  `full`: the whole stage lies below K.
  template <bool KC, int NLD>
  __device__ __forceinline__ static void gload_fast(const Operand& op, const uint32_t* voff,
                                                    const int* kk, int k0, bool full, u32x4_t* r) {
    const int kmax = KC ? op.cols : op.rows;  // K
    const uint32_t soff = KC ? (uint32_t)k0 * ESZ : (uint32_t)k0 * op.ld_bytes;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const uint32_t v = (full || k0 + kk[i] < kmax) ? voff[i] : kOOB;
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(op.rs, v, soff, 0);
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
        const int row = c / CPR, kc = c % CPR;
        off = row * KB + ((kc ^ swz(row)) << 4);
      } else {
        constexpr int RC = ROWS * ESZ / 16;
        off = (c / RC) * PITCH + (c % RC) * 16;
      }
      *reinterpret_cast<u32x4_t*>(lds + off) = r[i];
    }
  }

  // --------------------------------------------------------------- fragments
  // KC: lane reads chunk (2*ks + half) of its row.
  __device__ __forceinline__ static u32x4_t frag_kc(const char* lds, int row0, int ks) {
    const int lane = threadIdx.x & 63;
    const int row = row0 + (lane & 31);
    const int chunk = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const u32x4_t*>(lds + row * KB + ((chunk ^ swz(row)) << 4));
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

  // Fragments of one k step (KSTEP k values) for this wave's MI x NI blocks.
  __device__ __forceinline__ static void read_frags(const char* la, const char* lb, int wm, int wn,
                                                    int ks, u32x4_t* fa, u32x4_t* fb) {
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
  }

  __device__ __forceinline__ void mma_all(const u32x4_t* fa, const u32x4_t* fb) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) mma(acc[i][j], fa[i], fb[j]);
  }

  // Waits until at most n of this wave's vector-memory operations (here: the
  // LDS DMA loads) are outstanding.  n is wave-uniform and small.
  __device__ __forceinline__ static void wait_vm(int n) {
    switch (n) {
      // gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4 and lgkmcnt 11:8 left at max
      case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
      case 1: __builtin_amdgcn_s_waitcnt(0x0f71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0x0f72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0x0f73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0f75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0x0f76); break;
      case 7: __builtin_amdgcn_s_waitcnt(0x0f77); break;
      case 8: __builtin_amdgcn_s_waitcnt(0x0f78); break;
      default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    }
  }

  // Full K loop for one tile: acc += A * B.  `lds` holds LDS_BYTES.  Ends with a
  // barrier, so the caller may reuse LDS (or start another tile) right away.
  //
  // LDS ring of NS stages filled by DMA, NS - 1 stages ahead of the MFMA work:
  //   iteration kt: wait until stages kt and kt+1 have landed (this wave's
  //   DMA count), barrier (they are then visible to every wave, and every
  //   wave is done with stage kt-1), issue the DMA of stage kt+NS-1 into the
  //   slot of kt-1, then run KS fragment steps on stage kt with fragments
  //   double-buffered in registers; the last step already reads the first
  //   fragments of stage kt+1.
  __device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int K, char* lds) {
    if constexpr (DMA && NS == 2) mainloop_dma2(A, B, K, lds);
    else if constexpr (DMA) mainloop_dma(A, B, K, lds);
    else mainloop_regs(A, B, K, lds);
  }

  // DMA into two LDS stages.  Stage kt + 1 is in flight while stage kt is
  // consumed; after stage kt's last MFMAs: wait for this wave's share of
  // stage kt + 1, barrier (every share landed, every wave done with stage
  // kt), issue stage kt + 2 into stage kt's slot, read kt + 1's first
  // fragments.  The stage's k offset travels in the scalar offset; a chunk's
  // k bound is only checked on a partial last stage.
  template <bool KC, int NB, int J>
  __device__ __forceinline__ static void dma_issue2(const Operand& op, int wave, int k0, bool full,
                                                    char* dst, const uint32_t* off,
                                                    const int* krel, const bool* ok) {
    const uint32_t soff = KC ? (uint32_t)k0 * ESZ : (uint32_t)k0 * op.ld_bytes;
    const int klim = (KC ? op.cols : op.rows) - k0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int b = wave + NW * j;
      if (J * NW == NB || b < NB) {
        const bool v = ok[j] && (full || krel[j] < klim);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            op.rs, (__attribute__((address_space(3))) void*)(dst + b * 1024), 16,
            v ? off[j] : kOOB, __builtin_amdgcn_readfirstlane(soff), 0, 0);
      }
    }
  }

  __device__ __forceinline__ void mainloop_dma2(const Operand& A, const Operand& B, int K,
                                                char* lds) {
    static_assert(KS % 2 == 0, "fragment sets alternate within a stage");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int nk = (K + BK - 1) / BK;
    if (nk <= 0) return;
    uint32_t offa[A_J], offb[B_J];
    int ka[A_J], kb[B_J];
    bool oka[A_J], okb[B_J];
    dma_setup<A_KC, BM, A_PITCH, A_NB, A_J>(A, wave, offa, ka, oka);
    dma_setup<B_KC, BN, B_PITCH, B_NB, B_J>(B, wave, offb, kb, okb);
    // dma_setup's offsets include the operand origin at k = 0
    auto issue = [&](int t) {
      char* st = lds + (t & 1) * STAGE;
      const bool full = (t + 1) * BK <= K;
      dma_issue2<A_KC, A_NB, A_J>(A, wave, t * BK, full, st, offa, ka, oka);
      dma_issue2<B_KC, B_NB, B_J>(B, wave, t * BK, full, st + A_BYTES, offb, kb, okb);
    };
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 1) {
      const int per_stage = min(A_J, (A_NB - wave + NW - 1) / NW) + min(B_J, (B_NB - wave + NW - 1) / NW);
      wait_vm(per_stage);
    } else {
      wait_vm(0);
    }
    asm volatile("s_barrier" ::: "memory");
    u32x4_t fa[2][MI], fb[2][NI];
    read_frags(lds, lds + A_BYTES, wm, wn, 0, fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = lds + (kt & 1) * STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) read_frags(cur, cur + A_BYTES, wm, wn, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        mma_all(fa[ks & 1], fb[ks & 1]);
      }
      if (kt + 1 < nk) {
        wait_vm(0);
        asm volatile("s_barrier" ::: "memory");
        if (kt + 2 < nk) issue(kt + 2);
        const char* nx = lds + ((kt + 1) & 1) * STAGE;
        read_frags(nx, nx + A_BYTES, wm, wn, 0, fa[0], fb[0]);
      }
    }
    __syncthreads();
  }

  // Register-staged double buffer (NS == 2), LDS laid out [A0 A1 B0 B1] so
  // that with the stage parity fixed (loop unrolled by two) every LDS
  // address is a per-thread base plus an immediate:
  //   - fragments of step s+1 are read from LDS while step s's MFMAs run;
  //   - the next stage, already in registers, is written to the other LDS
  //     buffer after the second step and the loads of the stage after it are
  //     issued right then (global latency hides behind ~1.5 stages);
  //   - one barrier per stage.
  // Stages whose loads two ahead lie wholly below K run a branch-free body
  // (STEADY): one scheduling region per fragment step, in which the MFMAs
  // alternate with that step's LDS reads and, in the first step, with the
  // next stage's LDS writes and global loads (issued there, the loads run
  // ~1.75 stages ahead of their use); the last step issues half its
  // MFMAs, meets the barrier, reads the next stage's first fragments and
  // then issues its other half, so the matrix unit has work while those
  // reads are in flight.  The last few stages run the general body, whose
  // bounds checks and conditions are branches.
  __device__ __forceinline__ void mma_rows(const u32x4_t* fa, const u32x4_t* fb, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) mma(acc[i][j], fa[i], fb[j]);
  }

  // sched_group_barrier masks (LLVM AMDGPU): instruction classes
  static constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100,
                       kSchedDsWrite = 0x200;

  template <int P, bool STEADY>
  __device__ __forceinline__ void regs_stage(const Operand& A, const Operand& B, char* lds, int kt,
                                             int nk, int K, int wm, int wn, const uint32_t* va,
                                             const int* ka, const uint32_t* vb, const int* kb,
                                             u32x4_t* ra, u32x4_t* rb, u32x4_t (*fa)[MI],
                                             u32x4_t (*fb)[NI]) {
    const char* ca = lds + P * A_BYTES;
    const char* cb = lds + 2 * A_BYTES + P * B_BYTES;
    char* na = lds + (1 - P) * A_BYTES;
    char* nb = lds + 2 * A_BYTES + (1 - P) * B_BYTES;
    if constexpr (STEADY) {
      // LDS reads per step: one per K-contiguous fragment; two transpose
      // reads (bf16) or four scalar reads (fp32) per MN-contiguous one
      constexpr int RMC = ESZ == 2 ? 2 : 4;
      constexpr int NR = (A_KC ? MI : RMC * MI) + (B_KC ? NI : RMC * NI);
      constexpr int NM = MI * NI * (ESZ == 2 ? 1 : 4);                // MFMAs per step
      constexpr int NL = A_LD + B_LD;                                 // loads per stage
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          read_frags(ca, cb, wm, wn, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
          mma_all(fa[ks & 1], fb[ks & 1]);
          if (ks == 0) {
            lstore<A_KC, BM, A_PITCH, A_LD>(na, ra);
            lstore<B_KC, BN, B_PITCH, B_LD>(nb, rb);
            const int k0 = (kt + 2) * BK;
            gload_fast<A_KC, A_LD>(A, va, ka, k0, true, ra);
            gload_fast<B_KC, B_LD>(B, vb, kb, k0, true, rb);
          }
#pragma unroll
          for (int q = 0; q < NM; ++q) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (q < NR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            if (ks == 0 && q < NL) {
              __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
              __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
          mma_rows(fa[ks & 1], fb[ks & 1], 0, MI / 2);
          __builtin_amdgcn_sched_barrier(0);
          __syncthreads();
          read_frags(na, nb, wm, wn, 0, fa[0], fb[0]);
          mma_rows(fa[ks & 1], fb[ks & 1], MI / 2, MI);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NR, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, NM / 2, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) read_frags(ca, cb, wm, wn, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      mma_all(fa[ks & 1], fb[ks & 1]);
      if (ks == 1 && kt + 1 < nk) {
        lstore<A_KC, BM, A_PITCH, A_LD>(na, ra);
        lstore<B_KC, BN, B_PITCH, B_LD>(nb, rb);
        if (kt + 2 < nk) {
          const int k0 = (kt + 2) * BK;
          const bool full = k0 + BK <= K;
          gload_fast<A_KC, A_LD>(A, va, ka, k0, full, ra);
          gload_fast<B_KC, B_LD>(B, vb, kb, k0, full, rb);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < nk) read_frags(na, nb, wm, wn, 0, fa[0], fb[0]);
  }

  __device__ __forceinline__ void mainloop_regs(const Operand& A, const Operand& B, int K, char* lds) {
    static_assert(KS % 2 == 0 && KS >= 2, "fragment double buffer needs an even step count");
    static_assert(MI % 2 == 0, "the last step's MFMAs are issued in two halves");
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nk = (K + BK - 1) / BK;
    if (nk <= 0) return;
    uint32_t va[A_LD], vb[B_LD];
    int ka[A_LD], kb[B_LD];
    gprep<A_KC, BM, A_LD>(A, va, ka);
    gprep<B_KC, BN, B_LD>(B, vb, kb);
    u32x4_t ra[A_LD], rb[B_LD];
    gload_fast<A_KC, A_LD>(A, va, ka, 0, BK <= K, ra);
    gload_fast<B_KC, B_LD>(B, vb, kb, 0, BK <= K, rb);
    lstore<A_KC, BM, A_PITCH, A_LD>(lds, ra);
    lstore<B_KC, BN, B_PITCH, B_LD>(lds + 2 * A_BYTES, rb);
    if (nk > 1) {
      gload_fast<A_KC, A_LD>(A, va, ka, BK, 2 * BK <= K, ra);
      gload_fast<B_KC, B_LD>(B, vb, kb, BK, 2 * BK <= K, rb);
    }
    __syncthreads();
    u32x4_t fa[2][MI], fb[2][NI];
    read_frags(lds, lds + 2 * A_BYTES, wm, wn, 0, fa[0], fb[0]);
    // a pair of stages (kt, kt + 1) is steady when the stages they load,
    // kt + 2 and kt + 3, are whole: (kt + 4) * BK <= K
    const int nfull = K / BK;
    int kt = 0;
    for (; kt + 4 <= nfull; kt += 2) {
      regs_stage<0, true>(A, B, lds, kt, nk, K, wm, wn, va, ka, vb, kb, ra, rb, fa, fb);
      regs_stage<1, true>(A, B, lds, kt + 1, nk, K, wm, wn, va, ka, vb, kb, ra, rb, fa, fb);
    }
    for (; kt < nk; kt += 2) {
      regs_stage<0, false>(A, B, lds, kt, nk, K, wm, wn, va, ka, vb, kb, ra, rb, fa, fb);
      if (kt + 1 < nk) regs_stage<1, false>(A, B, lds, kt + 1, nk, K, wm, wn, va, ka, vb, kb, ra, rb, fa, fb);
    }
  }

  __device__ __forceinline__ void mainloop_dma(const Operand& A, const Operand& B, int K, char* lds) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int nk = (K + BK - 1) / BK;
    if (nk <= 0) return;
    uint32_t offa[A_J], offb[B_J];
    int ka[A_J], kb[B_J];
    bool oka[A_J], okb[B_J];
    dma_setup<A_KC, BM, A_PITCH, A_NB, A_J>(A, wave, offa, ka, oka);
    dma_setup<B_KC, BN, B_PITCH, B_NB, B_J>(B, wave, offb, kb, okb);
    // this wave's DMA instructions per stage
    const int per_stage = min(A_J, (A_NB - wave + NW - 1) / NW) + min(B_J, (B_NB - wave + NW - 1) / NW);

    auto issue = [&](int t) {
      char* st = lds + (t % NS) * STAGE;
      dma_issue<A_KC, A_NB, A_J>(A, wave, t * BK, st, offa, ka, oka);
      dma_issue<B_KC, B_NB, B_J>(B, wave, t * BK, st + A_BYTES, offb, kb, okb);
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < nk) issue(t);

    u32x4_t fa[2][MI], fb[2][NI];
    for (int kt = 0; kt < nk; ++kt) {
      // stages issued so far: 0 .. min(nk, kt + NS - 1) - 1; kt and kt + 1 must be done
      const int issued = min(nk, kt + NS - 1);
      const int later = max(0, issued - (kt + 2));
      wait_vm(later * per_stage);
      // A plain s_barrier: __syncthreads() would also drain every outstanding
      // DMA (vmcnt(0)) and serialise the ring.  The "memory" clobber keeps the
      // compiler from moving LDS accesses across it; this wave's reads of the
      // stage being recycled have all been consumed by MFMAs already.
      asm volatile("s_barrier" ::: "memory");
      if (kt + NS - 1 < nk) issue(kt + NS - 1);
      const char* cur = lds + (kt % NS) * STAGE;
      if (kt == 0) read_frags(cur, cur + A_BYTES, wm, wn, 0, fa[0], fb[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int nb = (ks + 1) & 1;
        if (ks + 1 < KS) {
          read_frags(cur, cur + A_BYTES, wm, wn, ks + 1, fa[nb], fb[nb]);
        } else {
          // first fragments of the next stage (unconditional, so that the
          // LDS counter waits stay exact; after the last stage the read is
          // of a stale slot and unused)
          const char* nx = lds + ((kt + 1) % NS) * STAGE;
          read_frags(nx, nx + A_BYTES, wm, wn, 0, fa[nb], fb[nb]);
        }
        mma_all(fa[ks & 1], fb[ks & 1]);
      }
      if constexpr (KS % 2 == 1) {
        // the next stage's first fragments sit in set 1: move them to set 0
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[0][i] = fa[1][i];
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[0][j] = fb[1][j];
      }
    }
    __syncthreads();
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

// Tile id -> (tm, tn): ids are rastered in column strips `group` tiles tall,
// so that a run of consecutive ids shares a few A (tm) and B (tn) panels.
__device__ __forceinline__ void raster(int id, int nm, int nn, int group, int& tm, int& tn) {
  const int span = group * nn;
  const int g = id / span, w = id % span;
  const int m0 = g * group;
  const int gs = min(nm - m0, group);
  tm = m0 + w % gs;
  tn = w / gs;
}

// Workgroup -> tile mapping that keeps the workgroups co-resident on one XCD
// (consecutive workgroup ids are dealt round-robin over the 8 XCDs, each with
// its own L2) on a compact block of tiles: XCD x takes a contiguous range of
// tile ids, rastered as above, so the ~32 workgroups an XCD runs at once
// share a few A and B panels in its L2.  Returns false for the padding
// workgroups past the last tile, and for every workgroup beyond the first
// xcd_grid(nm, nn) when the grid is larger (a tile count known only on the
// device), whose ids would otherwise alias the next XCD's range.
__device__ __forceinline__ bool xcd_tile(int bid, int nm, int nn, int group, int& tm, int& tn) {
  const int total = nm * nn;
  const int per = (total + 7) / 8;
  const int q = bid >> 3;
  if (q >= per) return false;
  const int id = (bid & 7) * per + q;
  if (id >= total) return false;
  raster(id, nm, nn, group, tm, tn);
  return true;
}

__host__ __device__ inline int xcd_grid(int nm, int nn) { return ((nm * nn + 7) / 8) * 8; }

}  // namespace flce
