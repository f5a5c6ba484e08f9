// Batched "NT" matrix product on MFMA for gfx950, with the Newton-Schulz epilogues fused.
//
//   C[b][i][j] = sum_k A[b][i][k] * B[b][j][k]     (A K-contiguous; B K-contiguous, or
//                                                   stored k-major as B[b][k][j])
//
// Every product of the method has this form:
//  - X X^T (the Gram / SYRK product): A = B = X (n x m, row-major), K = m;
//  - products of the symmetric n x n iterates (R R, R Z, Z (R Z), Z Q, A A): the right
//    operand is symmetric and stored in full, so its rows are its columns;
//  - the rectangular Q X and B X: the right operand is X itself (n x m row-major), read
//    k-major through gfx950's transposing LDS reads, so no transposed copy of X exists.
// TRI=true computes only the tiles on or above the diagonal of a symmetric result and
// writes each value to (i, j) and (j, i), so stored symmetric matrices are exactly
// symmetric.
//
// Tiles (TileCfg): every wave computes 64 x 64 as 2 x 2 blocks of the 32x32 MFMA (bf16/f16:
// v_mfma_f32_32x32x16, fp32: v_mfma_f32_32x32x2f32) with fp32 accumulation, and K moves
// through LDS 128 bytes per operand row at a time (64 half-precision or 32 fp32 values).
// Large problems: 256 x 256 per workgroup of 16 waves, operands DMA'd global -> LDS into a
// 2-deep ring of XOR-swizzled k-stages. Small problems: 128 x 128 per workgroup of 4 waves,
// staged through registers into LDS rows padded to 144 bytes.
//
// Epilogue (per matrix b, scale s_b from the norm kernel):
//   v = s_b^spow * (c2 * acc + c1 * E[i][j]) + c0 * [i == j < M]
// then any of: store v to C (i, j) [and (j, i) for TRI], store v to Ct (j, i), and the
// Muon update W <- wd_mul * W - lr * u_scale * v (optionally U <- u_scale * v).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mns {

struct GemmArgs {
  const void* A; int64_t lda, sA;
  const void* B; int64_t ldb, sB;
  int M, N, K;
  int tiles_m, tiles_n, tiles_per_mat, nblocks, group_m;
  const float* svec; int spow;
  float c0, c1, c2;
  const void* E; int e_dt; int64_t lde, sE; int e_rows, e_cols;
  void* C; int c_dt; int64_t ldc, sC; int c_rows, c_cols;
  void* Ct; int ct_dt; int64_t ldct, sCt; int ct_rows, ct_cols;
  void* W; int w_dt; int64_t ldw, sW; int w_trans;
  void* U; int u_dt; int64_t ldu, sU;
  float u_scale, lr, wd_mul;
  int32_t* flags;
  // 1 when 8-element vectors of that buffer are aligned (ld, stride and base)
  int c_vec, ct_vec, w_vec, u_vec;
  // nonzero: the typed fast epilogue applies (1: f16 out/f16 E, 2: bf16/bf16, 3: f16/bf16,
  // 4: bf16/f16, 5: f32/f32; 6, 7, 8: the weight update alone, W bf16, f16, f32)
  int fast_epi;
};

// Several independent problems of one product kind in one launch (a grouped GEMM). Each
// group's tile list (g[i].nblocks tiles) is cut into 8 equal parts, one per XCD, so every XCD
// gets the same share of every group (balanced whatever the groups' tile costs) and keeps
// neighbouring tiles of a group together (shared operand panels in its L2).
constexpr int MNS_MAXG = 4;
struct GemmBatch {
  GemmArgs g[MNS_MAXG];
  int ng;
};
__host__ __device__ inline int xcd_part_lo(int nblocks, int x) { return (int)((int64_t)nblocks * x / 8); }

template <typename T> struct MfmaTraits;
template <> struct MfmaTraits<__bf16> { static constexpr int ES = 2; };
template <> struct MfmaTraits<_Float16> { static constexpr int ES = 2; };
template <> struct MfmaTraits<float> { static constexpr int ES = 4; };

// Tile configuration: BM x BN per workgroup, WVM x WVN waves, each wave (BM/WVM) x (BN/WVN)
// made of 32 x 32 MFMA blocks. Each k-stage stages KB bytes of every operand row in LDS
// (KB = 128: 64 half / 32 fp32 values; KB = 64: half that). PF = number of k-stages whose
// global loads are in flight in registers (1: the next stage, 2: the next two). OCC = waves
// per SIMD the register budget is sized for.
template <int BM_, int BN_, int WVM_, int WVN_, int KB_, int PF_, int OCC_, int NST_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WVM = WVM_, WVN = WVN_, KB = KB_, PF = PF_, OCC = OCC_;
  // NST > 0: operands go global -> LDS by DMA (no register staging) into a ring of NST
  // unpadded, XOR-swizzled k-stages, NST - 1 stages ahead of the one being consumed.
  static constexpr int NST = NST_;
  static constexpr bool DL = NST_ > 0;
  static constexpr int STG = (BM_ + BN_) * KB_;          // bytes per DMA stage
  static constexpr int NT = 64 * WVM * WVN;
  static constexpr int WTM = BM / WVM, WTN = BN / WVN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int CPR = KB / 16;                    // 16-byte chunks per staged row
  static constexpr int NG = KB / 32;                     // 32-byte k-groups per stage (one MFMA k-step)
  static constexpr int ROWB = KB + 16;                   // LDS bytes per staged row (padded)
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int CA = BM * CPR / NT, CB = BN * CPR / NT;  // chunks per thread
  // Epilogue slab: SR wave-rows of the tile at a time, fp32, rows padded to 16-byte multiples.
  static constexpr int CP = BN + 4;
  static constexpr int SR = (WVM >= 4 && BM >= 256) ? 2 : 1;
  static constexpr int SLAB = SR * WTM * CP * 4;
  static constexpr int MAINLDS = DL ? NST * STG : 2 * STAGE;
  static constexpr int LDS = MAINLDS > SLAB ? MAINLDS : SLAB;
  static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tile must be whole MFMA blocks");
  static_assert(CA * NT == BM * CPR && CB * NT == BN * CPR, "chunks must divide evenly");
  static_assert(NT % CPR == 0, "a thread keeps one chunk column");
  static_assert(WVM % SR == 0 && BN % 16 == 0 && (SR * WTM) % 32 == 0, "epilogue slab shape");
};

// Small problems: 128 x 128, 4 waves of 64 x 64, 128-byte k-stages staged through registers,
// 2 waves per SIMD.
// Large problems: 256 x 256, 16 waves of 64 x 64, 128-byte k-stages DMA'd global -> LDS into a
// 2-deep ring, 4 waves per SIMD (one workgroup per CU; latency is hidden by the four waves
// each SIMD interleaves).
using Tile128 = TileCfg<128, 128, 2, 2, 128, 1, 2>;
using Tile256 = TileCfg<256, 256, 4, 4, 128, 1, 4, 2>;

// 8 consecutive elements of a buffer of runtime dtype (16-byte aligned for 16-bit types,
// 32-byte for fp32).
__device__ inline void load8(const void* p, int dt, int64_t idx, float (&v)[8]) {
  if (dt == F32) {
    const f32x4* q = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + idx);
    const f32x4 a = q[0], b = q[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p) + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t lo = (uint16_t)(w[e] & 0xffffu), hi = (uint16_t)(w[e] >> 16);
      v[2 * e] = dt == BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
      v[2 * e + 1] = dt == BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
    }
  }
}

__device__ inline void store8(void* p, int dt, int64_t idx, const float (&v)[8]) {
  if (dt == F32) {
    f32x4* q = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p) + idx);
    q[0] = f32x4{v[0], v[1], v[2], v[3]};
    q[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = dt == BF16 ? f32_to_bf16_bits(v[2 * e]) : f32_to_f16_bits(v[2 * e]);
      const uint32_t hi = dt == BF16 ? f32_to_bf16_bits(v[2 * e + 1]) : f32_to_f16_bits(v[2 * e + 1]);
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p) + idx) = w;
  }
}

// Store elements e in [lo, 8) of a vector at idx: whole vector when allowed, else one by one
// (only indices below `lim` are written in the scalar path).
__device__ inline void store_part(void* p, int dt, int64_t idx, const float (&v)[8], int lo,
                                  int lim, bool vec_ok) {
  if (lo == 0 && lim >= 8 && vec_ok) {
    store8(p, dt, idx, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= lo && e < lim) store_elem(p, dt, idx + e, v[e]);
  }
}

// Typed 8-element vector load/store (16-bit types: one 16-byte access; fp32: two).
template <typename OT> struct VecIO;
template <> struct VecIO<float> {
  typedef float raw __attribute__((ext_vector_type(8)));
  static __device__ inline raw load_raw(const void* p, int64_t idx) {
    const f32x4* q = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + idx);
    const f32x4 a = q[0], b = q[1];
    return raw{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  static __device__ inline void unpack(const raw& w, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = w[e];
  }
  static __device__ inline void load(const void* p, int64_t idx, float (&v)[8]) {
    const f32x4* q = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + idx);
    const f32x4 a = q[0], b = q[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
  }
  static __device__ inline void store(void* p, int64_t idx, const float (&v)[8]) {
    f32x4* q = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p) + idx);
    q[0] = f32x4{v[0], v[1], v[2], v[3]};
    q[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
};
template <typename H> struct VecIO16 {
  static __device__ inline float cvt(uint16_t h) {
    if constexpr (__is_same(H, __bf16)) return bf16_bits_to_f32(h); else return f16_bits_to_f32(h);
  }
  static __device__ inline uint32_t bits(float f) {
    if constexpr (__is_same(H, __bf16)) return f32_to_bf16_bits(f); else return f32_to_f16_bits(f);
  }
  typedef u32x4 raw;
  static __device__ inline raw load_raw(const void* p, int64_t idx) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p) + idx);
  }
  static __device__ inline void unpack(const raw& w, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = cvt((uint16_t)(w[e] & 0xffffu));
      v[2 * e + 1] = cvt((uint16_t)(w[e] >> 16));
    }
  }
  static __device__ inline void load(const void* p, int64_t idx, float (&v)[8]) { unpack(load_raw(p, idx), v); }
  static __device__ inline void store(void* p, int64_t idx, const float (&v)[8]) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack2<H>(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p) + idx) = w;
  }
};
template <> struct VecIO<__bf16> : VecIO16<__bf16> {};
template <> struct VecIO<_Float16> : VecIO16<_Float16> {};

// MFMA operand fragment of one 32-row block for one 16-byte k-chunk group: 8 half values or
// 4 fp32 values per lane (lane l holds row l % 32, chunk half l / 32 of the group).
template <typename T> struct Frag { typedef T type __attribute__((ext_vector_type(8))); };
template <> struct Frag<float> { typedef f32x4 type; };

template <typename T, int TM, int TN, int ROWB, bool LB = true>
__device__ inline void load_frags(const char* As, const char* Bs, int lane, int g,
                                  typename Frag<T>::type (&a)[TM], typename Frag<T>::type (&b)[TN]) {
  typedef typename Frag<T>::type F;
  const int l32 = lane & 31, hi = lane >> 5;
  const int off = g * 32 + hi * 16;
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const F*>(As + (i * 32 + l32) * ROWB + off);
  if constexpr (LB) {
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const F*>(Bs + (j * 32 + l32) * ROWB + off);
  }
}

// XOR swizzle of the 16-byte chunk index within an unpadded k-stage row, as a function of the
// row: conflict-free 16-byte fragment reads of 32 consecutive rows for 32- and 64-bank LDS.
template <int CPR>
__device__ __host__ constexpr int chunk_swizzle(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

template <typename T, int TM, int TN, int KB, bool LB = true>
__device__ inline void load_frags_dl(const char* As, const char* Bs, int lane, int g, int sw,
                                     typename Frag<T>::type (&a)[TM], typename Frag<T>::type (&b)[TN]) {
  typedef typename Frag<T>::type F;
  const int l32 = lane & 31, hi = lane >> 5;
  const int off = (((2 * g + hi) ^ sw) << 4);
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const F*>(As + (i * 32 + l32) * KB + off);
  if constexpr (LB) {
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const F*>(Bs + (j * 32 + l32) * KB + off);
  }
}

// B operand stored k-major (element (n, k) of the NT operand at B[k * ldb + n]: the X of a
// rectangular product Q X read in place). A stage holds BK k-rows of BN values; its 16-byte
// chunks are XOR-swizzled by kmajor_swizzle(k & 3), which keeps the transposing reads below
// free of bank conflicts for 32- and 64-bank LDS (rows at least 16 chunks long).
__device__ __host__ constexpr int kmajor_swizzle(int s) { return (4 * s) ^ (2 * (s >> 1)); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Per-lane byte offset of fragment column block j (16-bit types) inside a k-major B stage of
// RB bytes per k-row, before the k-group offset. ds_read_b64_tr_b16 hands lane i of each
// 16-lane group element (i mod 4) of the 8-byte pieces addressed by lanes 4e + i / 4
// (e = 0..3); addressing rows k0 + j16 / 4 at columns 16 qo + 4 (j16 mod 4) therefore gives
// lane (qo, i) the values B[k0 + e][16 qo + i], four consecutive k of one column.
template <int RB>
__device__ inline int kmajor_frag_off(int lane, int n0) {
  const int j16 = lane & 15, qo = (lane >> 4) & 1, hi = lane >> 5;
  const int n = n0 + 16 * qo + 4 * (j16 & 3);
  return (8 * hi + (j16 >> 2)) * RB + (((n >> 3) ^ kmajor_swizzle(j16 >> 2)) << 4) + 8 * (j16 & 1);
}

// B fragments (8 consecutive k of one column per lane, the layout load_frags gives) from a
// k-major stage: two transposing 8-byte reads per fragment (k 0..3 and 4..7 of the lane's
// half of the 16-wide k-group g).
//
// The reads are issued from inline assembly that also waits for them: the compiler treats
// the transposing-read builtin as possibly reading what the in-flight global -> LDS DMA of
// the next k-stage writes and would wait for that DMA before every read, serialising the
// DMA with the MFMAs. The DMA ring's own waits and barriers order these reads correctly.
template <typename T, int TN, int RB>
__device__ inline void load_b_kmajor(const char* Bs, const int (&boff)[TN], int g,
                                     typename Frag<T>::type (&b)[TN]) {
  typedef typename Frag<T>::type F;
  typedef __attribute__((address_space(3))) const char* lds_ptr;
  static_assert(TN == 2, "two column blocks per wave");
  const unsigned a0 = (unsigned)(size_t)(lds_ptr)(Bs + boff[0] + 16 * g * RB);
  const unsigned a1 = (unsigned)(size_t)(lds_ptr)(Bs + boff[1] + 16 * g * RB);
  s16x4 lo0, hi0, lo1, hi1;
  __asm__ __volatile__(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo0), "=&v"(hi0), "=&v"(lo1), "=&v"(hi1)
      : "v"(a0), "v"(a1), "i"(4 * RB)
      : "memory");
  b[0] = __builtin_bit_cast(F, (s16x8)__builtin_shufflevector(lo0, hi0, 0, 1, 2, 3, 4, 5, 6, 7));
  b[1] = __builtin_bit_cast(F, (s16x8)__builtin_shufflevector(lo1, hi1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// fp32 B fragments from a k-major stage (lane (l32, hi) holds k = 8 g + 4 hi + e of column
// n0 + l32): four 4-byte reads; consecutive lanes read consecutive columns.
template <int TN, int RB>
__device__ inline void load_b_kmajor_f32(const char* Bs, int lane, int n0, int g, f32x4 (&b)[TN]) {
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + j * 32 + l32;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 8 * g + 4 * hi + e;
      b[j][e] = *reinterpret_cast<const float*>(Bs + k * RB + (((n >> 2) ^ kmajor_swizzle(e)) << 4) + (n & 3) * 4);
    }
  }
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt low/high bits, expcnt
// and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt on the LDS / scalar-memory counter only (lgkmcnt(0); vmcnt and expcnt at their
// no-wait maxima).
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Value known to be equal across the wave (kept in scalar registers).
__device__ inline int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 16-byte global -> LDS DMA of one lane; the wave's 64 lanes fill 1 KB at lds_base (uniform).
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}

// Workgroup barrier without a memory fence (LDS DMA completion is waited for explicitly);
// the empty asm statements keep the compiler from moving memory operations across it.
__device__ inline void barrier_nofence() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// Empty asm that "modifies" the fragment registers: MFMAs that read them cannot move above it.
template <typename T, int TM, int TN>
__device__ inline void pin_frags(typename Frag<T>::type (&a)[TM], typename Frag<T>::type (&b)[TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i) __asm__ __volatile__("" : "+v"(a[i]));
#pragma unroll
  for (int j = 0; j < TN; ++j) __asm__ __volatile__("" : "+v"(b[j]));
}

template <typename T, int TM, int TN>
__device__ inline void mma(const typename Frag<T>::type (&a)[TM], const typename Frag<T>::type (&b)[TN],
                           f32x16 (&acc)[TM][TN]) {
  if constexpr (MfmaTraits<T>::ES == 2) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (__is_same(T, __bf16))
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
  } else {
    // lane (l32, hi) holds k = 4*hi + e of this 8-wide group; A and B agree, so the
    // products still pair equal k.
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
  }
}

// Raw buffer resource over one operand matrix: loads at byte offsets >= num_records return 0,
// which zero-fills rows past the end and the k tail without branches.
constexpr uint32_t OOB = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Accumulators of this wave to the fp32 epilogue slab (its rows from lrow0 of the slab).
template <class CFG>
__device__ inline void acc_to_slab(float* Cs, const f32x16 (&acc)[CFG::TM][CFG::TN], int lane, int wn, int lrow0) {
  constexpr int CP = CFG::CP;
  float* base = Cs + (lrow0 + 4 * (lane >> 5)) * CP + wn * CFG::WTN + (lane & 31);
#pragma unroll
  for (int i = 0; i < CFG::TM; ++i)
#pragma unroll
    for (int j = 0; j < CFG::TN; ++j)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) base[(i * 32 + 8 * (rr >> 2) + (rr & 3)) * CP + j * 32] = acc[i][j][rr];
}

// Barrier between epilogue passes: only this workgroup's LDS accesses need to be complete (the
// slab is rewritten by the next pass or the next tile's DMA); its global stores stay in flight.
__device__ inline void lds_barrier() {
  wait_lgkmcnt0();
  barrier_nofence();
}

// Fast epilogue for internal outputs: C (row-major; mirrored for symmetric results) and
// optionally C^T, both of dtype OT with rows padded to multiples of 8, E of dtype ET. No
// runtime dtype dispatch and whole 16-byte vectors only.
template <typename OT, typename ET, bool TRI, class CFG>
__device__ inline void epilogue_fast(const GemmArgs& p, char* lds, f32x16 (&acc)[CFG::TM][CFG::TN],
                                     int mat, int ti, int tj, int row0, int col0, int lane) {
  constexpr int BN = CFG::BN, NT = CFG::NT, WTM = CFG::WTM, CP = CFG::CP;
  constexpr int SR = CFG::SR, SROWS = SR * WTM, VPR = BN / 8, RVC = SROWS / 8;
  const int wave = wave_uniform(threadIdx.x >> 6), tid = wave * 64 + lane;
  const int wm = wave / CFG::WVN, wn = wave % CFG::WVN;
  float sc = 1.f;
  if (p.spow) {
    const float sb = p.svec[mat];
    sc = p.spow == 1 ? sb : sb * sb;
  }
  constexpr int OS = sizeof(OT);
  const char* Eb = p.E ? reinterpret_cast<const char*>(p.E) + (int64_t)mat * p.sE * sizeof(ET) : nullptr;
  char* Cb = p.C ? reinterpret_cast<char*>(p.C) + (int64_t)mat * p.sC * OS : nullptr;
  char* Ctb = p.Ct ? reinterpret_cast<char*>(p.Ct) + (int64_t)mat * p.sCt * OS : nullptr;
  const bool diag = TRI && ti == tj;
  const bool colpass = (TRI && Cb) || Ctb;
  const float c0 = p.c0, c1 = p.c1, c2 = p.c2;
  float* Cs = reinterpret_cast<float*>(lds);
  for (int sl = 0; sl < CFG::WVM / SR; ++sl) {
    if (wm / SR == sl) {
      acc_to_slab<CFG>(Cs, acc, lane, wn, (wm % SR) * WTM);
    }
    lds_barrier();
    const int srow0 = row0 + sl * SROWS;
    // E vector of element index i (8 values from row srow0 + i / VPR): issued one vector ahead
    // of its use, into two fixed registers, so that its wait does not also wait for the stores
    // issued in between. Every fetch is issued and used (a vector outside E reads E's first
    // vector and is discarded), so no path leaves a load in flight.
    constexpr int ITR = SROWS * VPR / NT;
    static_assert(ITR % 2 == 0 && ITR * NT == SROWS * VPR, "row pass in pairs of iterations");
    auto fetch_e = [&](int i, typename VecIO<ET>::raw& e) {
      const int r = srow0 + i / VPR, c = col0 + (i % VPR) * 8;
      const bool h = r < p.e_rows && c < p.e_cols;
      e = VecIO<ET>::load_raw(Eb, h ? (int64_t)r * p.lde + c : 0);
      return h;
    };
    auto row_vec = [&](int idx, const typename VecIO<ET>::raw* er, bool he) {
      const int lr = idx / VPR, lc = (idx - lr * VPR) * 8;
      const int r = srow0 + lr, c = col0 + lc;
      float* cs = Cs + lr * CP + lc;
      const f32x4 a = *reinterpret_cast<const f32x4*>(cs);
      const f32x4 b = *reinterpret_cast<const f32x4*>(cs + 4);
      float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= c2;
      if (er) {
        float ev[8];
        VecIO<ET>::unpack(*er, ev);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = he ? v[e] + c1 * ev[e] : v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] *= sc;
        if (r == c + e && r < p.M) v[e] += c0;
      }
      if (colpass) {
        *reinterpret_cast<f32x4*>(cs) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(cs + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
      if (Cb && r < p.c_rows && c < p.c_cols) {
        if (!diag || r <= c) {
          VecIO<OT>::store(Cb, (int64_t)r * p.ldc + c, v);
        } else if (r < c + 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e >= r) store_elem(Cb, sizeof(OT) == 4 ? F32 : (__is_same(OT, __bf16) ? BF16 : F16), (int64_t)r * p.ldc + c + e, v[e]);
        }
      }
    };
    if (Eb) {
      typename VecIO<ET>::raw e0, e1;
      bool h0 = fetch_e(tid, e0);
#pragma unroll 1
      for (int it = 0; it < ITR; it += 2) {
        const int idx = tid + it * NT;
        const bool h1 = fetch_e(idx + NT, e1);
        row_vec(idx, &e0, h0);
        if (it + 2 < ITR) h0 = fetch_e(idx + 2 * NT, e0);
        row_vec(idx + NT, &e1, h1);
      }
    } else {
#pragma unroll 1
      for (int idx = tid; idx < SROWS * VPR; idx += NT) row_vec(idx, nullptr, false);
    }
    if (colpass) {
      lds_barrier();
      for (int idx = tid; idx < BN * RVC; idx += NT) {
        const int ci = idx & 15, ri = (idx >> 4) & 3, blk = idx >> 6;
        const int cb = blk % (BN / 16), rb = blk / (BN / 16);
        const int lc = cb * 16 + ci, lr = (rb * 4 + ri) * 8;
        const int r = srow0 + lr, c = col0 + lc;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Cs[(lr + e) * CP + lc];
        if (TRI && Cb && c < p.c_rows && r < p.c_cols) {
          if (!diag || r + 8 <= c) {
            VecIO<OT>::store(Cb, (int64_t)c * p.ldc + r, v);
          } else if (r < c) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (r + e < c) store_elem(Cb, sizeof(OT) == 4 ? F32 : (__is_same(OT, __bf16) ? BF16 : F16), (int64_t)c * p.ldc + r + e, v[e]);
          }
        }
        if (Ctb && c < p.ct_rows && r < p.ct_cols) VecIO<OT>::store(Ctb, (int64_t)c * p.ldct + r, v);
      }
    }
    lds_barrier();
  }
}

// Weight-update epilogue for the last product of the Muon step (no E, C or U, c0 = 0): per
// element W <- wd_mul W - lr (u_scale v), v = s^spow c2 acc, W of dtype WT in 16-byte vectors (row-major,
// or transposed when the caller's matrix is m x n); bit 2 of flags[mat] marks a non-finite v.
template <typename WT, class CFG>
__device__ inline void epilogue_wupd(const GemmArgs& p, char* lds, f32x16 (&acc)[CFG::TM][CFG::TN],
                                     int mat, int row0, int col0, int lane) {
  constexpr int BN = CFG::BN, NT = CFG::NT, WTM = CFG::WTM, CP = CFG::CP;
  constexpr int SR = CFG::SR, SROWS = SR * WTM, VPR = BN / 8, RVC = SROWS / 8;
  const int wave = wave_uniform(threadIdx.x >> 6), tid = wave * 64 + lane;
  const int wm = wave / CFG::WVN, wn = wave % CFG::WVN;
  float sc = 1.f;
  if (p.spow) {
    const float sb = p.svec[mat];
    sc = p.spow == 1 ? sb : sb * sb;
  }
  char* Wb = reinterpret_cast<char*>(p.W) + (int64_t)mat * p.sW * sizeof(WT);
  bool bad = false;
  float* Cs = reinterpret_cast<float*>(lds);
  // the same operations in the same order as the generic epilogue, so both give the same W
  // (h: the vector lies inside W; its loaded value is always consumed, its store is not)
  auto update = [&](int64_t wi, bool h, const typename VecIO<WT>::raw& wraw, const float (&acc8)[8]) {
    float w[8];
    VecIO<WT>::unpack(wraw, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = p.c2 * acc8[e];
      v *= sc;
      bad |= h && !__builtin_isfinite(v);
      const float u = p.u_scale * v;
      w[e] = p.wd_mul * w[e] - p.lr * u;
    }
    if (h) VecIO<WT>::store(Wb, wi, w);
  };
  for (int sl = 0; sl < CFG::WVM / SR; ++sl) {
    const int srow0 = row0 + sl * SROWS;
    if (wm / SR == sl) {
      acc_to_slab<CFG>(Cs, acc, lane, wn, (wm % SR) * WTM);
    }
    lds_barrier();
    // each lane's 16-bit W vectors are loaded one vector ahead of their update, so that a load's
    // wait does not also wait for the W stores issued in between (fp32 W: loaded at its use,
    // which needs no extra registers)
    constexpr bool PFW = sizeof(WT) == 2;
    constexpr int ITR = SROWS * VPR / NT, ITC = BN * RVC / NT;
    static_assert(ITR % 2 == 0 && ITR * NT == SROWS * VPR && ITC % 2 == 0 && ITC * NT == BN * RVC,
                  "passes in pairs of iterations");
    typename VecIO<WT>::raw w0, w1;
    if (!p.w_trans) {
      auto w_at = [&](int i, bool& h) {
        const int r = srow0 + i / VPR, c = col0 + (i % VPR) * 8;
        h = r < p.M && c < p.N;
        return h ? (int64_t)r * p.ldw + c : (int64_t)0;
      };
      auto fetch_w = [&](int i, typename VecIO<WT>::raw& w) {
        bool h;
        const int64_t wi = w_at(i, h);
        if (PFW) w = VecIO<WT>::load_raw(Wb, wi);
        return h;
      };
      auto row_vec = [&](int idx, const typename VecIO<WT>::raw& w, bool) {
        bool h;
        const int64_t wi = w_at(idx, h);
        const int lr = idx / VPR, lc = (idx - lr * VPR) * 8;
        const float* cs = Cs + lr * CP + lc;
        const f32x4 a = *reinterpret_cast<const f32x4*>(cs), b = *reinterpret_cast<const f32x4*>(cs + 4);
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        update(wi, h, PFW ? w : VecIO<WT>::load_raw(Wb, wi), v);
      };
      bool h0 = fetch_w(tid, w0);
#pragma unroll 1
      for (int it = 0; it < ITR; it += 2) {
        const int idx = tid + it * NT;
        const bool h1 = fetch_w(idx + NT, w1);
        row_vec(idx, w0, h0);
        if (it + 2 < ITR) h0 = fetch_w(idx + 2 * NT, w0);
        row_vec(idx + NT, w1, h1);
      }
    } else {
      // W is the caller's m x n matrix: column c of this n x m tile is row c of W
      auto pos = [&](int i, int& lr, int& lc) {
        const int ci = i & 15, ri = (i >> 4) & 3, blk = i >> 6;
        const int cb = blk % (BN / 16), rb = blk / (BN / 16);
        lc = cb * 16 + ci;
        lr = (rb * 4 + ri) * 8;
      };
      auto w_at = [&](int i, bool& h) {
        int lr, lc;
        pos(i, lr, lc);
        const int r = srow0 + lr, c = col0 + lc;
        h = c < p.N && r < p.M;
        return h ? (int64_t)c * p.ldw + r : (int64_t)0;
      };
      auto fetch_w = [&](int i, typename VecIO<WT>::raw& w) {
        bool h;
        const int64_t wi = w_at(i, h);
        if (PFW) w = VecIO<WT>::load_raw(Wb, wi);
        return h;
      };
      auto col_vec = [&](int idx, const typename VecIO<WT>::raw& w, bool) {
        bool h;
        const int64_t wi = w_at(idx, h);
        int lr, lc;
        pos(idx, lr, lc);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Cs[(lr + e) * CP + lc];
        update(wi, h, PFW ? w : VecIO<WT>::load_raw(Wb, wi), v);
      };
      bool h0 = fetch_w(tid, w0);
#pragma unroll 1
      for (int it = 0; it < ITC; it += 2) {
        const int idx = tid + it * NT;
        const bool h1 = fetch_w(idx + NT, w1);
        col_vec(idx, w0, h0);
        if (it + 2 < ITC) h0 = fetch_w(idx + 2 * NT, w0);
        col_vec(idx + NT, w1, h1);
      }
    }
    lds_barrier();
  }
  if (p.flags && __builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(p.flags + mat, 4);
}

// EPI selects the epilogue at compile time: 0 = generic (any dtypes, caller buffers, weight
// update, flags); 1..5 = the typed fast epilogue (1: f16 out / f16 E, 2: bf16 / bf16,
// 3: f16 / bf16, 4: bf16 / f16, 5: f32 / f32); 6..8 = the weight update alone (W bf16, f16,
// f32).
// SHAPE: 0 = full product (both operands K-contiguous), 1 = symmetric product of n x n
// iterates, 2 = Gram (X X^T), 3 = rectangular product with the k-major right operand (Q X,
// B X); 1 and 2 run the same code (triangle tiles) and differ only in the kernel symbol, so
// that profiles separate the long-K Gram products from the n x n ones.
template <typename T, int SHAPE, class CFG, int EPI>
__global__ void __launch_bounds__(CFG::NT) __attribute__((amdgpu_waves_per_eu(CFG::OCC, CFG::OCC)))
gemm_nt_kernel(const GemmBatch gb) {
  constexpr bool TRI = SHAPE == 1 || SHAPE == 2;
  constexpr bool BKM = SHAPE == 3;
  constexpr int ES = MfmaTraits<T>::ES;
  constexpr int EPC = 16 / ES;     // elements per 16-byte chunk
  constexpr int BK = CFG::CPR * EPC;  // elements of K per stage
  constexpr int BM = CFG::BM, BN = CFG::BN, NT = CFG::NT, ROWB = CFG::ROWB;
  constexpr int TM = CFG::TM, TN = CFG::TN, WTM = CFG::WTM, WTN = CFG::WTN, CP = CFG::CP;
  __shared__ __attribute__((aligned(16))) char lds[CFG::LDS];

  // the wave index is uniform across a wave: keep it (and everything derived) in SGPRs
  const int tid = threadIdx.x, lane0 = tid & 63, wave = wave_uniform(tid >> 6);
  const int wm = wave / CFG::WVN, wn = wave % CFG::WVN;

  // Persistent: each workgroup walks a strided sequence of tiles inside its XCD's contiguous
  // share of the tile list, so concurrently running tiles of one XCD are neighbours (same
  // matrix, shared operand panels in that XCD's L2). The next tile's first k-stage is issued
  // right after a tile's epilogue; waiting for it also waits for that epilogue's stores (one
  // vector-memory counter covers both), and the whole first-stage wait is 2-3 us per tile.
  constexpr int NXCD = 8;
  const int xcd = blockIdx.x % NXCD, wgx = blockIdx.x / NXCD, per_xcd = gridDim.x / NXCD;
  int xtiles = 0;  // this XCD's share: part xcd of every group, one group after another
  for (int g = 0; g < gb.ng; ++g)
    xtiles += xcd_part_lo(gb.g[g].nblocks, xcd + 1) - xcd_part_lo(gb.g[g].nblocks, xcd);
  for (int j = wgx; j < xtiles; j += per_xcd) {
  // the lane's offsets (main loop and epilogue) are recomputed for every tile instead of being
  // kept across tiles
  int lane_t = lane0;
  __asm__ __volatile__("" : "+v"(lane_t));
  const int lane = lane_t;
  int gi = 0, jj = j;
  for (;;) {
    const int ps = xcd_part_lo(gb.g[gi].nblocks, xcd + 1) - xcd_part_lo(gb.g[gi].nblocks, xcd);
    if (jj < ps || gi + 1 == gb.ng) break;
    jj -= ps;
    ++gi;
  }
  const GemmArgs& p = gb.g[gi];
  const int glid = xcd_part_lo(p.nblocks, xcd) + jj;
  const int mat = glid / p.tiles_per_mat;
  int t = glid - mat * p.tiles_per_mat;
  int ti, tj;
  if constexpr (TRI) {
    const int nt = p.tiles_n;
    ti = 0;
    while (t >= nt - ti) { t -= nt - ti; ++ti; }
    tj = ti + t;
  } else {
    // grouped order: consecutive tiles walk down `group_m` tile rows, then move one tile
    // column right, so concurrently running tiles share both operands' panels in L2
    const int per = p.group_m * p.tiles_n;
    const int grp = t / per, first = grp * p.group_m;
    const int gsz = min(p.group_m, p.tiles_m - first);
    const int r = t - grp * per;
    ti = first + r % gsz;
    tj = r / gsz;
  }
  const int row0 = ti * BM, col0 = tj * BN;

  const char* Ab = reinterpret_cast<const char*>(p.A) + (int64_t)mat * p.sA * ES;
  const char* Bb = reinterpret_cast<const char*>(p.B) + (int64_t)mat * p.sB * ES;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(Ab, (uint32_t)((int64_t)p.M * p.lda * ES));
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Bb, (uint32_t)((int64_t)(BKM ? p.K : p.N) * p.ldb * ES));

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if constexpr (CFG::DL) {
    // ---- DMA main loop: global -> LDS without registers, NST-deep ring of k-stages
    constexpr int KB = CFG::KB, CPR = CFG::CPR, NST = CFG::NST, PD = NST - 1;
    constexpr int RPB = 1024 / KB;                 // rows per 1 KB DMA block (one wave instruction)
    constexpr int NBA = BM / RPB, NBB = BN / RPB;
    constexpr int NWAVE = NT / 64;
    constexpr int D = (NBA + NBB) / NWAVE;         // DMA instructions per wave per stage
    static_assert(D * NWAVE == NBA + NBB, "DMA blocks must divide over the waves");
    static_assert(D * (PD > 0 ? PD : 1) < 64, "vmcnt range");
    // per instruction j: LDS byte offset within a stage, operand, global byte offset (no k),
    // and the chunk's k offset (elements)
    uint32_t goff[D];
    int kchunk[D];
    int ldsoff[D];
    bool isA[D];
    const int rib = lane / CPR, pch = lane % CPR;
    // k-major B: a 1 KB block is KRB k-rows of BN values (CPK chunks each)
    constexpr int CPK = BN * ES / 16, KRB = 1024 / (BN * ES);
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int blk = wave * D + j;
      isA[j] = blk < NBA;
      if (BKM && !isA[j]) {
        const int krow = (blk - NBA) * KRB + lane / CPK;
        const int logical = (lane % CPK) ^ kmajor_swizzle(krow & 3);
        const int gcol = col0 + logical * EPC;
        goff[j] = gcol < p.N ? (uint32_t)(krow * p.ldb * ES + gcol * ES) : OOB;
        kchunk[j] = krow;
      } else {
        const int lrow = (isA[j] ? blk : blk - NBA) * RPB + rib;   // tile-local row
        const int logical = pch ^ chunk_swizzle<CPR>(lrow);
        const int grow = (isA[j] ? row0 : col0) + lrow;
        const int lim = isA[j] ? p.M : p.N;
        const int64_t ld = isA[j] ? p.lda : p.ldb;
        goff[j] = grow < lim ? (uint32_t)(grow * ld * ES + logical * 16) : OOB;
        kchunk[j] = logical * EPC;
      }
      ldsoff[j] = isA[j] ? blk * 1024 : BM * KB + (blk - NBA) * 1024;
    }
    const int nk = (p.K + BK - 1) / BK;
    auto issue = [&](int ks) {
      char* sb = lds + (ks % NST) * CFG::STG;
      const int k0 = ks * BK;
#pragma unroll
      for (int j = 0; j < D; ++j) {
        uint32_t off;
        if constexpr (BKM)  // k-major B advances by whole rows of ldb elements per unit of k
          off = (k0 + kchunk[j] < p.K) ? goff[j] + (uint32_t)k0 * (isA[j] ? (uint32_t)ES : (uint32_t)(p.ldb * ES)) : OOB;
        else
          off = (k0 + kchunk[j] < p.K) ? goff[j] + (uint32_t)(k0 * ES) : OOB;
        dma16(isA[j] ? rsA : rsB, sb + ldsoff[j], off);
      }
    };
    // wait until at most m stages' DMAs (of this wave) are still in flight
    auto wait_stages = [&](int m) {
      if (m >= 3) wait_vmcnt<(3 * D < 64 ? 3 * D : 63)>();
      else if (m == 2) wait_vmcnt<2 * D>();
      else if (m == 1) wait_vmcnt<D>();
      else wait_vmcnt<0>();
    };
    const int sw = chunk_swizzle<CPR>(lane & 31);
    typedef typename Frag<T>::type F;
    F fa[TM], fb[TN];
    int boff[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) boff[j] = BKM ? kmajor_frag_off<BN * ES>(lane, wn * WTN + j * 32) : 0;
#pragma unroll
    for (int s_ = 0; s_ < PD; ++s_)
      if (s_ < nk) issue(s_);
    wait_stages(min(PD, nk) - 1);
    barrier_nofence();
    for (int kt = 0; kt < nk; ++kt) {
      // the previous stage's last k-group, whose fragments were read before the barrier: these
      // MFMAs keep the pipe busy while this stage's first fragments are read
      if (kt > 0) mma<T, TM, TN>(fa, fb, acc);
      if (kt + PD < nk) issue(kt + PD);
      const char* sb = lds + (kt % NST) * CFG::STG;
      const char* As = sb + (wm * WTM) * KB;
      const char* Bs = sb + (BM + wn * WTN) * KB;
      // fragment addresses are recomputed every stage instead of being kept per stage slot
      int swv = sw;
      __asm__ __volatile__("" : "+v"(swv));
      int boffv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        boffv[j] = boff[j];
        __asm__ __volatile__("" : "+v"(boffv[j]));
      }
#pragma unroll
      for (int g = 0; g < CFG::NG; ++g) {
        if constexpr (BKM && ES == 2) {
          load_frags_dl<T, TM, TN, KB, false>(As, Bs, lane, g, swv, fa, fb);
          load_b_kmajor<T, TN, BN * ES>(sb + BM * KB, boffv, g, fb);
        } else if constexpr (BKM) {
          load_frags_dl<T, TM, TN, KB, false>(As, Bs, lane, g, swv, fa, fb);
          load_b_kmajor_f32<TN, BN * ES>(sb + BM * KB, lane, wn * WTN, g, fb);
        } else {
          load_frags_dl<T, TM, TN, KB>(As, Bs, lane, g, swv, fa, fb);
        }
        if (g + 1 < CFG::NG) mma<T, TM, TN>(fa, fb, acc);
      }
      // the deferred fragments must be in registers before the next DMA refills their slot
      wait_lgkmcnt0();
      // stage kt + 1 must have landed; stages kt + 2 .. min(kt + PD, nk - 1) may be in flight
      if (kt + 1 < nk) wait_stages(min(kt + PD, nk - 1) - (kt + 1));
      barrier_nofence();
      pin_frags<T, TM, TN>(fa, fb);
    }
    mma<T, TM, TN>(fa, fb, acc);
  } else {
  // Global -> register staging, 16-byte chunks: chunk c = tid + NT q covers staged row
  // c / CPR, bytes 16 (c % CPR) .. +15. Row offsets are fixed per thread; rows past the end
  // get an out-of-range offset.
  constexpr int CPR = CFG::CPR, PF = CFG::PF;
  uint32_t offA[CFG::CA], offB[CFG::CB];
#pragma unroll
  for (int q = 0; q < CFG::CA; ++q) {
    const int c = tid + NT * q, ga = row0 + c / CPR;
    offA[q] = ga < p.M ? (uint32_t)(ga * p.lda * ES + (c % CPR) * 16) : OOB;
  }
  // k-major B: chunk c is logical chunk c % CPK of k-row c / CPK, stored swizzled
  constexpr int CPK = BN * ES / 16;
  int krowB[CFG::CB];
#pragma unroll
  for (int q = 0; q < CFG::CB; ++q) {
    const int c = tid + NT * q;
    if constexpr (BKM) {
      const int gcol = col0 + (c % CPK) * EPC;
      krowB[q] = c / CPK;
      offB[q] = gcol < p.N ? (uint32_t)(krowB[q] * p.ldb * ES + gcol * ES) : OOB;
    } else {
      const int gb = col0 + c / CPR;
      krowB[q] = 0;
      offB[q] = gb < p.N ? (uint32_t)(gb * p.ldb * ES + (c % CPR) * 16) : OOB;
    }
  }
  const int kc = (tid % CPR) * EPC;  // k offset of this thread's A (and row-major B) chunks
  u32x4 ra[PF][CFG::CA], rb[PF][CFG::CB];
  const int nk = (p.K + BK - 1) / BK;

  auto load_stage = [&](int k0, int set) {
    const bool kin = k0 + kc < p.K;
    const uint32_t kb = (uint32_t)(k0 * ES);
#pragma unroll
    for (int q = 0; q < CFG::CA; ++q)
      ra[set][q] = __builtin_amdgcn_raw_buffer_load_b128(rsA, kin ? offA[q] + kb : OOB, 0, 0);
    if constexpr (BKM) {
      const uint32_t kbB = (uint32_t)k0 * (uint32_t)(p.ldb * ES);
#pragma unroll
      for (int q = 0; q < CFG::CB; ++q)
        rb[set][q] = __builtin_amdgcn_raw_buffer_load_b128(rsB, k0 + krowB[q] < p.K ? offB[q] + kbB : OOB, 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < CFG::CB; ++q)
        rb[set][q] = __builtin_amdgcn_raw_buffer_load_b128(rsB, kin ? offB[q] + kb : OOB, 0, 0);
    }
  };
  auto store_stage = [&](int buf, int set) {
    char* As_ = lds + buf * CFG::STAGE;
    char* Bs_ = As_ + BM * ROWB;
#pragma unroll
    for (int q = 0; q < CFG::CA; ++q) {
      const int c = tid + NT * q;
      *reinterpret_cast<u32x4*>(As_ + (c / CPR) * ROWB + (c % CPR) * 16) = ra[set][q];
    }
#pragma unroll
    for (int q = 0; q < CFG::CB; ++q) {
      const int c = tid + NT * q;
      if constexpr (BKM)
        *reinterpret_cast<u32x4*>(Bs_ + krowB[q] * (BN * ES) + (((c % CPK) ^ kmajor_swizzle(krowB[q] & 3)) << 4)) = rb[set][q];
      else
        *reinterpret_cast<u32x4*>(Bs_ + (c / CPR) * ROWB + (c % CPR) * 16) = rb[set][q];
    }
  };


  typedef typename Frag<T>::type F;
  F fa[TM], fb[TN];
  int boff[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) boff[j] = BKM ? kmajor_frag_off<BN * ES>(lane, wn * WTN + j * 32) : 0;
  // Prologue: stage 0 in LDS, stages 1 .. PF-1 in flight in register sets 1 .. PF-1.
#pragma unroll
  for (int s_ = 0; s_ < PF; ++s_)
    if (s_ < nk) load_stage(s_ * BK, s_);
  store_stage(0, 0);
  __syncthreads();

  // One k-stage: compute from LDS buffer `cur`, prefetch stage kt + PF into register set
  // kt % PF (freed when stage kt went to LDS), then move stage kt + 1 from its register set
  // into the other LDS buffer. Register sets are compile-time indices (the loop below is
  // unrolled by a multiple of PF and 2).
  auto step = [&](int kt, auto cur_c, auto set_c, auto next_set_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int set = decltype(set_c)::value;
    constexpr int nset = decltype(next_set_c)::value;
    if (kt + PF < nk) load_stage((kt + PF) * BK, set);
    const char* As = lds + cur * CFG::STAGE + (wm * WTM) * ROWB;
    const char* Bs = lds + cur * CFG::STAGE + (BM + wn * WTN) * ROWB;
    // one fragment set: the other waves of the SIMD cover the LDS latency
#pragma unroll
    for (int g = 0; g < CFG::NG; ++g) {
      if constexpr (BKM && ES == 2) {
        load_frags<T, TM, TN, ROWB, false>(As, Bs, lane, g, fa, fb);
        load_b_kmajor<T, TN, BN * ES>(lds + cur * CFG::STAGE + BM * ROWB, boff, g, fb);
      } else if constexpr (BKM) {
        load_frags<T, TM, TN, ROWB, false>(As, Bs, lane, g, fa, fb);
        load_b_kmajor_f32<TN, BN * ES>(lds + cur * CFG::STAGE + BM * ROWB, lane, wn * WTN, g, fb);
      } else {
        load_frags<T, TM, TN, ROWB>(As, Bs, lane, g, fa, fb);
      }
      mma<T, TM, TN>(fa, fb, acc);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1, nset);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int kt = 0;
  if constexpr (PF == 1) {
    for (; kt + 1 < nk; kt += 2) { step(kt, I0{}, I0{}, I0{}); step(kt + 1, I1{}, I0{}, I0{}); }
    if (kt < nk) step(kt, I0{}, I0{}, I0{});
  } else if constexpr (PF == 2) {
    for (; kt + 1 < nk; kt += 2) { step(kt, I0{}, I0{}, I1{}); step(kt + 1, I1{}, I1{}, I0{}); }
    if (kt < nk) step(kt, I0{}, I0{}, I1{});
  } else {
    static_assert(PF == 3, "PF must be 1, 2 or 3");
    for (; kt + 5 < nk; kt += 6) {
      step(kt, I0{}, I0{}, I1{}); step(kt + 1, I1{}, I1{}, I2{}); step(kt + 2, I0{}, I2{}, I0{});
      step(kt + 3, I1{}, I0{}, I1{}); step(kt + 4, I0{}, I1{}, I2{}); step(kt + 5, I1{}, I2{}, I0{});
    }
    if (kt < nk) step(kt, I0{}, I0{}, I1{});
    if (kt + 1 < nk) step(kt + 1, I1{}, I1{}, I2{});
    if (kt + 2 < nk) step(kt + 2, I0{}, I2{}, I0{});
    if (kt + 3 < nk) step(kt + 3, I1{}, I0{}, I1{});
    if (kt + 4 < nk) step(kt + 4, I0{}, I1{}, I2{});
  }

  }  // register-staged main loop

  // ---------------------------------------------------------------- epilogue
  if constexpr (EPI != 0) {
    if constexpr (EPI == 1) epilogue_fast<_Float16, _Float16, TRI, CFG>(p, lds, acc, mat, ti, tj, row0, col0, lane);
    else if constexpr (EPI == 2) epilogue_fast<__bf16, __bf16, TRI, CFG>(p, lds, acc, mat, ti, tj, row0, col0, lane);
    else if constexpr (EPI == 3) epilogue_fast<_Float16, __bf16, TRI, CFG>(p, lds, acc, mat, ti, tj, row0, col0, lane);
    else if constexpr (EPI == 4) epilogue_fast<__bf16, _Float16, TRI, CFG>(p, lds, acc, mat, ti, tj, row0, col0, lane);
    else if constexpr (EPI == 5) epilogue_fast<float, float, TRI, CFG>(p, lds, acc, mat, ti, tj, row0, col0, lane);
    else if constexpr (EPI == 6) epilogue_wupd<__bf16, CFG>(p, lds, acc, mat, row0, col0, lane);
    else if constexpr (EPI == 7) epilogue_wupd<_Float16, CFG>(p, lds, acc, mat, row0, col0, lane);
    else epilogue_wupd<float, CFG>(p, lds, acc, mat, row0, col0, lane);
    continue;
  } else {
  // A) finish v = s^spow (c2 acc + c1 E) + c0 [i == j] in registers
  float sc = 1.f;
  if (p.spow) {
    const float sb = p.svec[mat];
    sc = p.spow == 1 ? sb : sb * sb;
  }
  const char* Eb = p.E ? reinterpret_cast<const char*>(p.E) + (int64_t)mat * p.sE * dtype_size(p.e_dt) : nullptr;
  char* Cb = p.C ? reinterpret_cast<char*>(p.C) + (int64_t)mat * p.sC * dtype_size(p.c_dt) : nullptr;
  char* Ctb = p.Ct ? reinterpret_cast<char*>(p.Ct) + (int64_t)mat * p.sCt * dtype_size(p.ct_dt) : nullptr;
  char* Wb = p.W ? reinterpret_cast<char*>(p.W) + (int64_t)mat * p.sW * dtype_size(p.w_dt) : nullptr;
  char* Ub = p.U ? reinterpret_cast<char*>(p.U) + (int64_t)mat * p.sU * dtype_size(p.u_dt) : nullptr;
  const bool diag = TRI && ti == tj;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int r = row0 + wm * WTM + i * 32 + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
        const int c = col0 + wn * WTN + j * 32 + (lane & 31);
        float v = p.c2 * acc[i][j][rr];
        if (Eb && r < p.e_rows && c < p.e_cols) v += p.c1 * load_elem(Eb, p.e_dt, (int64_t)r * p.lde + c);
        v *= sc;
        if (r == c && r < p.M) v += p.c0;
        if (r < p.M && c < p.N) bad |= !__builtin_isfinite(v);
        acc[i][j][rr] = v;
      }

  // B) through LDS SR wave-rows at a time: row-major pass (direct stores, W update) and
  //    column-major pass (mirror / transposed stores, transposed W update), 8 elements per
  //    lane and 16-byte accesses where the buffer allows.
  float* Cs = reinterpret_cast<float*>(lds);
  constexpr int SR = CFG::SR, SROWS = SR * WTM, VPR = BN / 8, RVC = SROWS / 8;
  const bool mirror = TRI && Cb;
  const bool colpass = mirror || Ctb || (Wb && p.w_trans);
  for (int sl = 0; sl < CFG::WVM / SR; ++sl) {
    if (wm / SR == sl) {
      acc_to_slab<CFG>(Cs, acc, lane, wn, (wm % SR) * WTM);
    }
    __syncthreads();
    const int srow0 = row0 + sl * SROWS;
    if (Cb || (Wb && !p.w_trans)) {
      for (int idx = tid; idx < SROWS * VPR; idx += NT) {
        const int lr = idx / VPR, lc = (idx - lr * VPR) * 8;
        const int r = srow0 + lr, c = col0 + lc;
        const f32x4 a = *reinterpret_cast<const f32x4*>(Cs + lr * CP + lc);
        const f32x4 b = *reinterpret_cast<const f32x4*>(Cs + lr * CP + lc + 4);
        float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        if (Cb && r < p.c_rows) {
          const int lo = diag ? max(0, min(8, r - c)) : 0;  // lower-triangle part of a diagonal tile
          if (lo < 8) store_part(Cb, p.c_dt, (int64_t)r * p.ldc + c, v, lo, p.c_cols - c, p.c_vec);
        }
        if (Wb && !p.w_trans && r < p.M) {
          const int64_t wi = (int64_t)r * p.ldw + c;
          float w[8], u[8];
          const int lim = p.N - c;
          if (lim >= 8 && p.w_vec) load8(Wb, p.w_dt, wi, w);
          else {
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = e < lim ? load_elem(Wb, p.w_dt, wi + e) : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) { u[e] = p.u_scale * v[e]; w[e] = p.wd_mul * w[e] - p.lr * u[e]; }
          store_part(Wb, p.w_dt, wi, w, 0, lim, p.w_vec);
          if (Ub) store_part(Ub, p.u_dt, (int64_t)r * p.ldu + c, u, 0, lim, p.u_vec);
        }
      }
    }
    if (colpass) {
      // lanes: 16 columns x 4 row-vectors, so 4 lanes write 64 contiguous bytes of a row of C^T
      for (int idx = tid; idx < BN * RVC; idx += NT) {
        const int ci = idx & 15, ri = (idx >> 4) & 3, blk = idx >> 6;
        const int ncb = BN / 16;
        const int cb = blk % ncb, rb = blk / ncb;
        const int lc = cb * 16 + ci, lr = (rb * 4 + ri) * 8;
        if (lr >= SROWS) continue;
        const int r = srow0 + lr, c = col0 + lc;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Cs[(lr + e) * CP + lc];
        if (mirror && c < p.c_rows) {
          // element (r + e, c) goes to (c, r + e) when r + e < c on a diagonal tile
          const int hi = diag ? max(0, min(8, c - r)) : 8;
          if (hi > 0) store_part(Cb, p.c_dt, (int64_t)c * p.ldc + r, v, 0, min(hi, p.c_cols - r), p.c_vec && hi == 8);
        }
        if (Ctb && c < p.ct_rows) store_part(Ctb, p.ct_dt, (int64_t)c * p.ldct + r, v, 0, p.ct_cols - r, p.ct_vec);
        if (Wb && p.w_trans && c < p.N) {
          const int64_t wi = (int64_t)c * p.ldw + r;
          float w[8], u[8];
          const int lim = p.M - r;
          if (lim >= 8 && p.w_vec) load8(Wb, p.w_dt, wi, w);
          else {
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = e < lim ? load_elem(Wb, p.w_dt, wi + e) : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) { u[e] = p.u_scale * v[e]; w[e] = p.wd_mul * w[e] - p.lr * u[e]; }
          store_part(Wb, p.w_dt, wi, w, 0, lim, p.w_vec);
          if (Ub) store_part(Ub, p.u_dt, (int64_t)c * p.ldu + r, u, 0, lim, p.u_vec);
        }
      }
    }
    __syncthreads();
  }
  if (p.flags && bad) atomicOr(p.flags + mat, 4);
  break;  // the generic epilogue runs one tile per workgroup (no loop-carried state)
  }  // generic epilogue
  }  // tile loop
}

}  // namespace mns
