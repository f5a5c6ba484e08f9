// AdamW for the parameters Muon does not take (RMSNorm scales, biases, router projections,
// token embeddings): one launch updates a table of flat tensors. Purely HBM-bound: per element
// it reads the parameter, gradient and both fp32 moments and writes the parameter and moments.
#pragma once

#include "common.hpp"

namespace mns {

constexpr int ADAM_MAXT = 48;                 // tensors per launch (kernel-argument table)
constexpr int ADAM_BLOCK = 256;
constexpr int ADAM_EPT = 4;                   // consecutive elements per thread and iteration
constexpr int ADAM_ITERS = 4;
constexpr int ADAM_CHUNK = ADAM_BLOCK * ADAM_EPT * ADAM_ITERS;   // elements per workgroup

struct AdamTable {
  void* p[ADAM_MAXT];
  const void* g[ADAM_MAXT];
  float* m[ADAM_MAXT];
  float* v[ADAM_MAXT];
  int64_t numel[ADAM_MAXT];
  int blk_start[ADAM_MAXT + 1];               // first workgroup of each tensor
  int nt;
  float lr, beta1, beta2, eps, wd_mul;        // wd_mul = 1 - lr * weight_decay
  float bc1, bc2;                             // bias-correction factors (1 when off)
};

template <typename PT>
__device__ inline float ld_param(const PT* p, int64_t i) {
  if constexpr (sizeof(PT) == 4) return p[i];
  else if constexpr (__is_same(PT, __bf16)) return bf16_bits_to_f32(__builtin_bit_cast(uint16_t, p[i]));
  else return (float)p[i];
}
template <typename PT>
__device__ inline float bits_to_f32(uint16_t h) {
  if constexpr (__is_same(PT, __bf16)) return bf16_bits_to_f32(h); else return f16_bits_to_f32(h);
}
template <typename PT>
__device__ inline PT to_param(float x) {
  if constexpr (sizeof(PT) == 4) return x;
  else if constexpr (__is_same(PT, __bf16)) return __builtin_bit_cast(__bf16, f32_to_bf16_bits(x));
  else return __builtin_bit_cast(_Float16, f32_to_f16_bits(x));
}

// m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2; p <- (1 - lr wd) p - lr m^ / (sqrt(v^) + eps)
__device__ inline void adam_elem(const AdamTable& t, float g, float& m, float& v, float& p) {
  m = t.beta1 * m + (1.f - t.beta1) * g;
  v = t.beta2 * v + (1.f - t.beta2) * (g * g);
  const float upd = (m * t.bc1) / (__builtin_sqrtf(v * t.bc2) + t.eps);
  p = t.wd_mul * p - t.lr * upd;
}

template <typename PT>
__global__ void __launch_bounds__(ADAM_BLOCK) adamw_kernel(const AdamTable t) {
  int ti = 0;
  while (ti + 1 < t.nt && (int)blockIdx.x >= t.blk_start[ti + 1]) ++ti;
  const int64_t n = t.numel[ti];
  const int64_t base = (int64_t)((int)blockIdx.x - t.blk_start[ti]) * ADAM_CHUNK;
  PT* p = reinterpret_cast<PT*>(t.p[ti]);
  const PT* g = reinterpret_cast<const PT*>(t.g[ti]);
  float* m = t.m[ti];
  float* v = t.v[ti];
  // 4-element vectors when every buffer is aligned for them
  const bool vec = ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g)) % (4 * sizeof(PT)) == 0) &&
                   ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) % 16 == 0);
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  // all loads of the thread's vectors first (one memory latency for the lot), then the math
  float pf[ADAM_ITERS][ADAM_EPT], gf[ADAM_ITERS][ADAM_EPT];
  f32x4 mv[ADAM_ITERS], vv[ADAM_ITERS];
  bool full[ADAM_ITERS];
#pragma unroll
  for (int it = 0; it < ADAM_ITERS; ++it) {
    const int64_t e0 = base + ((int64_t)it * ADAM_BLOCK + threadIdx.x) * ADAM_EPT;
    full[it] = vec && e0 + ADAM_EPT <= n;
    if (!full[it]) continue;
    mv[it] = *reinterpret_cast<const f32x4*>(m + e0);
    vv[it] = *reinterpret_cast<const f32x4*>(v + e0);
    if constexpr (sizeof(PT) == 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p + e0), b = *reinterpret_cast<const f32x4*>(g + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) { pf[it][e] = a[e]; gf[it][e] = b[e]; }
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2*>(p + e0), b = *reinterpret_cast<const u32x2*>(g + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[it][e] = bits_to_f32<PT>((uint16_t)((e & 1) ? (a[e >> 1] >> 16) : (a[e >> 1] & 0xffffu)));
        gf[it][e] = bits_to_f32<PT>((uint16_t)((e & 1) ? (b[e >> 1] >> 16) : (b[e >> 1] & 0xffffu)));
      }
    }
  }
#pragma unroll
  for (int it = 0; it < ADAM_ITERS; ++it) {
    const int64_t e0 = base + ((int64_t)it * ADAM_BLOCK + threadIdx.x) * ADAM_EPT;
    if (full[it]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float me = mv[it][e], ve = vv[it][e];
        adam_elem(t, gf[it][e], me, ve, pf[it][e]);
        mv[it][e] = me;
        vv[it][e] = ve;
      }
      *reinterpret_cast<f32x4*>(m + e0) = mv[it];
      *reinterpret_cast<f32x4*>(v + e0) = vv[it];
      if constexpr (sizeof(PT) == 4) {
        *reinterpret_cast<f32x4*>(p + e0) = f32x4{pf[it][0], pf[it][1], pf[it][2], pf[it][3]};
      } else {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, to_param<PT>(pf[it][e]));
        *reinterpret_cast<u32x2*>(p + e0) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      }
    } else if (e0 < n) {
      // tail or unaligned tensor: element by element
      const int64_t e1 = e0 + ADAM_EPT < n ? e0 + ADAM_EPT : n;
      for (int64_t e = e0; e < e1; ++e) {
        float mf = m[e], vf = v[e], pe = ld_param<PT>(p, e);
        adam_elem(t, ld_param<PT>(g, e), mf, vf, pe);
        m[e] = mf;
        v[e] = vf;
        p[e] = to_param<PT>(pe);
      }
    }
  }
}

}  // namespace mns
