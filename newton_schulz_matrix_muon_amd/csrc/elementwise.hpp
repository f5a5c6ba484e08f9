// HBM-bound kernels around the products:
//  - prep_kernel: reads one 64 x 64 tile of a caller matrix (any dtype/ld/stride), writes it
//    to the internal n x m row-major X the products read (a straight copy, or the transpose
//    when the caller's matrix is m x n), zero-fills its padded columns, and emits a
//    deterministic per-tile partial of sum x^2 (the Frobenius norm, guide's normalisation).
//    With momentum enabled it first applies the Muon momentum rule to the fp32 buffer M and
//    orthogonalizes N instead of G. prep_vec_kernel is the same tile walk in 16-byte vectors
//    for aligned buffers; prep_stream_kernel streams whole rows when no transpose is needed.
//  - finalize_kernel: sums the partials of one matrix in a fixed order, s = 1/(sqrt + eps),
//    and writes the per-matrix flags.
//  - copy2d_kernel: strided copy with dtype conversion (the Gram-iterate trace).
#pragma once

#include "common.hpp"

namespace mns {

struct PrepArgs {
  const void* G; int g_dt; int64_t ldg, sg;
  int rows, cols;                      // caller orientation
  void* out_same; int64_t ld_same, s_same;   // rows x ld_same (pad cols zero), or null
  void* out_tr; int64_t ld_tr, s_tr;         // cols x ld_tr   (pad cols zero), or null
  int io_dt;
  double* partials;                    // [batch][tiles]
  int tiles_x, tiles;                  // tiles_x = ceil(cols/64)
  // momentum (optional)
  float* M; int64_t ldm, sm;
  float mu; int nesterov;
};

constexpr int PREP_T = 64;

__global__ void __launch_bounds__(256) prep_kernel(const PrepArgs p) {
  __shared__ float tile[PREP_T][PREP_T + 1];
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int mat = blockIdx.y;
  const int tx = blockIdx.x % p.tiles_x, ty = blockIdx.x / p.tiles_x;
  const int r0 = ty * PREP_T, c0 = tx * PREP_T;
  const int es = dtype_size(p.g_dt), ios = dtype_size(p.io_dt);
  const char* Gb = reinterpret_cast<const char*>(p.G) + (int64_t)mat * p.sg * es;
  float* Mb = p.M ? p.M + (int64_t)mat * p.sm : nullptr;
  char* Sb = p.out_same ? reinterpret_cast<char*>(p.out_same) + (int64_t)mat * p.s_same * ios : nullptr;
  char* Tb = p.out_tr ? reinterpret_cast<char*>(p.out_tr) + (int64_t)mat * p.s_tr * ios : nullptr;

  // load: thread -> 4 consecutive columns of rows ty + 16q
  const int cc = (tid & 15) * 4, rbase = tid >> 4;
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = rbase + 16 * q, r = r0 + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + cc + e;
      float v = 0.f;
      if (r < p.rows && c < p.cols) {
        v = load_elem(Gb, p.g_dt, (int64_t)r * p.ldg + c);
        if (Mb) {
          const int64_t mi = (int64_t)r * p.ldm + c;
          const float m = p.mu * Mb[mi] + (1.f - p.mu) * v;
          Mb[mi] = m;
          v = p.nesterov ? p.mu * m + (1.f - p.mu) * v : m;
        }
        // round to the internal dtype first: the norm is of the values the products read
        if (p.io_dt == BF16) v = bf16_bits_to_f32(f32_to_bf16_bits(v));
        else if (p.io_dt == F16) v = f16_bits_to_f32(f32_to_f16_bits(v));
      }
      tile[lr][cc + e] = v;
      ss += (double)v * (double)v;
    }
  }
  __syncthreads();
  // same orientation: rows r < rows, columns c < ld_same (pad written as zero)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = rbase + 16 * q, r = r0 + lr;
    if (!Sb || r >= p.rows) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + cc + e;
      if (c < p.ld_same) store_elem(Sb, p.io_dt, (int64_t)r * p.ld_same + c, tile[lr][cc + e]);
    }
  }
  // transposed: row c (< cols), column r (< ld_tr)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lc = rbase + 16 * q, c = c0 + lc;
    if (!Tb || c >= p.cols) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + cc + e;
      if (r < p.ld_tr) store_elem(Tb, p.io_dt, (int64_t)c * p.ld_tr + r, tile[cc + e][lc]);
    }
  }
  // fixed-order block reduction of the partial sum of squares
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) p.partials[(int64_t)mat * p.tiles + blockIdx.x] = red[0];
}


// Vectorised prep for aligned buffers (ld, stride and base multiples of 8 elements / 16 B):
// a 64 x 64 tile, each thread moves two 8-element vectors per direction. T is the input
// dtype, which is also the internal dtype of the copies.
template <typename T>
__device__ inline void ld8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t lo = (uint16_t)(w[e] & 0xffffu), hi = (uint16_t)(w[e] >> 16);
      if constexpr (__is_same(T, __bf16)) { v[2 * e] = bf16_bits_to_f32(lo); v[2 * e + 1] = bf16_bits_to_f32(hi); }
      else { v[2 * e] = f16_bits_to_f32(lo); v[2 * e + 1] = f16_bits_to_f32(hi); }
    }
  }
}

template <typename T>
__device__ inline void st8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack2<T>(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
}

template <typename T>
__device__ inline float round_to(float v) {
  if constexpr (__is_same(T, __bf16)) return bf16_bits_to_f32(f32_to_bf16_bits(v));
  else if constexpr (__is_same(T, _Float16)) return f16_bits_to_f32(f32_to_f16_bits(v));
  else return v;
}

template <typename T>
__global__ void __launch_bounds__(256) prep_vec_kernel(const PrepArgs p) {
  __shared__ float tile[PREP_T][PREP_T + 4];
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int mat = blockIdx.y;
  const int tx = blockIdx.x % p.tiles_x, ty = blockIdx.x / p.tiles_x;
  const int r0 = ty * PREP_T, c0 = tx * PREP_T;
  const T* Gb = reinterpret_cast<const T*>(p.G) + (int64_t)mat * p.sg;
  float* Mb = p.M ? p.M + (int64_t)mat * p.sm : nullptr;
  T* Sb = p.out_same ? reinterpret_cast<T*>(p.out_same) + (int64_t)mat * p.s_same : nullptr;
  T* Tb = p.out_tr ? reinterpret_cast<T*>(p.out_tr) + (int64_t)mat * p.s_tr : nullptr;
  // thread -> rows (tid >> 3) and (tid >> 3) + 32, columns 8 (tid & 7) .. + 7
  const int cv = (tid & 7) * 8;
  double ss = 0.0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int lr = (tid >> 3) + 32 * h, r = r0 + lr, c = c0 + cv;
    float v[8];
    if (r < p.rows && c < p.cols) {  // cols % 8 == 0: the vector is whole
      const int64_t gi = (int64_t)r * p.ldg + c;
      ld8<T>(Gb + gi, v);
      if (Mb) {
        const int64_t mi = (int64_t)r * p.ldm + c;
        float m[8];
        ld8<float>(Mb + mi, m);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          m[e] = p.mu * m[e] + (1.f - p.mu) * v[e];
          v[e] = p.nesterov ? p.mu * m[e] + (1.f - p.mu) * v[e] : m[e];
        }
        st8<float>(Mb + mi, m);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = round_to<T>(v[e]);
        ss += (double)v[e] * (double)v[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    if (Sb && r < p.rows && c < p.ld_same) st8<T>(Sb + (int64_t)r * p.ld_same + c, v);
    if (Tb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[lr][cv + e] = v[e];
    }
  }
  __syncthreads();
  // transposed: thread -> tile column (tid >> 3) and +32, rows 8 (tid & 7) .. + 7
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int lc = (tid >> 3) + 32 * h, c = c0 + lc, r = r0 + cv;
    if (Tb && c < p.cols && r < p.ld_tr) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[cv + e][lc];
      st8<T>(Tb + (int64_t)c * p.ld_tr + r, v);
    }
  }
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) p.partials[(int64_t)mat * p.tiles + blockIdx.x] = red[0];
}

// Streaming prep for the common case: X in the caller's orientation (rows <= cols), aligned
// buffers, cols a multiple of 8 (so X has no padded columns). Block b of a matrix handles the
// 512 consecutive 8-element vectors from 512 b on (two per thread, 256 apart: every wave
// reads and writes contiguous runs), with the arithmetic of prep_vec_kernel and a fixed-order
// reduction of its partial sum of squares.
constexpr int PREP_SV = 512;

template <typename T>
__global__ void __launch_bounds__(256) prep_stream_kernel(const PrepArgs p) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int mat = blockIdx.y;
  const int vpr = p.cols / 8;
  const int64_t nvec = (int64_t)p.rows * vpr;
  const T* Gb = reinterpret_cast<const T*>(p.G) + (int64_t)mat * p.sg;
  float* Mb = p.M ? p.M + (int64_t)mat * p.sm : nullptr;
  T* Sb = reinterpret_cast<T*>(p.out_same) + (int64_t)mat * p.s_same;
  double ss = 0.0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t v = (int64_t)blockIdx.x * PREP_SV + h * 256 + tid;
    if (v >= nvec) continue;
    const int64_t r = v / vpr;
    const int c = (int)(v - r * vpr) * 8;
    float x[8];
    ld8<T>(Gb + r * p.ldg + c, x);
    if (Mb) {
      const int64_t mi = r * p.ldm + c;
      float m[8];
      ld8<float>(Mb + mi, m);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        m[e] = p.mu * m[e] + (1.f - p.mu) * x[e];
        x[e] = p.nesterov ? p.mu * m[e] + (1.f - p.mu) * x[e] : m[e];
      }
      st8<float>(Mb + mi, m);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = round_to<T>(x[e]);
      ss += (double)x[e] * (double)x[e];
    }
    st8<T>(Sb + r * p.ld_same + c, x);
  }
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) p.partials[(int64_t)mat * p.tiles + blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(256) finalize_kernel(const double* partials, int tiles,
                                                       float eps, float* svec,
                                                       int32_t* flags) {
  __shared__ double red[256];
  const int tid = threadIdx.x, mat = blockIdx.x;
  double s = 0.0;
  for (int i = tid; i < tiles; i += 256) s += partials[(int64_t)mat * tiles + i];
  red[tid] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (tid < k) red[tid] += red[tid + k];
    __syncthreads();
  }
  if (tid == 0) {
    const double ss = red[0];
    const double nrm = sqrt(ss);
    svec[mat] = (float)(1.0 / (nrm + (double)eps));
    if (flags) flags[mat] = (__builtin_isfinite(ss) ? 0 : 1) | (ss == 0.0 ? 2 : 0);
  }
}

// rows x cols copy with dtype conversion between two strided 2-D buffers (diagnostics)
__global__ void __launch_bounds__(256) copy2d_kernel(const void* src, int s_dt, int64_t lds_, void* dst,
                                                     int d_dt, int64_t ldd, int rows, int cols) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols, c = i - r * cols;
    store_elem(dst, d_dt, r * ldd + c, load_elem(src, s_dt, r * lds_ + c));
  }
}

}  // namespace mns
