// The normalisation kernels around the q/k/v projections of a Wan2.2 block
// (Wan2.2 source reading (blog.leeguoo.com), ch. 4, "1つの block の完全な
// forward" and "3D RoPE"): the self-attention input is norm1(x) * (1 + e1) + e0
// with the modulation in fp32, and q and k each pass an RMSNorm (QK-Norm)
// after their projection.  Both kernels are HBM-bound row passes: one wave per
// token row, the row held in registers (16 bytes per lane per 512 columns:
// NCH = ceil(dim / 512) chunks, a template argument so that only the registers
// a row needs are allocated), fp32 reductions across the wave, so each row is
// read from HBM once and written once.
#pragma once

#include "common.h"

namespace wanattn {

constexpr int kMaxRowChunks = 16;                 // rows of up to 16 * 512 = 8192 columns
constexpr int kMaxRowDim = kMaxRowChunks * 512;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

struct LnModParams {
  const uint16_t* x;  // [rows, dim] bf16
  const float* e0;    // [B, dim] shift
  const float* e1;    // [B, dim] scale (applied as 1 + e1)
  uint16_t* y;        // [rows, dim] bf16
  long long rows;     // B * N
  int N, dim;         // dim a multiple of 8, at most kMaxRowDim
  float eps;
};

// y = LayerNorm(x) * (1 + e1[b]) + e0[b]: LayerNorm over dim without affine
// parameters (mean, then the mean squared deviation from it; eps inside the
// root), modulation in fp32, y rounded to bf16 (nearest even).
template <int NCH>
__global__ void __launch_bounds__(256) ln_mod_kernel(LnModParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int b = (int)(row / p.N);
  const uint16_t* xr = p.x + row * p.dim;
  u32x4 w[NCH];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    w[i] = c < p.dim ? *(const u32x4*)(xr + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16_lo(w[i][e]) + bf16_hi(w[i][e]);
  }
  const float mean = wave_sum(s) / (float)p.dim;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (i * 512 + lane * 8 >= p.dim) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(w[i][e]) - mean, d = bf16_hi(w[i][e]) - mean;
      ss += a * a + d * d;
    }
  }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)p.dim + p.eps);
  const float* e0 = p.e0 + (size_t)b * p.dim;
  const float* e1 = p.e1 + (size_t)b * p.dim;
  uint16_t* yr = p.y + row * p.dim;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    if (c >= p.dim) continue;
    const floatx4 s0 = *(const floatx4*)(e0 + c), s1 = *(const floatx4*)(e0 + c + 4);
    const floatx4 g0 = *(const floatx4*)(e1 + c), g1 = *(const floatx4*)(e1 + c + 4);
    const float sh[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    const float sc[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = (bf16_lo(w[i][e]) - mean) * inv * (1.0f + sc[2 * e]) + sh[2 * e];
      const float d = (bf16_hi(w[i][e]) - mean) * inv * (1.0f + sc[2 * e + 1]) + sh[2 * e + 1];
      o[e] = pack_bf16x2(a, d);
    }
    *(u32x4*)(yr + c) = o;
  }
}

struct RmsParams {
  uint16_t* q;          // [rows, dim] bf16, normalised in place
  uint16_t* k;          // [rows, dim] bf16, normalised in place
  const uint16_t* gq;   // [dim] bf16 weight
  const uint16_t* gk;   // [dim] bf16 weight
  long long rows;       // B * N (the grid covers 2 * rows: q rows, then k rows)
  int dim;              // a multiple of 8, at most kMaxRowDim
  float eps;
};

// x = x / sqrt(mean(x^2) + eps) * gamma over the whole row, in place, for q and k
template <int NCH>
__global__ void __launch_bounds__(256) qk_rmsnorm_kernel(RmsParams p) {
  const int lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= 2 * p.rows) return;
  const bool is_k = r >= p.rows;
  uint16_t* xr = (is_k ? p.k : p.q) + (is_k ? r - p.rows : r) * p.dim;
  const uint16_t* g = is_k ? p.gk : p.gq;
  u32x4 w[NCH];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    w[i] = c < p.dim ? *(const u32x4*)(xr + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(w[i][e]), d = bf16_hi(w[i][e]);
      ss += a * a + d * d;
    }
  }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)p.dim + p.eps);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    if (c >= p.dim) continue;
    const u32x4 gw = *(const u32x4*)(g + c);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2(bf16_lo(w[i][e]) * inv * bf16_lo(gw[e]), bf16_hi(w[i][e]) * inv * bf16_hi(gw[e]));
    *(u32x4*)(xr + c) = o;
  }
}

struct RmsStatParams {
  const uint16_t* q;    // [rows, dim] bf16 (q, k projections before the RMSNorm)
  const uint16_t* k;
  float* rms;           // [2][rows]: 1 / sqrt(mean(x^2) + eps) of each q row, then each k row
  long long rows;
  int dim;
  float eps;
};

// The RMSNorm's factor of every q and k row, the rows left as they are: the
// attention call applies x * factor * gamma where it reads q and rotates k.
// One wave per row; reads each row once and writes one float.
template <int NCH>
__global__ void __launch_bounds__(256) qk_rms_stats_kernel(RmsStatParams p) {
  const int lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= 2 * p.rows) return;
  const bool is_k = r >= p.rows;
  const uint16_t* xr = (is_k ? p.k : p.q) + (is_k ? r - p.rows : r) * p.dim;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i * 512 + lane * 8;
    if (c >= p.dim) continue;
    const u32x4 w = *(const u32x4*)(xr + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(w[e]), d = bf16_hi(w[e]);
      ss += a * a + d * d;
    }
  }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)p.dim + p.eps);
  if (lane == 0) p.rms[r] = inv;
}

// launch either kernel with NCH = ceil(dim / 512) (1 <= NCH <= kMaxRowChunks)
template <template <int> class Launch, typename P>
hipError_t launch_rows(int dim, dim3 grid, hipStream_t st, const P& p) {
  switch ((dim + 511) / 512) {
#define WANATTN_ROWS_CASE(n) \
  case n: return Launch<n>::run(grid, st, p);
    WANATTN_ROWS_CASE(1) WANATTN_ROWS_CASE(2) WANATTN_ROWS_CASE(3) WANATTN_ROWS_CASE(4)
    WANATTN_ROWS_CASE(5) WANATTN_ROWS_CASE(6) WANATTN_ROWS_CASE(7) WANATTN_ROWS_CASE(8)
    WANATTN_ROWS_CASE(9) WANATTN_ROWS_CASE(10) WANATTN_ROWS_CASE(11) WANATTN_ROWS_CASE(12)
    WANATTN_ROWS_CASE(13) WANATTN_ROWS_CASE(14) WANATTN_ROWS_CASE(15) WANATTN_ROWS_CASE(16)
#undef WANATTN_ROWS_CASE
  }
  return hipErrorInvalidValue;
}

template <int NCH>
struct LnModLaunch {
  static hipError_t run(dim3 grid, hipStream_t st, const LnModParams& p) {
    hipLaunchKernelGGL(ln_mod_kernel<NCH>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
  }
};

template <int NCH>
struct QkRmsStatLaunch {
  static hipError_t run(dim3 grid, hipStream_t st, const RmsStatParams& p) {
    hipLaunchKernelGGL(qk_rms_stats_kernel<NCH>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
  }
};

template <int NCH>
struct QkRmsLaunch {
  static hipError_t run(dim3 grid, hipStream_t st, const RmsParams& p) {
    hipLaunchKernelGGL(qk_rmsnorm_kernel<NCH>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
  }
};

}  // namespace wanattn
