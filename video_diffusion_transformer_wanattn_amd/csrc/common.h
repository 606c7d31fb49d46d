// Shared device helpers for the wanattn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wanattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kPairs = kHeadDim / 2;          // 64 complex pairs per head vector
constexpr int kMaxPos = 1024;                 // rows of each axis table
constexpr int kTabStride = 32;                // float2 entries per (axis, position) row
// Pairs per axis for head_dim 128: time 44/2, height 42/2, width 42/2.
constexpr int kPairsT = 22, kPairsH = 21, kPairsW = 21;
constexpr int kFirstPairH = kPairsT, kFirstPairW = kPairsT + kPairsH;  // 22, 43

// Rotary table: float2 (cos, sin) of pos * theta^(-2k/D_axis), laid out as
// tab[(axis * kMaxPos + pos) * kTabStride + k].
constexpr int kTabEntries = 3 * kMaxPos * kTabStride;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two floats -> packed bf16x2 (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// axis (0 time, 1 height, 2 width) and index within the axis of complex pair c
__device__ __forceinline__ int pair_axis(int c) { return c < kFirstPairH ? 0 : (c < kFirstPairW ? 1 : 2); }
__device__ __forceinline__ int pair_index(int c) {
  return c < kFirstPairH ? c : (c < kFirstPairW ? c - kFirstPairH : c - kFirstPairW);
}

// Exact n / d and n % d for 0 <= n < 2^31, d >= 1, through fp64 with one
// correction step (the fp64 quotient is off by at most one).
__device__ __forceinline__ void divmod(int n, int d, double inv_d, int& q, int& r) {
  q = (int)((double)n * inv_d);
  r = n - q * d;
  if (r < 0) { q -= 1; r += d; }
  if (r >= d) { q += 1; r -= d; }
}

// value of lane l ^ 32 combined with our own: permlane32_swap(x, x) returns
// (x[l & 31], x[l | 32]) on every lane, which covers both halves of the wave.
__device__ __forceinline__ float wave_half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace wanattn
