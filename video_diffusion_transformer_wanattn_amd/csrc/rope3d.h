// Standalone 3D rotary embedding over a whole [B, N, heads, 128] bf16 tensor.
//
// Wan2.2 source reading (blog.leeguoo.com), ch. 4, subsection "3D RoPE": each
// token takes the table rows of its (f, h, w) coordinates for the time, height
// and width segments of the head (44/42/42 wide) and multiplies q or k by them
// as complex numbers.
//
// Memory-bound: one thread rotates one 16-byte chunk (4 complex pairs);
// consecutive threads cover consecutive chunks, so loads and stores are fully
// coalesced.  Bytes moved per element: 2 read + 2 written.
#pragma once

#include "common.h"

namespace wanattn {

struct RopeParams {
  const u32x4* x;
  u32x4* y;
  const float2* tab;
  long long tab_hstride;  // float2 entries between consecutive heads' tables (0: one shared table)
  // optional QK-Norm applied before the rotation (null: none): x * rms[token
  // row] * gamma[head * 128 + d], rms indexed by b * N + n
  const float* rms;
  const uint16_t* gamma;
  long long chunks;  // B * N * heads * 16
  int N, heads, H, W;
  int f0, h0, w0;
  double inv_hw, inv_w;
};

__global__ void __launch_bounds__(256) rope3d_kernel(RopeParams p) {
  long long stride = (long long)gridDim.x * blockDim.x;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < p.chunks; idx += stride) {
    int dc = (int)(idx & 15);                       // 16-byte chunk in the head vector
    long long tok_head = idx >> 4;
    const long long tok = tok_head / p.heads;
    int n = (int)(tok % p.N);                       // token index in its batch
    const float2* tab = p.tab + (tok_head - tok * p.heads) * p.tab_hstride;
    int f, rem, h, w;
    divmod(n, p.H * p.W, p.inv_hw, f, rem);
    divmod(rem, p.W, p.inv_w, h, w);
    u32x4 in = p.x[idx];
    u32x4 out;
    float s = 1.0f;
    u32x4 g = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 ones
    if (p.rms) {
      s = p.rms[tok];
      g = *(const u32x4*)(p.gamma + (tok_head - tok * p.heads) * kHeadDim + 8 * dc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int c = 4 * dc + e;
      int a = pair_axis(c);
      int pa = a == 0 ? f + p.f0 : (a == 1 ? h + p.h0 : w + p.w0);
      float2 cs = tab[(a * kMaxPos + pa) * kTabStride + pair_index(c)];
      float re = bf16_lo(in[e]) * s * bf16_lo(g[e]), im = bf16_hi(in[e]) * s * bf16_hi(g[e]);
      out[e] = pack_bf16x2(re * cs.x - im * cs.y, re * cs.y + im * cs.x);
    }
    p.y[idx] = out;
  }
}

// Per-head rotary tables for multi-head RoPE jitter (long-video survey
// (atlascloud.ai), "ルート2 · LoL": a random per-head perturbation of the RoPE
// phase; here head h rotates with its own base theta_h).  Same layout as the
// shared table, one table per head: entry (axis, pos, k) of head h holds
// (cos, sin) of pos * theta_h^(-2k/D_axis) for k < D_axis / 2 and zeros after,
// computed in fp64 and rounded to fp32.
constexpr int kMaxJitterHeads = 256;

struct TableParams {
  float2* tab;                      // heads * kTabEntries entries
  int heads;
  double theta[kMaxJitterHeads];
};

__global__ void __launch_bounds__(256) rope_table_kernel(TableParams p) {
  const long long total = (long long)p.heads * kTabEntries;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int h = (int)(idx / kTabEntries);
    const int rem = (int)(idx - (long long)h * kTabEntries);
    const int k = rem % kTabStride;
    const int row = rem / kTabStride;              // axis * kMaxPos + pos
    const int a = row / kMaxPos, pos = row - a * kMaxPos;
    const int D = a == 0 ? kHeadDim - 4 * (kHeadDim / 6) : 2 * (kHeadDim / 6);
    float2 v = make_float2(0.0f, 0.0f);
    if (k < D / 2) {
      const double ang = (double)pos * pow(p.theta[h], -2.0 * k / D);
      v = make_float2((float)cos(ang), (float)sin(ang));
    }
    p.tab[idx] = v;
  }
}

}  // namespace wanattn
