// Standalone 3D rotary embedding over a whole [B, N, heads, 128] bf16 tensor.
//
// Wan2.2 source reading (blog.leeguoo.com), ch. 4, subsection "3D RoPE": each
// token takes the table rows of its (f, h, w) coordinates for the time, height
// and width segments of the head (44/42/42 wide) and multiplies q or k by them
// as complex numbers.
//
// Memory-bound: one wave per token row (heads x 256 bytes, contiguous): lane
// (hq, dc) = (lane / 16, lane % 16) takes 16-byte chunk dc (4 complex pairs)
// of heads hq, hq + 4, hq + 8, ..., so every load and store instruction moves
// 1 KiB of the row (4 whole head vectors).  The token's (f, h, w) and the
// chunk's four (cos, sin) pairs are found once per wave and lane (with
// per-head tables, per head).  Measured at 75,600 tokens x 40 heads: 5.3 TB/s,
// against 4.9 TB/s for waves over 4 tokens' rows (256 bytes of each per
// instruction) and 4.0 TB/s with 8 loads per lane issued before any rotation.
// Bytes moved per element: 2 read + 2 written.
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
  long long tokens;  // B * N
  int N, heads, H, W;
  int f0, h0, w0;
  double inv_hw, inv_w;
};

__global__ void __launch_bounds__(256) rope3d_kernel(RopeParams p) {
  const int lane = threadIdx.x & 63;
  const int hq = lane >> 4, dc = lane & 15;
  const long long waves = (long long)gridDim.x * (blockDim.x >> 6);
  for (long long t = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < p.tokens; t += waves) {
    const unsigned tok = (unsigned)t;               // b * N + n (fewer than 2^31 tokens fit in memory)
    const int n = (int)(tok % (unsigned)p.N);       // token index in its batch
    int f, rem, h, w;
    divmod(n, p.H * p.W, p.inv_hw, f, rem);
    divmod(rem, p.W, p.inv_w, h, w);
    int row[4];                                     // table row of each pair: axis, position
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * dc + e;
      const int a = pair_axis(c);
      const int pa = a == 0 ? f + p.f0 : (a == 1 ? h + p.h0 : w + p.w0);
      row[e] = (a * kMaxPos + pa) * kTabStride + pair_index(c);
    }
    float2 cs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = p.tab[row[e]];
    const float s = p.rms ? p.rms[tok] : 1.0f;
    const u32x4* src = p.x + (size_t)tok * p.heads * 16 + dc;
    u32x4* dst = p.y + (size_t)tok * p.heads * 16 + dc;
#pragma unroll 4
    for (int hd = hq; hd < p.heads; hd += 4) {
      const u32x4 in = src[(size_t)hd * 16];
      if (p.tab_hstride != 0) {
        const float2* tab = p.tab + hd * p.tab_hstride;
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[e] = tab[row[e]];
      }
      u32x4 g = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 ones
      if (p.gamma) g = *(const u32x4*)(p.gamma + (size_t)hd * kHeadDim + 8 * dc);
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float re = bf16_lo(in[e]) * s * bf16_lo(g[e]), im = bf16_hi(in[e]) * s * bf16_hi(g[e]);
        out[e] = pack_bf16x2(re * cs[e].x - im * cs[e].y, re * cs[e].y + im * cs[e].x);
      }
      dst[(size_t)hd * 16] = out;
    }
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
