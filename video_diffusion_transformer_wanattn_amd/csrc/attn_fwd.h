// Flash-style attention forward for head_dim 128 on gfx950 (wave64, bf16 MFMA).
//
// What it computes (per batch b, head, query row i):
//   o_i = sum_j p_ij v_j,  p_ij = softmax_j(q'_i . k'_j * scale) over visible j
// where q', k' are q, k rotated by the 3D RoPE of their tokens (self attention,
// Wan2.2 source reading (blog.leeguoo.com) ch. 4, "3D RoPE") or left as they
// are (cross attention to text tokens, Wan paper explainer (0h-n0.github.io),
// text-encoder section).  The N x N score matrix is never stored (ch. 8 of the
// source reading sizes it; the long-video survey (atlascloud.ai) puts it at
// ~10 GB for 32.7k tokens): scores are produced tile by tile and folded into a
// running softmax.
//
// Work decomposition
//   one workgroup = 4 waves = 256 query rows of one (batch, head); a wave owns
//   64 rows as two 32-row MFMA blocks.  Keys stream through LDS in tiles of 64,
//   double buffered, one barrier per tile.
//
// Per 64-key tile and wave:
//   S^T (keys x queries) = K' Q'^T   v_mfma_f32_32x32x16_bf16, 2 x 2 x 8 issues
//   online softmax on S^T: a lane holds 32 scores of ONE query, so row max and
//   row sum are in-lane plus one permlane32 swap
//   O^T (d x queries) += V^T P^T     2 x 4 x 4 issues; P stays in registers
//
// Key order inside a 32-key MFMA block is free (the contraction is a sum), so
// the K rows are stored in LDS permuted (bits 2 and 3 of the key index swapped):
// the S^T accumulator of lane l (half hh = l / 32) then holds, at register
// positions 8s .. 8s+7, the physical keys 16s + 8hh + 0..7 -- exactly the B
// operand layout of the PV product, so P never leaves registers.  V is kept
// row-major in LDS and read with ds_read_b64_tr_b16, which hands each lane
// four keys of one d column.
//
// Softmax is in base 2: the query is multiplied by scale * log2(e) while it is
// rotated, so p = exp2(s - m) maps to v_exp_f32.  The running max is only moved
// when a row's tile max exceeds it by more than 8 (p <= 256 in between), which
// makes the O rescale rare; the result is the same softmax (the final division
// by the running sum uses the same reference point).
#pragma once

#include "common.h"
#include "wanattn.h"

namespace wanattn {

constexpr int kBM = 256;                       // query rows per workgroup
constexpr int kBN = 64;                        // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKRow = 272;                     // bytes per K row in LDS (256 + 16 pad)
constexpr int kKTile = kBN * kKRow;            // 17408
constexpr int kVRow = 256;                     // V rows unpadded; 16-byte chunks XOR-swizzled
constexpr int kVTile = kBN * kVRow;            // 16384
constexpr int kStage = kKTile + kVTile;        // 33792
constexpr int kLdsBytes = 2 * kStage;          // 67584 (of 160 KiB)
constexpr float kLazyRescale = 8.0f;           // log2 units

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const float2* tab;  // rotary table (self attention only)
  int N;              // query tokens per batch
  int Nk;             // key tokens per batch
  int heads;
  int ntq;            // query tiles per (batch, head)
  int total;          // workgroups = B * heads * ntq
  float qscale;       // scale * log2(e)
  int H, W, f0, h0, w0;
  double inv_hw, inv_w;
  int chunk_tokens;   // block-causal chunk length in tokens
  int lens[WANATTN_MAX_LEN_BATCH];  // visible keys per batch (1..Nk)
};

// K row slot of physical key t inside a 64-key tile: swap bits 2 and 3
__device__ __forceinline__ int k_slot(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}
// byte offset of 16-byte chunk c of V row t inside a V tile
__device__ __forceinline__ int v_off(int t, int c) { return t * kVRow + 16 * (c ^ (4 * (t & 3))); }

template <bool ROPE, bool CAUSAL>
__device__ __forceinline__ int row_limit(const AttnParams& p, int kvl, int i) {
  int lim = kvl;
  if (CAUSAL) {
    int ce = (i / p.chunk_tokens + 1) * p.chunk_tokens;
    lim = ce < lim ? ce : lim;
  }
  return lim;
}

template <bool ROPE>
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, const float2* tab, int c, int pf, int ph,
                                                int pw, float scale) {
  float re = bf16_lo(w), im = bf16_hi(w);
  if (ROPE) {
    int a = pair_axis(c);
    int pa = a == 0 ? pf : (a == 1 ? ph : pw);
    float2 cs = tab[(a * kMaxPos + pa) * kTabStride + pair_index(c)];
    float r2 = re * cs.x - im * cs.y;
    float i2 = re * cs.y + im * cs.x;
    re = r2;
    im = i2;
  }
  return pack_bf16x2(re * scale, im * scale);
}

template <bool ROPE, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];

  // ---- workgroup -> (batch, head, query tile).  Workgroup w runs on XCD w % 8;
  // give each XCD a contiguous run of tiles so that the concurrent workgroups of
  // an XCD walk the same head's K/V through their shared L2.
  const int wg = blockIdx.x;
  const int per = p.total >> 3, rem = p.total & 7, x = wg & 7;
  const int L = x * per + (x < rem ? x : rem) + (wg >> 3);
  const int bh = L / p.ntq;
  int tq = L - bh * p.ntq;
  if (CAUSAL) tq = p.ntq - 1 - tq;  // heaviest tiles of a head first
  const int b = bh / p.heads, head = bh - b * p.heads;
  const int i0 = tq * kBM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hh = lane >> 5;
  const int kvl = p.lens[b];
  const int i_last = min(i0 + kBM, p.N) - 1;
  const int kv_end = row_limit<ROPE, CAUSAL>(p, kvl, i_last);
  const int kv_full = row_limit<ROPE, CAUSAL>(p, kvl, i0);
  const int nt = (kv_end + kBN - 1) / kBN;

  const size_t row_stride = (size_t)p.heads * kHeadDim;  // elements between tokens
  const uint16_t* qbase = p.q + ((size_t)b * p.N * p.heads + head) * kHeadDim;
  const uint16_t* kbase = p.k + ((size_t)b * p.Nk * p.heads + head) * kHeadDim;
  const uint16_t* vbase = p.v + ((size_t)b * p.Nk * p.heads + head) * kHeadDim;

  // ---- Q: load, rotate, scale, round to bf16; kept in registers as the B
  // operand of K Q^T: lane holds d = 16 kk + 8 hh + 0..7 of its query.
  bf16x8 qf[2][8];
  int lim[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = i0 + wave * 64 + qb * 32 + r;
    const bool valid = i < p.N;
    const int ic = valid ? i : p.N - 1;
    lim[qb] = row_limit<ROPE, CAUSAL>(p, kvl, ic);
    int pf = 0, ph = 0, pw = 0;
    if (ROPE) {
      int f, rm, h, w;
      divmod(ic, p.H * p.W, p.inv_hw, f, rm);
      divmod(rm, p.W, p.inv_w, h, w);
      pf = f + p.f0;
      ph = h + p.h0;
      pw = w + p.w0;
    }
    const u32x4* src = (const u32x4*)(qbase + (size_t)ic * row_stride);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 raw = valid ? src[2 * kk + hh] : u32x4{0, 0, 0, 0};
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[e] = rotate_pair<ROPE>(raw[e], p.tab, 8 * kk + 4 * hh + e, pf, ph, pw, p.qscale);
      qf[qb][kk] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  // ---- K/V staging through registers: thread (g, dc) moves chunk dc of keys
  // 4g .. 4g+3 of a tile; 16 consecutive threads read one 256-byte row.
  const int dc = tid & 15, g = tid >> 4;
  u32x4 kr[4], vr[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = t * kBN + 4 * g + rr;
      const bool valid = key < p.Nk;
      const size_t off = (size_t)(valid ? key : 0) * row_stride + 8 * dc;
      kr[rr] = valid ? *(const u32x4*)(kbase + off) : u32x4{0, 0, 0, 0};
      vr[rr] = valid ? *(const u32x4*)(vbase + off) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int t, int buf) {
    char* kt = smem + buf * kStage;
    char* vt = kt + kKTile;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int tk = 4 * g + rr;
      u32x4 kv = kr[rr];
      if (ROPE) {
        const int key = min(t * kBN + tk, p.Nk - 1);
        int f, rm, h, w;
        divmod(key, p.H * p.W, p.inv_hw, f, rm);
        divmod(rm, p.W, p.inv_w, h, w);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kv[e] = rotate_pair<true>(kv[e], p.tab, 4 * dc + e, f + p.f0, h + p.h0, w + p.w0, 1.0f);
      }
      *(u32x4*)(kt + k_slot(tk) * kKRow + 16 * dc) = kv;
      *(u32x4*)(vt + v_off(tk, dc)) = vr[rr];
    }
  };

  floatx16 acc[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[qb][db][j] = 0.0f;
  float mrun[2] = {-1e30f, -1e30f}, lrun[2] = {0.0f, 0.0f};

  // per-lane pieces of the V transpose-read address (see the header comment)
  const int vg = lane >> 4;            // 16-lane group: hh = vg >> 1, d half = vg & 1
  const int vu = (lane & 15) >> 2;     // key offset supplied by this lane
  const int vq = lane & 3;             // d quad supplied by this lane

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) load_tile(t + 1);
    const char* kt = smem + buf * kStage;
    const char* vt = kt + kKTile;

    // S^T = K' Q'^T
    floatx16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[0][kb][j] = 0.0f;
        s[1][kb][j] = 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        bf16x8 a = *(const bf16x8*)(kt + (32 * kb + r) * kKRow + 32 * kk + 16 * hh);
        s[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][kk], s[0][kb], 0, 0, 0);
        s[1][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][kk], s[1][kb], 0, 0, 0);
      }
    }

    // visibility: key index of register j of block kb is 32 kb + 16 (j/8) + 8 hh + j%8
    if (t * kBN + kBN > kv_full) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = t * kBN + 32 * kb + 16 * (j >> 3) + 8 * hh + (j & 7);
            if (key >= lim[qb]) s[qb][kb][j] = -__builtin_inff();
          }
    }

    // online softmax (base 2) and P = exp2(S - m) packed as bf16 MFMA operands
    bf16x8 pb[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[qb][kb][j]);
      mx = wave_half_max(mx);
      const float mnew = fmaxf(mrun[qb], mx);
      const bool need = mnew > mrun[qb] + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(mrun[qb] - mnew) : 1.0f;
        mrun[qb] = need ? mnew : mrun[qb];
        lrun[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[qb][db][j] *= alpha;
      }
      float sum = 0.0f;
      const float m = mrun[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(s[qb][kb][8 * sl + 2 * e] - m);
            const float p1 = __builtin_amdgcn_exp2f(s[qb][kb][8 * sl + 2 * e + 1] - m);
            sum += p0 + p1;
            pk[e] = pack_bf16x2(p0, p1);
          }
          pb[qb][kb][sl] = __builtin_bit_cast(bf16x8, pk);
        }
      }
      lrun[qb] += sum;
    }

    // O^T += V^T P^T; V read transposed from its row-major LDS tile
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          shortx4 tr[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int key = 32 * kb + 16 * sl + 8 * (vg >> 1) + 4 * e + vu;
            const int chunk = 4 * db + 2 * (vg & 1) + (vq >> 1);
            const char* addr = vt + v_off(key, chunk) + 8 * (vq & 1);
            tr[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) shortx4*)(addr));
          }
          // whole-vector casts: element-wise assembly of this operand was
          // lowered to a splat of element 0 by the compiler
          const bf16x8 a = __builtin_shufflevector(__builtin_bit_cast(bf16x4, tr[0]),
                                                   __builtin_bit_cast(bf16x4, tr[1]), 0, 1, 2, 3, 4,
                                                   5, 6, 7);
          acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0][kb][sl], acc[0][db], 0, 0, 0);
          acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[1][kb][sl], acc[1][db], 0, 0, 0);
        }
      }
    }

    if (t + 1 < nt) store_tile(t + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16; lane holds d = 32 db + 8 g4 + 4 hh + 0..3
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float inv = 1.0f / wave_half_sum(lrun[qb]);
    const int i = i0 + wave * 64 + qb * 32 + r;
    if (i < p.N) {
      uint16_t* dst = p.o + ((size_t)b * p.N + i) * row_stride + (size_t)head * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[qb][db][4 * g4 + 0] * inv, acc[qb][db][4 * g4 + 1] * inv);
          w[1] = pack_bf16x2(acc[qb][db][4 * g4 + 2] * inv, acc[qb][db][4 * g4 + 3] * inv);
          *(u32x2*)(dst + 32 * db + 8 * g4 + 4 * hh) = w;
        }
    }
  }
}

}  // namespace wanattn
