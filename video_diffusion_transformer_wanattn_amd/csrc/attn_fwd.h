// Flash-style attention forward for head_dim 128 on gfx950 (wave64, bf16 MFMA).
//
// What it computes (per batch b, head, query row i):
//   o_i = sum_j p_ij v_j,  p_ij = softmax_j(q'_i . k'_j * scale) over visible j
// where q' is q rotated by the 3D RoPE of its token (self attention, Wan2.2
// source reading (blog.leeguoo.com) ch. 4, "3D RoPE") or left as it is (cross
// attention to text tokens, Wan paper explainer (0h-n0.github.io), text-encoder
// section), and k' is the key as the caller hands it in: for self attention the
// library first rotates k once into a workspace with the rope3d kernel.  The
// N x N score matrix is never stored (ch. 8 of the source reading sizes it; the
// long-video survey (atlascloud.ai) puts it at ~10 GB for 32.7k tokens).
//
// Work decomposition
//   one work item = 4 waves = 256 query rows of one (batch, head); a wave owns
//   64 rows as two 32-row MFMA blocks.  Keys stream through LDS in tiles of 64
//   (K' 16 KiB + V 16 KiB), 4 stages, filled with global_load_lds_dwordx4 (no
//   staging registers), two tiles in flight ahead of the one being computed.
//   A plain launch runs one item per workgroup; a persistent launch runs one
//   workgroup per compute unit that draws items from per-XCD queues (XCDs run
//   at different speeds), the last items being key ranges of the last query
//   tiles, whose partial results split_merge_kernel combines.
//
// Per 32-key block and wave (two blocks per tile):
//   S^T (keys x queries) = K' Q'^T   v_mfma_f32_32x32x16_bf16, 2 x 8 issues
//   online softmax on S^T: a lane holds 16 scores of ONE query per block, so
//   row sums are in-lane (plus one permlane32 swap at the end)
//   O^T (d x queries) += V^T P^T     2 x 4 x 2 issues; P stays in registers
// The loop is software-pipelined over blocks: the QK^T products of block j+1
// are issued next to the exp work of keys 16..31 of block j, and the PV
// products of block j next to the exp work of keys 0..15 of block j+1, so each
// MFMA has a few independent VALU instructions beside it (one wave per SIMD:
// the VALU work only overlaps the MFMA pipe when it is spread out like this).
//
// Key order inside a 32-key MFMA block is free (the contraction is a sum), so
// K rows sit in LDS permuted (bits 2 and 3 of the key index swapped): the S^T
// accumulator of lane l (half hh = l / 32) then holds, at register positions
// 8s .. 8s+7, the physical keys 16s + 8hh + 0..7 -- exactly the B operand
// layout of the PV product.  V stays row-major in LDS and is read with
// ds_read_b64_tr_b16, which hands each lane four keys of one d column.  Both
// tiles XOR-swizzle their 16-byte chunks so that the MFMA operand reads are
// free of bank conflicts.
//
// Softmax is in base 2: the query is multiplied by scale * log2(e) when it is
// loaded, so p = exp2(s - m) maps to v_exp_f32, and the subtraction of the row
// reference m is folded into the QK^T product: its first k-step starts from an
// accumulator tile holding -m instead of zero.  The O accumulators live in
// AGPRs (the PV products are inline asm, see acc_fence).  The reference
// starts at the max of the first block and is only moved when a
// lane's block sum of p exceeds 2^16 (some p above 2^12, or an overflow), which
// makes the O rescale rare; the result is the same softmax (the final division
// by the running sum uses the same reference point).
#pragma once

#include <type_traits>

#include "common.h"
#include "wanattn.h"

namespace wanattn {

constexpr int kBM = 256;                       // query rows per workgroup
constexpr int kBN = 64;                        // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = 256;                 // one 128-wide bf16 row
constexpr int kHalfTile = kBN * kRowBytes;     // 16 KiB: K' or V of one tile
constexpr int kTileBytes = 2 * kHalfTile;      // 32 KiB
constexpr int kVHalves = 4 * kHalfTile;        // V halves of the 4 stages start here (64 KiB)
constexpr int kStages = 4;
constexpr int kLdsBytes = kStages * kTileBytes;  // 128 KiB of 160
constexpr float kLazySum = 65536.0f;           // lane partial block sum that moves the reference
// Cross attention's persistent launch prefetches the next item during the
// epilogue: its first two tiles into stages 0 and 1, its 256 query rows into
// the K' and V halves of stages 2 and 3 (wave w's 64 rows at kPrefetchQ[w];
// tile 2 overwrites them only after the next item's first barrier), and the
// output is staged in 32-row halves above the stages.
constexpr int kPrefetchStaging = 128 * 1024;                                    // 8 KiB per wave
constexpr int kLdsPrefetchBytes = kPrefetchStaging + kWaves * 32 * kRowBytes;  // 160 KiB
__device__ __forceinline__ int prefetch_q_base(int wave) {
  return wave < 2 ? 2 * kHalfTile + wave * 64 * kRowBytes : kVHalves + 2 * kHalfTile + (wave - 2) * 64 * kRowBytes;
}

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;  // keys as used in the product (already rotated for self attention)
  const uint16_t* v;
  uint16_t* o;
  const float2* tab;  // rotary table for the query (self attention only)
  long long tab_hstride;  // float2 entries between consecutive heads' tables (0: one shared table)
  int N;              // query tokens per batch
  int Nk;             // key tokens per batch
  int heads;
  int ntq;            // query tiles per (batch, head)
  int total;          // workgroups = B * heads * ntq
  float qscale;       // scale * log2(e)
  int H, W, f0, h0, w0;
  double inv_hw, inv_w;
  int chunk_tokens;   // block-causal chunk length in tokens
  // Persistent launches (PERSIST kernels): one workgroup per compute unit
  // takes work items from queue (9 counters, zero at launch): the query tiles
  // 0 .. total-1, split into 8 contiguous runs, one per XCD (own run first,
  // then the other runs), and then the split items 0 .. nsplit_items-1 of the
  // key-split tail: item s runs key range s % nsplit of query tile
  // total + s / nsplit, writing partial results to part_o and part_lb instead
  // of O (see split_merge_kernel)
  unsigned* queue;
  float4* part_o;
  float2* part_lb;
  int nsplit, nsplit_items;
  // QK-Norm of the queries applied as they are loaded (QNORM kernels): q *
  // q_rms[b * N + n] * gq[head * 128 + d] before the rotation
  const float* q_rms;
  const uint16_t* gq;
  int lens[WANATTN_MAX_LEN_BATCH];  // visible keys per batch (1..Nk)
};

constexpr int kQueueCounters = 9;  // one per XCD, then the split items

// Partial results of one split workgroup, in the order its lanes hold them:
// O (not normalised) as kBM * kHeadDim / 4 float4, index
// ((2 * wave + qb) * 16 + 4 * db + g4) * 64 + lane for query row
// 64 wave + 32 qb + (lane & 31) and d = 32 db + 8 g4 + 4 (lane >> 5) + 0..3;
// the row sum l and the bias b (minus the reference O and l are taken
// against) as kBM float2, index (2 * wave + qb) * 32 + row % 32.
constexpr int kPartO = kBM * kHeadDim / 4;

// K row slot of physical key t inside a tile: swap bits 2 and 3 (an involution)
__device__ __forceinline__ int k_slot(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }
// 16-byte chunk swizzles (chunk index 0..15 within a 256-byte row)
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return 4 * (row & 3); }

// (P: the argument block, in whichever address space the kernel reads it from)
template <bool CAUSAL, class P>
__device__ __forceinline__ int row_limit(const P& p, int kvl, int i) {
  int lim = kvl;
  if (CAUSAL) {
    int ce = (i / p.chunk_tokens + 1) * p.chunk_tokens;
    lim = ce < lim ? ce : lim;
  }
  return lim;
}

// (sre, sim: factors applied before the rotation, 1 unless the queries are
// RMS-normalised here)
template <bool ROPE>
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, const float2* tab, int c, int pf, int ph,
                                                int pw, float scale, float sre = 1.0f, float sim = 1.0f) {
  float re = bf16_lo(w) * sre, im = bf16_hi(w) * sim;
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

// Next work item of a persistent workgroup on XCD x (one lane calls this):
// a query tile from XCD x's run, else from the runs of XCDs x+1, x+2, .. (k
// is the caller's cursor over them), else a split item (returned as total +
// s), else -1.  Counters only grow; a draw past the end of a run is unused.
__device__ __forceinline__ int next_item(const AttnParams& p, int x, int& k) {
  const int per = p.total >> 3, rem = p.total & 7;
  while (k < 8) {
    const int y = (x + k) & 7;
    const int n = per + (y < rem ? 1 : 0);
    const unsigned j = __hip_atomic_fetch_add(p.queue + y, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (j < (unsigned)n) return y * per + (y < rem ? y : rem) + (int)j;
    ++k;
  }
  const unsigned s = __hip_atomic_fetch_add(p.queue + 8, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return s < (unsigned)p.nsplit_items ? p.total + (int)s : -1;
}

// wait until at most n of this wave's vector-memory operations are outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
  if constexpr (n == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (n == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else static_assert(n == 0 || n == 8, "unsupported count");
}

// workgroup barrier without the memory fence of __syncthreads (which would
// drain the prefetches in flight); LDS reads of this wave are completed first
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from gbase + voff into LDS at lds + 16 * lane.  Written as
// asm so that the compiler does not track the LDS write (the kernel waits for
// these loads itself with vmcnt and a barrier).  The LDS address is an m0
// operand: the compiler writes m0 itself and knows it is in use.
__device__ __forceinline__ void dma16(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(lds) : "memory");
}

template <bool ROPE, bool CAUSAL, bool PERSIST = false, bool QNORM = false>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_kernel(AttnParams p_arg) {
  // Cross attention's persistent launch (PERSIST without RoPE) takes its items
  // in a fixed order, with no queue, and issues the next item's first two
  // key tiles and its query loads before the current item's epilogue, whose
  // output staging then moves above the stages (kPrefetchStaging).  Its items
  // are short (512 text keys), so the per-item query load and epilogue would
  // otherwise take about half of each one.
  constexpr bool PREFETCH = PERSIST && !ROPE;
  // LDS: the K' halves of the 4 stages in the first 64 KiB, their V halves in
  // the second, so that every operand read is one base register (per lane)
  // plus an immediate offset below 64 KiB (the ds_read offset field)
  __shared__ __attribute__((aligned(1024))) char lds[PREFETCH ? kLdsPrefetchBytes : kLdsBytes];
  // K' half of a stage, as a compile-time constant (main loop) or a run-time
  // index (masked tail); its V half is kVHalves further
  auto stage = [&](auto S) __attribute__((always_inline)) -> char* {
    if constexpr (std::is_integral_v<decltype(S)>) return lds + (S & (kStages - 1)) * kHalfTile;
    else return lds + decltype(S)::value * kHalfTile;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  __shared__ int s_item;
  int cursor = 0;  // lane 0 of wave 0: the queue it draws from (next_item)
  const int xcc = PERSIST ? (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7) : 0;  // HW_REG_XCC_ID
  // fixed item order of the prefetching launch: workgroup w (of 8 c, run on XCD
  // w % 8) takes items w / 8, w / 8 + c, ... of XCD w % 8's contiguous run
  int pass = 0;
  // this pass's queries (qpre) and first two tiles (tpre) were loaded last pass
  bool qpre = false, tpre = false;
  auto static_item = [&](const auto& pp, int ps) -> int {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3, c = gridDim.x >> 3;
    const int per = pp.total >> 3, rem = pp.total & 7;
    const int idx = j + c * ps;
    return idx < per + (x < rem ? 1 : 0) ? x * per + (x < rem ? x : rem) + idx : -1;
  };

  // one work item per pass; a plain launch makes one pass
  for (;;) {
    // A persistent pass reads the arguments again from the kernel argument
    // segment (through a pointer the compiler cannot see through) and derives
    // the lane constants again: otherwise they are all kept in registers across
    // passes (70 SGPRs and 37 VGPRs of spills, against 4 and 0).
    const auto& p = [&]() -> decltype(auto) {
      if constexpr (PERSIST) {
        auto kp = (const __attribute__((address_space(4))) AttnParams*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kp));
        return *kp;
      } else {
        return (const AttnParams&)p_arg;
      }
    }();
    int tid = threadIdx.x;
    if constexpr (PERSIST) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, hh = lane >> 5;
    // ---- work item -> (batch, head, query tile).  A plain launch runs workgroup w
    // on XCD w % 8; it gives each XCD a contiguous run of tiles so that the
    // concurrent workgroups of an XCD walk the same head's K/V through their
    // shared L2.  A persistent launch keeps those runs as the XCDs' queues.
    // A split item takes key range ks of tile total + item / nsplit.
    int L, ks = 0, item = 0;
    bool split = false;
    if constexpr (PREFETCH) {
      L = static_item(p, pass);
      if (L < 0) break;
    } else if constexpr (PERSIST) {
      // every thread has read the previous item (its pass had barriers since)
      if (tid == 0) s_item = next_item(p_arg, xcc, cursor);
      __syncthreads();
      const int it = s_item;
      if (it < 0) break;
      split = it >= p.total;
      L = it;
      if (split) {
        item = it - p.total;
        L = p.total + item / p.nsplit;
        ks = item - (item / p.nsplit) * p.nsplit;
      }
    } else {
      const int wg = blockIdx.x;
      const int per = p.total >> 3, rem = p.total & 7, x = wg & 7;
      L = x * per + (x < rem ? x : rem) + (wg >> 3);
    }
    const int bh = L / p.ntq;
    int tq = L - bh * p.ntq;
    if (CAUSAL) tq = p.ntq - 1 - tq;  // heaviest tiles of a head first
    const int b = bh / p.heads, head = bh - b * p.heads;
    const int i0 = tq * kBM;

    // keys [k0, k0 + Nk) of the batch are this workgroup's (all of them unless split)
    int k0 = 0, Nk = p.Nk, kvl = p.lens[b];
    if (split) {
      // the host launches splits only where every range holds a key
      const int nkt = (kvl + kBN - 1) / kBN;
      const int t_lo = ks * nkt / p.nsplit, t_hi = (ks + 1) * nkt / p.nsplit;
      k0 = t_lo * kBN;
      Nk = min(t_hi * kBN, kvl) - k0;
      kvl = Nk;
    }
    const int i_last = min(i0 + kBM, p.N) - 1;
    const int kv_end = row_limit<CAUSAL>(p, kvl, i_last);
    const int kv_full = row_limit<CAUSAL>(p, kvl, i0);
    const int nt = (kv_end + kBN - 1) / kBN;
    const int nb = 2 * nt;

    const size_t row_stride = (size_t)p.heads * kHeadDim;  // elements between tokens
    const uint32_t rsb = (uint32_t)(row_stride * 2);        // bytes between tokens
    const uint16_t* qbase = p.q + ((size_t)b * p.N * p.heads + head) * kHeadDim;
    const char* kbase = (const char*)(p.k + (((size_t)b * p.Nk + k0) * p.heads + head) * kHeadDim);
    const char* vbase = (const char*)(p.v + (((size_t)b * p.Nk + k0) * p.heads + head) * kHeadDim);

    // ---- tile loads straight into LDS.  Instruction i of wave w fills 1 KiB:
    // rows m = 16w + 4i + l/16 (l = lane), stored chunk l%16 holding global chunk
    // (l%16) ^ swizzle(m).  K row m holds key k_slot(m) = 16w + 4 swap01(i) + l/16.
    // Full tiles: a uniform row base plus a fixed per-lane offset.  The last,
    // partial tile clamps every row to the last key (those rows are masked).
    const int ld_row = lane >> 4, ld_chunk = lane & 15;
    // byte offsets from the tile's first key, the row of each load included, so
    // that all loads of a tile share one scalar base (64 rows fit in 32 bits:
    // the library limits heads so that 64 token rows span less than 2^31 bytes)
    uint32_t koff_ld[4], voff_ld[4];
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int krow = 16 * wave + 4 * ((i >> 1) | ((i & 1) << 1));
      const int vrow = 16 * wave + 4 * i;
      koff_ld[i] = (krow + ld_row) * rsb + 16 * (ld_chunk ^ (4 * i + ld_row));
      voff_ld[i] = (vrow + ld_row) * rsb + 16 * (ld_chunk ^ (4 * ld_row));
    }
    // a tile known to hold kBN keys
    auto issue_full_tile = [&](auto S, int t) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)stage(S);
      const char* kt = kbase + (size_t)t * kBN * rsb;
      const char* vt = vbase + (size_t)t * kBN * rsb;
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int blk = 4 * wave + i;
        dma16(kt, koff_ld[i], st + blk * 1024);
        dma16(vt, voff_ld[i], st + kVHalves + blk * 1024);
      }
    };
    // load n (0..7) of a full tile: K (n even) or V (n odd) rows of group n / 2
    auto issue_one = [&](auto S, int t, int n) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)stage(S);
      const int i = n >> 1, blk = 4 * wave + i;
      if (n & 1) dma16(vbase + (size_t)t * kBN * rsb, voff_ld[i], st + kVHalves + blk * 1024);
      else dma16(kbase + (size_t)t * kBN * rsb, koff_ld[i], st + blk * 1024);
    };
    auto issue_tile = [&](auto S, int t) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)stage(S);
      const char* kt = kbase + (size_t)t * kBN * rsb;
      const char* vt = vbase + (size_t)t * kBN * rsb;
      if (t * kBN + kBN <= Nk) {
        issue_full_tile(S, t);
      } else {
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int blk = 4 * wave + i;
          const int m = 4 * blk + ld_row;
          const int kkey = min(t * kBN + k_slot(m), Nk - 1) - t * kBN;
          const int vkey = min(t * kBN + m, Nk - 1) - t * kBN;
          dma16(kt, (uint32_t)kkey * rsb + 16 * (ld_chunk ^ k_swz(m)), st + blk * 1024);
          dma16(vt, (uint32_t)vkey * rsb + 16 * (ld_chunk ^ v_swz(m)), st + kVHalves + blk * 1024);
        }
      }
    };

    // (prefetching launch) this wave's 64 query rows of query tile tq_ of
    // (batch bq, head hq) into LDS at prefetch_q_base(wave): instruction i fills
    // rows 4 i + lane / 16, stored chunk lane % 16 holding chunk (lane % 16) ^
    // (row & 15).  Rows past the last token repeat it; a wave whose rows all lie
    // past it (a partial last tile) reads the last token's row: the load base is
    // the wave's first row clamped, so every offset is 0..63 rows.
    auto dma_q = [&](int bq, int hq, int tq_) __attribute__((always_inline)) {
      const int ibase = tq_ * kBM + wave * 64;
      const int ib0 = min(ibase, p.N - 1);
      const char* qn = (const char*)(p.q + (((size_t)bq * p.N + ib0) * p.heads + hq) * kHeadDim);
      const uint32_t qst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lds + prefetch_q_base(wave));
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 4 * i + ld_row;
        const int rowc = min(ibase + row, p.N - 1) - ib0;
        dma16(qn, (uint32_t)rowc * rsb + 16 * (ld_chunk ^ (row & 15)), qst + i * 1024);
      }
    };
    // the look-ahead scoring of the block after the last one reads the next
    // stage: with fewer tiles than stages that stage was never filled, so zero
    // the stages then (with more, it holds an earlier tile: finite values whose
    // scores are discarded).  nt is uniform over the workgroup.
    auto zero_stages = [&]() __attribute__((always_inline)) {
  #pragma unroll
      for (int i = 0; i < kLdsBytes / 16 / kThreads; ++i)
        *(u32x4*)(lds + 16 * (tid + i * kThreads)) = u32x4{0, 0, 0, 0};
    };
    if constexpr (PREFETCH) {
      // the queries always come through LDS: loaded last pass, else now (the
      // first pass); the tiles follow the query reads when not prefetched
      if (!qpre) dma_q(b, head, tq);
    } else {
      if (nt < kStages) {
        zero_stages();
        tile_barrier();
      }
      // prefetch the first two tiles while the queries are loaded
      issue_tile(S0{}, 0);
      if (nt > 1) issue_tile(S1{}, 1);
    }

    // ---- Q: load, rotate, scale, round to bf16; kept in registers as the B
    // operand of K Q^T: lane holds d = 16 kk + 8 hh + 0..7 of its query.
    // All 16 loads are issued before any is used (a pin per chunk made the
    // compiler wait for each load in turn: ~7 us per workgroup).
    bf16x8 qf[2][8];
    int lim[2];
    const float2* qtab = p.tab + (size_t)head * p.tab_hstride;
    u32x4 qraw[2][8];
    int pf[2] = {0, 0}, ph[2] = {0, 0}, pw[2] = {0, 0};
  #pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int i = i0 + wave * 64 + qb * 32 + r;
      const int ic = i < p.N ? i : p.N - 1;
      lim[qb] = row_limit<CAUSAL>(p, kvl, ic);
      if (ROPE) {
        int f, rm, h, w;
        divmod(ic, p.H * p.W, p.inv_hw, f, rm);
        divmod(rm, p.W, p.inv_w, h, w);
        pf[qb] = f + p.f0;
        ph[qb] = h + p.h0;
        pw[qb] = w + p.w0;
      }
      const u32x4* src = (const u32x4*)(qbase + (size_t)ic * row_stride);
      if constexpr (PREFETCH) {
        // from LDS, where this wave's own loads put its rows (row rho's chunk c
        // stored at c ^ (rho & 15)).  The wait is for every outstanding vector
        // memory operation, the last epilogue's output stores included: a store
        // can complete before a load issued ahead of it, so a count that leaves
        // the stores outstanding does not prove the loads done (with vmcnt(16),
        // rows of some waves were read before their loads landed).  No global
        // load of q exists in this kernel (a path that could leave one in
        // flight to these registers made the compiler wait before each read).
        if (qb == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int rho = qb * 32 + r;
        const char* qrow = lds + prefetch_q_base(wave) + rho * kRowBytes;
  #pragma unroll
        for (int kk = 0; kk < 8; ++kk) qraw[qb][kk] = *(const u32x4*)(qrow + 16 * ((2 * kk + hh) ^ (rho & 15)));
      } else {
  #pragma unroll
        for (int kk = 0; kk < 8; ++kk) qraw[qb][kk] = src[2 * kk + hh];
      }
    }
    if constexpr (QNORM) {
      // RMSNorm of the queries: each row's factor times the head's gamma (d = 16
      // kk + 8 hh + 0..7 in chunk kk), then the rotation
      float qs[2];
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int i = i0 + wave * 64 + qb * 32 + r;
        qs[qb] = p.q_rms[(size_t)b * p.N + (i < p.N ? i : p.N - 1)];
      }
  #pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 gw = *(const u32x4*)(p.gq + (size_t)head * kHeadDim + 16 * kk + 8 * hh);
  #pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          u32x4 pk;
  #pragma unroll
          for (int e = 0; e < 4; ++e)
            pk[e] = rotate_pair<ROPE>(qraw[qb][kk][e], qtab, 8 * kk + 4 * hh + e, pf[qb], ph[qb], pw[qb], p.qscale,
                                      qs[qb] * bf16_lo(gw[e]), qs[qb] * bf16_hi(gw[e]));
          qf[qb][kk] = __builtin_bit_cast(bf16x8, pk);
        }
      }
    } else {
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb)
  #pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          u32x4 pk;
  #pragma unroll
          for (int e = 0; e < 4; ++e)
            pk[e] = rotate_pair<ROPE>(qraw[qb][kk][e], qtab, 8 * kk + 4 * hh + e, pf[qb], ph[qb], pw[qb], p.qscale);
          qf[qb][kk] = __builtin_bit_cast(bf16x8, pk);
        }
    }
    // keep Q in AGPRs: the MFMA reads its B operand from there directly and the
    // arch VGPRs stay free for the scores and the softmax
    asm volatile(""
                 : "+a"(qf[0][0]), "+a"(qf[0][1]), "+a"(qf[0][2]), "+a"(qf[0][3]), "+a"(qf[0][4]), "+a"(qf[0][5]),
                   "+a"(qf[0][6]), "+a"(qf[0][7]), "+a"(qf[1][0]), "+a"(qf[1][1]), "+a"(qf[1][2]), "+a"(qf[1][3]),
                   "+a"(qf[1][4]), "+a"(qf[1][5]), "+a"(qf[1][6]), "+a"(qf[1][7]));

    floatx16 acc[2][4];
  #pragma unroll
    for (int qb = 0; qb < 2; ++qb)
  #pragma unroll
      for (int db = 0; db < 4; ++db)
  #pragma unroll
        for (int j = 0; j < 16; ++j) acc[qb][db][j] = 0.0f;
    // The O products (phase B below) are inline asm so that their accumulators
    // live in AGPRs for the whole loop: the arch VGPRs then hold the scores,
    // the operands and the loop invariants without parking any of them in AGPRs
    // (which cost ~20 copies per block).  The compiler does not know these asm
    // statements are MFMAs and inserts no wait states around them, so this fence
    // does: 24 wait states (more than the 8-pass MFMA's result latency) before
    // any VALU access of O after an O product, and after VALU writes of O
    // (initialisation, rescale) before the next product reads them.  Dependent
    // MFMA -> MFMA accumulation needs none (the hardware interlocks it).
    auto acc_fence = [&]() __attribute__((always_inline)) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                     "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
    };
    acc_fence();
    // Running softmax reference per query row, kept as a bias b = -m added to the
    // scores inside the QK^T product: the first k-step of the product starts
    // from an accumulator tile holding b (every value a lane holds in S^T
    // belongs to its own query column, so the tile is b repeated).  The scores
    // come out of the product already shifted, and p = exp2(s) needs no
    // subtraction; the tile only changes when the reference moves.
    float bias[2] = {0.0f, 0.0f}, lrun[2] = {0.0f, 0.0f};
    floatx16 btile[2];
    auto set_bias = [&](int qb, float b) __attribute__((always_inline)) {
      bias[qb] = b;
  #pragma unroll
      for (int e = 0; e < 16; ++e) btile[qb][e] = b;
    };
    set_bias(0, 0.0f);
    set_bias(1, 0.0f);

    // LDS operand offsets inside a stage.  K: row r (+32 kb), stored chunk
    // (2 kk + hh) ^ (r & 15).  V (transposed reads): lane (vg, vu, vq) supplies
    // key 8 (vg>>1) + vu (+ 32 kb + 16 sl + 4 e) and d 32 db + 16 (vg&1) + 4 vq,
    // whose chunk 4 db + 2 (vg&1) + vq/2 is stored at 4 (db ^ vu) + 2 (vg&1) + vq/2.
    int koff[8];
  #pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      koff[kk] = r * kRowBytes + 16 * ((2 * kk + hh) ^ (r & 15));
      asm volatile("" : "+v"(koff[kk]));
    }
    const int vg = lane >> 4, vu = (lane & 15) >> 2, vq = lane & 3;
    int voff[4];
  #pragma unroll
    for (int db = 0; db < 4; ++db)
      voff[db] = kVHalves + (8 * (vg >> 1) + vu) * kRowBytes +
                 16 * (4 * (db ^ vu) + 2 * (vg & 1) + (vq >> 1)) + 8 * (vq & 1);
  #pragma unroll
    for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(voff[db]));

    bf16x8 kop[8];      // K' operands of the next block to score
    bf16x8 vop[4][2];   // V operands of the block being accumulated
    float sv[2][16];    // scores of the block being finished (base 2, VGPR copy)
    floatx16 sacc[2];   // MFMA accumulators of the block being scored
    bf16x8 pcar[2];     // P of keys 0..15 of the block being finished, taken one phase early
    float scar[2];      // and this lane's sums of them

    auto load_kops = [&](auto S, int kb) __attribute__((always_inline)) {
      const char* kt = stage(S) + kb * 32 * kRowBytes;
  #pragma unroll
      for (int kk = 0; kk < 8; ++kk) kop[kk] = *(const bf16x8*)(kt + koff[kk]);
    };
    // single operand reads, for the hand-ordered block step
    auto load_kop = [&](auto S, int kb, int kk) __attribute__((always_inline)) {
      kop[kk] = *(const bf16x8*)(stage(S) + kb * 32 * kRowBytes + koff[kk]);
    };
    auto load_vop = [&](auto S, int kb, int db, int sl) __attribute__((always_inline)) {
      const char* vt = stage(S) + kb * 32 * kRowBytes;
      shortx4 tr[2];
  #pragma unroll
      for (int e = 0; e < 2; ++e)
        tr[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(vt + (16 * sl + 4 * e) * kRowBytes + voff[db]));
      // whole-vector casts: assembling this operand element by element was
      // lowered to a splat of element 0 by the compiler
      vop[db][sl] = __builtin_shufflevector(__builtin_bit_cast(bf16x4, tr[0]), __builtin_bit_cast(bf16x4, tr[1]),
                                            0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto qk = [&]() __attribute__((always_inline)) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qf[0][0], btile[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qf[1][0], btile[1], 0, 0, 0);
  #pragma unroll
      for (int kk = 1; kk < 8; ++kk) {
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[0][kk], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[1][kk], sacc[1], 0, 0, 0);
      }
    };
    // exp2 of the shifted scores in sv: bf16 operands of the PV product and this
    // lane's fp32 block sums.  One pair of probabilities (keys 16 sl + 2 e, + 1)
    // of row block qb: packed word into pk[e], sum into acc2[e & 1].  (Plain adds:
    // the dot-product VALU instructions wait for the MFMA pipe to drain.)
    auto exp_pair = [&](int qb, int sl, int e, u32x4& pk, float (&acc2)[2]) __attribute__((always_inline)) {
      const float p0 = __builtin_amdgcn_exp2f(sv[qb][8 * sl + 2 * e]);
      const float p1 = __builtin_amdgcn_exp2f(sv[qb][8 * sl + 2 * e + 1]);
      // pairs e = 0, 1 start the two partial sums (every caller takes e in
      // order 0..3): assigning rather than adding to 0 saves an add, which the
      // compiler may not drop itself (0 + x is not x for x = -0)
      if (e < 2) acc2[e & 1] = p0 + p1;
      else acc2[e & 1] += p0 + p1;
      pk[e] = pack_bf16x2(p0, p1);
    };
    // (half sl of the block: keys 16 sl .. 16 sl + 15, registers 8 sl .. 8 sl + 7)
    auto exp_half = [&](int qb, int sl, bf16x8& out, float& sum) __attribute__((always_inline)) {
      float acc2[2];
      u32x4 pk;
  #pragma unroll
      for (int e = 0; e < 4; ++e) exp_pair(qb, sl, e, pk, acc2);
      out = __builtin_bit_cast(bf16x8, pk);
      sum = acc2[0] + acc2[1];
    };
    auto softmax_exp_row = [&](int qb, bf16x8 (&pb)[2][2], float (&bsum)[2]) __attribute__((always_inline)) {
      float h0, h1;
      exp_half(qb, 0, pb[qb][0], h0);
      exp_half(qb, 1, pb[qb][1], h1);
      bsum[qb] = h0 + h1;
    };
    // copy the scored block to VGPRs
    auto take_scores = [&]() __attribute__((always_inline)) {
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb)
  #pragma unroll
        for (int e = 0; e < 16; ++e) sv[qb][e] = sacc[qb][e];
    };
    // visibility of block j: key of register e is 32 j + 16 (e/8) + 8 hh + e%8
    auto mask_scores = [&](int j) __attribute__((always_inline)) {
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb)
  #pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = 32 * j + 16 * (e >> 3) + 8 * hh + (e & 7);
          if (key >= lim[qb]) sv[qb][e] = -__builtin_inff();
        }
    };
    auto row_max = [&](int qb) __attribute__((always_inline)) -> float {
      float m0 = fmaxf(sv[qb][0], sv[qb][1]);
  #pragma unroll
      for (int e = 2; e < 16; e += 2) m0 = fmaxf(m0, fmaxf(sv[qb][e], sv[qb][e + 1]));
      return wave_half_max(m0);
    };
    // Lazy reference (rare after the first blocks).  The probabilities of block
    // j were taken against the current reference; when a lane's partial block
    // sum exceeds kLazySum (some p above 2^12, or an overflow to inf), every row
    // whose block max lies above its reference moves the reference to that max:
    // O and l are scaled by 2^(b_new - b_old), block j's probabilities are taken
    // again, and the scores of block j+1 (already formed against the old
    // reference) are shifted alike.  One wave-uniform branch for both row blocks.
    auto move_reference = [&](bf16x8 (&pb)[2][2], float (&bsum)[2]) __attribute__((always_inline)) {
      acc_fence();
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m = row_max(qb);
        const float old = bias[qb];
        set_bias(qb, m > 0.0f ? old - m : old);
        const float delta = bias[qb] - old;
        const float alpha = __builtin_amdgcn_exp2f(delta);
        lrun[qb] *= alpha;
  #pragma unroll
        for (int db = 0; db < 4; ++db)
  #pragma unroll
          for (int e = 0; e < 16; ++e) acc[qb][db][e] *= alpha;
  #pragma unroll
        for (int e = 0; e < 16; ++e) {
          sv[qb][e] += delta;
          sacc[qb][e] += delta;
        }
        softmax_exp_row(qb, pb, bsum);
      }
      acc_fence();
      // P was just rewritten by VALU and is read next by the O products
      asm volatile("s_nop 1" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]));
    };

    if constexpr (PREFETCH) {
      if (!tpre) {
        // every wave has read its queries, which lie in stages 2 and 3
        if (nt < kStages) {
          tile_barrier();
          zero_stages();
          tile_barrier();
        }
        issue_tile(S0{}, 0);
        if (nt > 1) issue_tile(S1{}, 1);
      }
    }
    // ---- prologue: tile 0 resident, tile 2 requested, block 0 scored and
    // finished, K' operands of block 1 loaded (prefetched tiles are resident
    // since the wait for the prefetched queries, which were loaded after them)
    if (!(PREFETCH && tpre)) {
      if (nt > 1) wait_vm<8>();
      else wait_vm<0>();
    }
    tile_barrier();
    if (nt > 2) issue_tile(S2{}, 2);
    load_kops(S0{}, 0);
    qk();
    load_kops(S0{}, 1);
    {
      // block 0 was scored with b = 0; its row max becomes the first reference
      // (every row sees key 0, so the max is finite; O and l are still zero)
      take_scores();
      if (32 > kv_full) mask_scores(0);
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        set_bias(qb, -row_max(qb));
  #pragma unroll
        for (int e = 0; e < 16; ++e) sv[qb][e] += bias[qb];
        exp_half(qb, 0, pcar[qb], scar[qb]);
      }
    }

    // ---- main pipeline.  Block j of tile t (stage S) with j = 2t + kb:
    //   (first block of a tile: tile t+1 resident, tile t+3 requested)
    //   A: V operands of block j; S(j+1) = K'(j+1) Q'^T + b  next to  P(j) = exp2(S(j))
    //      for keys 16..31 and the block sums of P(j)
    //   (rare, wave-uniform: move the reference, see move_reference)
    //   B: O += V(j)^T P(j)^T  next to  K' operands of block j+2, the copy of
    //      S(j+1) to VGPRs, its mask (tiles that need one) and P(j+1) for keys 0..15:
    //      each group is product (row block 0), a pair's exps, product (row block
    //      1), the previous pair's sum and packing (one group after its exps,
    //      clear of their latency); groups 0..3 also read two K' operands each,
    //      so that the wait for them at the start of phase A finds them done.
    //      One wave issues in order and an MFMA leaves the VALU about 4 simple
    //      slots: with the two products back to back, the first one's slots
    //      went unused.
    // so that both phases carry about the same exp work beside their MFMAs
    // The step is written as small groups fenced by scheduling barriers, each an
    // MFMA pair plus the VALU and LDS work meant to run beside it: an MFMA leaves
    // the VALU only part of its cycles, so that work must be spread evenly.
    // MASKED steps (the tail loop) check at run time which tiles exist; the
    // others (the unrolled main loop) only run where tiles t+1..t+3 exist and
    // t+3 is full, and need no element mask.
    auto block_step = [&](auto S, auto SN, auto SNN, auto MASKED, int t, int kb) __attribute__((always_inline)) {
      const int j = 2 * t + kb;
      // (prefetched tiles: at tile 0, tile 1 is resident since the item's
      // first wait, for all outstanding loads, and the barrier after it, and
      // every wave has read its queries from stages 2 and 3)
      const bool first_ready = PREFETCH && tpre && t == 0;
      // (clean items' last tiles: past the last tile, the last tile again; see clean below)
      const int tn = decltype(MASKED)::value == 2 ? min(t + 3, nt - 1) : t + 3;
      if constexpr (decltype(MASKED)::value != 1) {
        // the loads of tile t+3 are spread over the QK^T groups below
        if (kb == 0 && !first_ready) {
          wait_vm<8>();
          tile_barrier();
        }
      } else if (kb == 0 && t + 1 < nt) {
        if (!first_ready) {
          if (t + 2 < nt) wait_vm<8>();
          else wait_vm<0>();
          tile_barrier();
        }
        if (t + 3 < nt) issue_tile(SNN, t + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- phase A: S(j+1) = K'(j+1) Q'^T + b; P(j) for keys 16..31; V(j) operands
      // lgkmcnt(0), as an instruction the compiler accounts for: the K' operands
      // read during the previous phase are complete here, so no drain is needed
      // later in this phase, after the V reads below have been issued
      __builtin_amdgcn_s_waitcnt(0xC07F);
      u32x4 pk1[2];
      float h1[2][2];  // set by pairs 0 and 1, added to by 2 and 3
  #pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[0][kk], kk == 0 ? btile[0] : sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[1][kk], kk == 0 ? btile[1] : sacc[1], 0, 0, 0);
        exp_pair(kk >> 2, 1, kk & 3, pk1[kk >> 2], h1[kk >> 2]);
        // keep the packed word here: it is only read after the check below,
        // and would otherwise be sunk past it
        asm volatile("" : "+v"(pk1[kk >> 2][kk & 3]));
        load_vop(S, kb, kk >> 1, kk & 1);
        if constexpr (decltype(MASKED)::value != 1) {
          if (kb == 0) issue_one(SNN, tn, kk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 pb[2][2];
      float bsum[2];
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        pb[qb][0] = pcar[qb];
        pb[qb][1] = __builtin_bit_cast(bf16x8, pk1[qb]);
        bsum[qb] = scar[qb] + (h1[qb][0] + h1[qb][1]);
      }
      // rare: marked unlikely so that the rescale is placed out of line and the
      // common path runs on without a taken branch (inline, every block ended in a
      // jump over it)
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(fmaxf(bsum[0], bsum[1]) > kLazySum) != 0, 0))
        move_reference(pb, bsum);
      lrun[0] += bsum[0];
      lrun[1] += bsum[1];
      __builtin_amdgcn_sched_barrier(0);
      // ---- phase B: O += V(j)^T P(j)^T; K'(j+2) operands; S(j+1) to VGPRs (and
      // its mask); P(j+1) for keys 0..15
      u32x4 pk0[2];
      float h0[2][2];  // set by pairs 0 and 1, added to by 2 and 3
      float lag0, lag1;  // the previous group's pair, summed and packed one group later
      auto finish_pair = [&](int gp, float a0, float a1) __attribute__((always_inline)) {
        const int qb = gp >> 2, e = gp & 3;
        if (e < 2) h0[qb][e & 1] = a0 + a1;
        else h0[qb][e & 1] += a0 + a1;
        pk0[qb][e] = pack_bf16x2(a0, a1);
        asm volatile("" : "+v"(pk0[qb][e]), "+v"(h0[qb][e & 1]));
      };
  #pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int db = g >> 1, sl = g & 1;
        const int qb = g >> 2, e = g & 3;  // the pair (keys 2e, 2e+1 of row block qb) of this group
        // O^T += V^T P^T with the accumulator in AGPRs (see acc_fence)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[0][db]) : "a"(vop[db][sl]), "v"(pb[0][sl]));
        if (g == 0) {
          take_scores();
          // (tail tiles: only blocks that reach past a row's visible keys)
          if constexpr (decltype(MASKED)::value == 1)
            if (32 * (j + 1) + 32 > kv_full) mask_scores(j + 1);
        }
        // the exps after this product, not hoisted above it (the two products
        // of a group would otherwise issue back to back)
        asm volatile("" : "+v"(sv[qb][2 * e]), "+v"(sv[qb][2 * e + 1]));
        const float p0 = __builtin_amdgcn_exp2f(sv[qb][2 * e]);
        const float p1 = __builtin_amdgcn_exp2f(sv[qb][2 * e + 1]);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[1][db]) : "a"(vop[db][sl]), "v"(pb[1][sl]));
        if (g > 0) asm volatile("" : "+v"(lag0), "+v"(lag1));
        if (g < 4) {
          load_kop(SN, kb, 2 * g);
          load_kop(SN, kb, 2 * g + 1);
        }
        if (g > 0) finish_pair(g - 1, lag0, lag1);
        lag0 = p0;
        lag1 = p1;
        __builtin_amdgcn_sched_barrier(0);
      }
      finish_pair(7, lag0, lag1);
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        pcar[qb] = __builtin_bit_cast(bf16x8, pk0[qb]);
        scar[qb] = h0[qb][0] + h0[qb][1];
      }
    };
    // step kinds: unmasked, masked (run-time checks of which tiles exist), and
    // unmasked with the load of tile t+3 clamped to the last tile
    using NoMask = std::integral_constant<int, 0>;
    using Mask = std::integral_constant<int, 1>;
    using Clamp = std::integral_constant<int, 2>;
    // Block j+1 (scored in step j) needs the element mask iff 32 (j+1) + 32 > kv_full,
    // i.e. from block jm = kv_full / 32 on.  Whole tiles whose steps score only
    // earlier blocks, and for which tile t+3 exists and is full, run in the
    // unrolled loop with compile-time stages; the rest (the last few tiles, or
    // the chunk a causal query tile straddles) run in a loop with run-time stages.
    const int jm = kv_full / 32;
    const int tm = max(0, min(min(nt, (jm - 1) / 2), Nk / kBN - 3));
    // A clean item (every visible key of every row in whole tiles: no causal
    // straddle, kv_end a multiple of kBN, at least kStages tiles) runs its last
    // tiles unmasked too, four at a time: those steps load the last tile again
    // into the stage that would take a tile past the last (one every wave has
    // left; only the discarded look-ahead block past the last reads it), so that
    // every tile start waits on the same count.  Cross attention over 512 text
    // keys is one; only its kernel has this copy of the step (in the main loop
    // the clamp cost register moves, and self attention's tails are short).
    const bool clean = kv_full == kv_end && kv_end == nt * kBN && nt >= kStages;
    auto tile_step = [&](auto S, auto SN, auto SNN, auto MASKED, int t) __attribute__((always_inline)) {
      block_step(S, SN, SNN, MASKED, t, 0);
      block_step(S, SN, SNN, MASKED, t, 1);
    };
    // unrolled over 8 tiles (the loop-carried scores and operands then return
    // to their registers without the copies a 4-tile body needed), then 4
    int t = 0;
    for (; t + 8 <= tm; t += 8) {
      tile_step(S0{}, S1{}, S3{}, NoMask{}, t);
      tile_step(S1{}, S2{}, S0{}, NoMask{}, t + 1);
      tile_step(S2{}, S3{}, S1{}, NoMask{}, t + 2);
      tile_step(S3{}, S0{}, S2{}, NoMask{}, t + 3);
      tile_step(S0{}, S1{}, S3{}, NoMask{}, t + 4);
      tile_step(S1{}, S2{}, S0{}, NoMask{}, t + 5);
      tile_step(S2{}, S3{}, S1{}, NoMask{}, t + 6);
      tile_step(S3{}, S0{}, S2{}, NoMask{}, t + 7);
    }
    for (; t + 4 <= tm; t += 4) {
      tile_step(S0{}, S1{}, S3{}, NoMask{}, t);
      tile_step(S1{}, S2{}, S0{}, NoMask{}, t + 1);
      tile_step(S2{}, S3{}, S1{}, NoMask{}, t + 2);
      tile_step(S3{}, S0{}, S2{}, NoMask{}, t + 3);
    }
    if constexpr (PREFETCH) {
      if (clean) {
        for (; t + 4 <= nt; t += 4) {
          tile_step(S0{}, S1{}, S3{}, Clamp{}, t);
          tile_step(S1{}, S2{}, S0{}, Clamp{}, t + 1);
          tile_step(S2{}, S3{}, S1{}, Clamp{}, t + 2);
          tile_step(S3{}, S0{}, S2{}, Clamp{}, t + 3);
        }
      }
    }
    for (; t < nt; ++t) tile_step(t, t + 1, t + 3, Mask{}, t);

    // 32 staged output rows (row m's chunk c at c ^ (m & 15), 256 bytes a row)
    // to O: lane (sr, sc) = (lane / 16, lane % 16) writes chunk sc of rows
    // 4 it + sr, 1 KiB (4 whole rows) per instruction.  All reads are issued
    // before the stores; a block that reaches past the last token checks each
    // row.  (irow0: the token of row sr)
    auto store_rows = [&](const char* rows, uint16_t* dst, bool whole, int irow0) __attribute__((always_inline)) {
      const int sr = lane >> 4, sc = lane & 15;
      u32x4 w[8];
  #pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = 4 * it + sr;
        w[it] = *(const u32x4*)(rows + row * kRowBytes + 16 * (sc ^ (row & 15)));
      }
      const size_t step = 4 * ((size_t)p.heads * kHeadDim);
      if (whole) {
  #pragma unroll
        for (int it = 0; it < 8; ++it) *(u32x4*)(dst + it * step) = w[it];
      } else {
  #pragma unroll
        for (int it = 0; it < 8; ++it)
          if (irow0 + 4 * it < p.N) *(u32x4*)(dst + it * step) = w[it];
      }
    };
    if (split) {
      // ---- partial epilogue: O, l and the bias as they stand, fp32, one
      // whole 1 KiB run of float4 per store instruction
      acc_fence();
      float4* po = p.part_o + (size_t)item * kPartO + (size_t)(2 * wave) * 16 * 64 + lane;
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float l = wave_half_sum(lrun[qb]);
        if (hh == 0) p.part_lb[(size_t)item * kBM + (2 * wave + qb) * 32 + r] = make_float2(l, bias[qb]);
  #pragma unroll
        for (int db = 0; db < 4; ++db)
  #pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            po[(qb * 16 + 4 * db + g4) * 64] =
                make_float4(acc[qb][db][4 * g4 + 0], acc[qb][db][4 * g4 + 1], acc[qb][db][4 * g4 + 2],
                            acc[qb][db][4 * g4 + 3]);
      }
      wait_vm<0>();
      continue;
    }

    // ---- epilogue: O = O^T / l, bf16.  A lane holds d = 32 db + 8 g4 + 4 hh + 0..3
    // of one query; each wave writes its 64 rows into LDS (chunks XOR-swizzled
    // by row) and reads them back as whole 256-byte rows, so that the stores to
    // O are 16 bytes per lane and 1 KiB (4 full rows) per instruction instead
    // of 8-byte pieces of 32 rows.  Every wave is past its last LDS operand read
    // and no tile load is in flight after the barrier.
    acc_fence();
    wait_vm<0>();
    tile_barrier();
    if constexpr (PREFETCH) {
      // the next item's first two tiles (into stages 0 and 1, which every
      // wave has left) and its query loads, issued before this epilogue
      qpre = tpre = false;
      const int Ln = static_item(p, pass + 1);
      if (Ln >= 0) {
        const int bhn = Ln / p.ntq, tqn = Ln - bhn * p.ntq;
        const int bn = bhn / p.heads, headn = bhn - bn * p.heads;
        // (an item with fewer tiles than stages zeroes the stages first)
        if ((p.lens[bn] + kBN - 1) / kBN >= kStages) {
          const char* kn = (const char*)(p.k + ((size_t)bn * p.Nk * p.heads + headn) * kHeadDim);
          const char* vn = (const char*)(p.v + ((size_t)bn * p.Nk * p.heads + headn) * kHeadDim);
          const uint32_t st0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)stage(S0{});
          const uint32_t st1 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)stage(S1{});
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int blk = 4 * wave + i;
            dma16(kn, koff_ld[i], st0 + blk * 1024);
            dma16(vn, voff_ld[i], st0 + kVHalves + blk * 1024);
          }
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int blk = 4 * wave + i;
            dma16(kn + (size_t)kBN * rsb, koff_ld[i], st1 + blk * 1024);
            dma16(vn + (size_t)kBN * rsb, voff_ld[i], st1 + kVHalves + blk * 1024);
          }
          tpre = true;
        }
        dma_q(bn, headn, tqn);
        qpre = true;
      }
      ++pass;
    }
    if constexpr (PREFETCH) {
      // O in two 32-row halves through this wave's 8 KiB above the stages
      char* orows = lds + kPrefetchStaging + wave * (32 * kRowBytes);
      const int sr = lane >> 4, sc = lane & 15;
  #pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float inv = 1.0f / wave_half_sum(lrun[qb]);
  #pragma unroll
        for (int db = 0; db < 4; ++db)
  #pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[qb][db][4 * g4 + 0] * inv, acc[qb][db][4 * g4 + 1] * inv);
            w[1] = pack_bf16x2(acc[qb][db][4 * g4 + 2] * inv, acc[qb][db][4 * g4 + 3] * inv);
            *(u32x2*)(orows + r * kRowBytes + 16 * ((4 * db + g4) ^ (r & 15)) + 8 * hh) = w;
          }
        const int irow0 = i0 + wave * 64 + qb * 32 + sr;
        store_rows(orows, p.o + ((size_t)b * p.N + irow0) * row_stride + (size_t)head * kHeadDim + 8 * sc,
                   i0 + wave * 64 + qb * 32 + 32 <= p.N, irow0);
      }
      continue;
    }
    char* orows = lds + wave * (64 * kRowBytes);
  #pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float inv = 1.0f / wave_half_sum(lrun[qb]);
      const int row = qb * 32 + r;
  #pragma unroll
      for (int db = 0; db < 4; ++db)
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[qb][db][4 * g4 + 0] * inv, acc[qb][db][4 * g4 + 1] * inv);
          w[1] = pack_bf16x2(acc[qb][db][4 * g4 + 2] * inv, acc[qb][db][4 * g4 + 3] * inv);
          *(u32x2*)(orows + row * kRowBytes + 16 * ((4 * db + g4) ^ (row & 15)) + 8 * hh) = w;
        }
    }
    const int sr = lane >> 4, sc = lane & 15;
  #pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int irow0 = i0 + wave * 64 + 32 * hf + sr;
      store_rows(orows + 32 * hf * kRowBytes,
                 p.o + ((size_t)b * p.N + irow0) * row_stride + (size_t)head * kHeadDim + 8 * sc,
                 i0 + wave * 64 + 32 * hf + 32 <= p.N, irow0);
    }
    if constexpr (!PERSIST) break;
  }
}

// the work queue counters of a persistent launch, zeroed before it (a kernel
// rather than a memset, so that the sequence can be captured in a graph)
__global__ void zero_queue_kernel(unsigned* queue) {
  if (threadIdx.x < kQueueCounters)
    __hip_atomic_store(queue + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- the key splits of the tail tiles combined.  Split s holds O_s and l_s
// against its own reference m_s = -b_s; with M = max_s m_s the row is
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s (the same rescaling the
// streaming softmax applies when its reference moves).  Workgroup: one
// (tile, 32-row block) of a tail tile; thread: 4 consecutive d of a row, in
// the partials' own order, so that every read is a whole 1 KiB run.
struct MergeParams {
  const float4* part_o;
  const float2* part_lb;
  uint16_t* o;
  int first;   // tile index (in the attention kernel's order) of the first tail tile
  int ntq, heads, N, nsplit;
};

__global__ void __launch_bounds__(256) split_merge_kernel(MergeParams p) {
  const int tile = blockIdx.x >> 3, blk = blockIdx.x & 7;  // blk = 2 wave + qb
  const int L = p.first + tile;
  const int bh = L / p.ntq, tq = L - bh * p.ntq;
  const int b = bh / p.heads, head = bh - b * p.heads;
  const int item0 = tile * p.nsplit;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = threadIdx.x + 256 * k;  // (4 db + g4) * 64 + lane
    const int lane = c & 63, dg = c >> 6, r = lane & 31, hh = lane >> 5;
    const int row = tq * kBM + 32 * blk + r;
    float m = -__builtin_inff();
    for (int s = 0; s < p.nsplit; ++s) m = fmaxf(m, -p.part_lb[(size_t)(item0 + s) * kBM + 32 * blk + r].y);
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float l = 0.0f;
    for (int s = 0; s < p.nsplit; ++s) {
      const float2 lb = p.part_lb[(size_t)(item0 + s) * kBM + 32 * blk + r];
      const float w = __builtin_amdgcn_exp2f(-lb.y - m);
      const float4 os = p.part_o[(size_t)(item0 + s) * kPartO + (16 * blk + dg) * 64 + lane];
      l += w * lb.x;
      o.x += w * os.x;
      o.y += w * os.y;
      o.z += w * os.z;
      o.w += w * os.w;
    }
    const float inv = 1.0f / l;
    if (row < p.N) {
      u32x2 wd;
      wd[0] = pack_bf16x2(o.x * inv, o.y * inv);
      wd[1] = pack_bf16x2(o.z * inv, o.w * inv);
      const int d = 32 * (dg >> 2) + 8 * (dg & 3) + 4 * hh;
      *(u32x2*)(p.o + ((size_t)b * p.N + row) * ((size_t)p.heads * kHeadDim) + (size_t)head * kHeadDim + d) = wd;
    }
  }
}

}  // namespace wanattn
