// C ABI of libwanattn: argument checks, the rotary tables, kernel launches.
// The operations are defined in include/wanattn.h.

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn_fwd.h"
#include "prologue.h"
#include "rope3d.h"
#include "wanattn.h"

using namespace wanattn;

#define WA_TRY(x)                        \
  do {                                   \
    wanattn_status st_ = (x);            \
    if (st_ != WANATTN_OK) return st_;   \
  } while (0)


namespace {

constexpr int kSlots = 8;       // distinct theta values kept per device
constexpr int kMaxDevices = 64;

// Rotary tables, one per theta slot, resident on every device the library runs on.
__device__ float2 g_rope_tab[kSlots][kTabEntries];

}  // namespace

// Scratch memory of wanattn_self_noalloc: the rotated keys, the key-split
// partials and the work-queue counters of one call, for callers that cannot
// allocate.  Every device the library runs on holds its own copy until the
// process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (DeviceState::scratch).
static __device__ __align__(256) unsigned char scratch[WANATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// Per-device state, set up once per device by the first call that runs there
// (device_state): the device addresses of the module-scope arrays and one
// event per theta slot.  A slot's table is built by rope_table_kernel on the
// stream of the first call that uses its theta; the event recorded after that
// build lets calls on other streams wait for it.
struct DeviceState {
  bool ready = false;
  float2* tab = nullptr;                 // g_rope_tab on this device
  unsigned char* scratch = nullptr;      // scratch on this device
  double theta[kSlots];
  bool built[kSlots];                    // an eager build of the slot was enqueued ...
  hipStream_t built_on[kSlots];          // ... on this stream,
  hipEvent_t ev[kSlots];                 // followed by this event
  bool done[kSlots];                     // the event has completed
  int used = 0;
};
DeviceState g_dev[kMaxDevices];
std::mutex g_mu;

thread_local char t_err[512] = "";

wanattn_status fail(wanattn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
wanattn_status fail(wanattn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_err, sizeof t_err, fmt, ap);
  va_end(ap);
  return s;
}

// the current device's state, set up on first use (caller holds g_mu)
wanattn_status device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(WANATTN_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(WANATTN_E_UNSUPPORTED, "device %d out of range", dev);
  DeviceState& d = g_dev[dev];
  if (!d.ready) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_rope_tab));
    if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipGetSymbolAddress(rotary tables): %s", hipGetErrorString(e));
    d.tab = (float2*)ptr;
    ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    d.scratch = (unsigned char*)ptr;
    for (int s = 0; s < kSlots; ++s) {
      e = hipEventCreateWithFlags(&d.ev[s], hipEventDisableTiming);
      if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipEventCreate: %s", hipGetErrorString(e));
      d.built[s] = d.done[s] = false;
      d.built_on[s] = nullptr;
    }
    d.ready = true;
  }
  *out = &d;
  return WANATTN_OK;
}

// rope_table_kernel for one theta into one slot, on `stream`
wanattn_status launch_table(double theta, float2* tab, hipStream_t stream) {
  TableParams tp;
  memset(&tp, 0, sizeof tp);
  tp.tab = tab;
  tp.heads = 1;
  tp.theta[0] = theta;
  hipLaunchKernelGGL(rope_table_kernel, dim3(kTabEntries / 256), dim3(256), 0, stream, tp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WANATTN_E_HIP, "rope_table launch: %s", hipGetErrorString(e));
  return WANATTN_OK;
}

// Device address of the table for theta on the current device, ready for
// work enqueued on `stream` after this call.  The first use of a theta on a
// device builds its slot on `stream` (the same fp64 formula as the per-head
// tables of the jitter calls); a later use on another stream waits for that
// build's event until it is known to have completed.  Under stream capture
// the graph gets its own build of the slot (identical values) instead of a
// dependency on work outside the graph, and an eager call later builds the
// slot again.  Nothing here blocks the host.
wanattn_status table_for(double theta, hipStream_t stream, const float2** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState* dp = nullptr;
  WA_TRY(device_state(&dp));
  DeviceState& d = *dp;
  int s = 0;
  while (s < d.used && d.theta[s] != theta) ++s;
  if (s == d.used) {
    if (d.used == kSlots) return fail(WANATTN_E_UNSUPPORTED, "more than %d distinct theta values on one device", kSlots);
    d.theta[s] = theta;
    d.built[s] = d.done[s] = false;
    ++d.used;
  }
  float2* tab = d.tab + (size_t)s * kTabEntries;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cap != hipStreamCaptureStatusNone) {
    // the graph builds the slot itself unless an eager build is known complete
    if (!d.built[s] || !d.done[s]) WA_TRY(launch_table(theta, tab, stream));
  } else if (!d.built[s]) {
    WA_TRY(launch_table(theta, tab, stream));
    e = hipEventRecord(d.ev[s], stream);
    if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    d.built[s] = true;
    d.built_on[s] = stream;
  } else if (!d.done[s]) {
    e = hipEventQuery(d.ev[s]);
    if (e == hipSuccess) {
      d.done[s] = true;
    } else if (e != hipErrorNotReady) {
      return fail(WANATTN_E_HIP, "hipEventQuery: %s", hipGetErrorString(e));
    } else if (stream != d.built_on[s]) {
      e = hipStreamWaitEvent(stream, d.ev[s], 0);
      if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
    }
  }
  *out = tab;
  return WANATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

wanattn_status check_grid(const wanattn_grid3d* g, int32_t N) {
  if (!g) return fail(WANATTN_E_INVALID, "grid is NULL");
  if (g->F < 1 || g->H < 1 || g->W < 1) return fail(WANATTN_E_INVALID, "grid dims must be >= 1");
  if ((long long)g->F * g->H * g->W != N)
    return fail(WANATTN_E_INVALID, "N=%d != F*H*W = %d*%d*%d", N, g->F, g->H, g->W);
  if (g->f0 < 0 || g->h0 < 0 || g->w0 < 0) return fail(WANATTN_E_INVALID, "position offsets must be >= 0");
  if ((long long)g->F + g->f0 > kMaxPos || (long long)g->H + g->h0 > kMaxPos ||
      (long long)g->W + g->w0 > kMaxPos)
    return fail(WANATTN_E_INVALID, "RoPE positions must stay below %d", kMaxPos);
  return WANATTN_OK;
}

wanattn_status check_theta(double theta) {
  if (!(theta > 0.0) || !std::isfinite(theta)) return fail(WANATTN_E_INVALID, "theta must be finite and > 0");
  return WANATTN_OK;
}

wanattn_status check_tensor_sizes(int32_t B, int32_t N, int32_t heads, int32_t head_dim) {
  if (B < 1 || N < 1 || heads < 1) return fail(WANATTN_E_INVALID, "B, N and heads must be >= 1");
  if (N > (1 << 30)) return fail(WANATTN_E_INVALID, "N=%d above 2^30 tokens", N);
  if (head_dim != kHeadDim) return fail(WANATTN_E_UNSUPPORTED, "head_dim %d (only 128 is built)", head_dim);
  if ((long long)B * N * heads * kHeadDim > (1ll << 40)) return fail(WANATTN_E_INVALID, "tensor too large");
  // the attention kernels address 64 consecutive token rows with 32-bit offsets
  if (heads > WANATTN_MAX_HEADS) return fail(WANATTN_E_UNSUPPORTED, "heads=%d above %d", heads, WANATTN_MAX_HEADS);
  return WANATTN_OK;
}

// one attention launch covers up to WANATTN_MAX_LEN_BATCH batches x heads x
// query tiles workgroups of kThreads; a launch takes at most 2^32 - 1 threads
wanattn_status check_launch_size(int32_t B, int32_t N, int32_t heads) {
  const long long nb = B < WANATTN_MAX_LEN_BATCH ? B : WANATTN_MAX_LEN_BATCH;
  const long long wgs = nb * heads * ((N + kBM - 1) / kBM);
  if (wgs * kThreads > 0xFFFFFFFFll)
    return fail(WANATTN_E_UNSUPPORTED, "%lld workgroups of %d threads exceed one launch", wgs, kThreads);
  return WANATTN_OK;
}

wanattn_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WANATTN_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return WANATTN_OK;
}

wanattn_status check_lens(int32_t B, const int32_t* lens, int32_t maxlen, const char* name) {
  if (!lens) return WANATTN_OK;
  for (int b = 0; b < B; ++b)
    if (lens[b] < 1 || lens[b] > maxlen)
      return fail(WANATTN_E_INVALID, "%s[%d]=%d outside [1, %d]", name, b, lens[b], maxlen);
  return WANATTN_OK;
}

// Persistent launches and tail splitting of bidirectional self attention.
// The XCDs of one chip run at measurably different speeds (mean workgroup
// times up to ~7% apart at 75,600 x 40), while a plain launch gives every XCD
// the same share of workgroups.  With room in the workspace, the self-attention kernel is
// launched with one workgroup per compute unit, and each workgroup takes query
// tiles from its XCD's run of tiles, then from the other XCDs' runs, then the
// split items below (next_item): a fast XCD ends up doing more tiles.
// A launch of T workgroups on
// a chip of C compute units runs floor(T / C) full waves of workgroups and then
// T % C alone, which leaves most of the chip idle for a whole workgroup's time;
// and the workgroups of the last full wave end over a spread of times (they
// started over one), during which the chip empties.  The last query tiles run
// instead as nsplit workgroups each, every one over a range of the key tiles,
// writing fp32 partials into the caller's workspace; a small kernel then
// combines them.  The short workgroups fill the chip as it empties:
//  - a remainder of at most C / 2 tiles: nsplit = C / remainder (at most 8);
//  - no remainder, at least 12 waves: the last wave, nsplit = 2 (the spread
//    builds up over the waves: at 6 waves the split cost 0.5%, at 20 it gained
//    0.7%).
// (Measured inside the persistent launch, 40 heads: 75,600 tokens 81.1 ->
// 80.8 ms, 32,760 tokens 15.49 -> 15.34 ms.)
// kSplitItemBytes per split workgroup.
constexpr int kMaxSplit = 8;
constexpr int kMaxSplitItems = 512;
constexpr size_t kSplitItemBytes = (size_t)kPartO * sizeof(float4) + (size_t)kBM * sizeof(float2);

constexpr size_t kQueueBytes = 256;  // the persistent launch's queue counters

// split workgroups a self-attention call can use (its workspace holds that many)
size_t split_items(int32_t B, int32_t N, int32_t heads) {
  const long long nb = B < WANATTN_MAX_LEN_BATCH ? B : WANATTN_MAX_LEN_BATCH;
  const long long wgs = nb * heads * ((N + kBM - 1) / kBM);
  return (size_t)(wgs < kMaxSplitItems ? wgs : kMaxSplitItems);
}

// compute units of the current device (0 if unknown)
int device_cus() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return ncu;
}

// the split (0: none) for a launch of `total` tiles on ncu compute units whose
// shortest visible key range is minlen, with room for `room` split items
int choose_split(int total, int ncu, int minlen, size_t room, int* tail_out) {
  if (ncu < 2) return 0;
  const int rem = total % ncu;
  int tail, nsplit;
  if (rem == 0 && total >= 12 * ncu) {
    tail = ncu;
    nsplit = 2;
  } else if (rem > 0 && total > ncu && 2 * rem <= ncu) {
    tail = rem;
    nsplit = ncu / rem < kMaxSplit ? ncu / rem : kMaxSplit;
  } else {
    return 0;
  }
  // at least 8 key tiles per range: shorter ones gain less than they cost
  const int nkt = (minlen + kBN - 1) / kBN;
  while (nsplit > 1 && nkt < 8 * nsplit) --nsplit;
  while (nsplit > 1 && (size_t)tail * nsplit > room) --nsplit;
  if (nsplit < 2) return 0;
  *tail_out = tail;
  return nsplit;
}

// Launch over groups of at most WANATTN_MAX_LEN_BATCH batches so that the
// per-batch key lengths always fit the kernel argument block.  `part` (room
// for part_items split items followed by kQueueBytes, or null) enables
// persistent launches and tail splitting.
template <bool ROPE, bool CAUSAL, bool QNORM = false>
wanattn_status launch_attn(AttnParams p, int32_t B, const int32_t* lens, hipStream_t stream,
                           void* part = nullptr, size_t part_items = 0) {
  const size_t qstride = (size_t)p.N * p.heads * kHeadDim, kstride = (size_t)p.Nk * p.heads * kHeadDim;
  const uint16_t *q0 = p.q, *k0 = p.k, *v0 = p.v;
  uint16_t* o0 = p.o;
  const float* q_rms0 = p.q_rms;
  p.ntq = (p.N + kBM - 1) / kBM;
  for (int b0 = 0; b0 < B; b0 += WANATTN_MAX_LEN_BATCH) {
    const int nb = B - b0 < WANATTN_MAX_LEN_BATCH ? B - b0 : WANATTN_MAX_LEN_BATCH;
    p.q = q0 + (size_t)b0 * qstride;
    p.k = k0 + (size_t)b0 * kstride;
    p.v = v0 + (size_t)b0 * kstride;
    p.o = o0 + (size_t)b0 * qstride;
    if constexpr (QNORM) p.q_rms = q_rms0 + (size_t)b0 * p.N;
    for (int b = 0; b < nb; ++b) p.lens[b] = lens ? lens[b0 + b] : p.Nk;
    p.total = nb * p.heads * p.ntq;
    if constexpr (ROPE) {
      const int ncu = part ? device_cus() : 0;
      if (ncu > 0 && p.total >= ncu) {
        // key splits only under the bidirectional mask
        int minlen = p.Nk, tail = 0;
        for (int b = 0; b < nb; ++b) minlen = p.lens[b] < minlen ? p.lens[b] : minlen;
        const int nsplit = CAUSAL ? 0 : choose_split(p.total, ncu, minlen, part_items, &tail);
        p.total -= tail;
        p.nsplit = nsplit > 0 ? nsplit : 1;
        p.nsplit_items = tail * nsplit;
        p.part_o = (float4*)part;
        p.part_lb = (float2*)((char*)part + part_items * kPartO * sizeof(float4));
        p.queue = (unsigned*)((char*)part + part_items * kSplitItemBytes);
        hipLaunchKernelGGL(zero_queue_kernel, dim3(1), dim3(64), 0, stream, p.queue);
        WA_TRY(launched("queue reset"));
        hipLaunchKernelGGL((attn_fwd_kernel<ROPE, CAUSAL, true, QNORM>), dim3(ncu), dim3(kThreads), 0, stream, p);
        WA_TRY(launched("attention"));
        if (nsplit) {
          MergeParams m{p.part_o, p.part_lb, p.o, p.total, p.ntq, p.heads, p.N, nsplit};
          hipLaunchKernelGGL(split_merge_kernel, dim3(tail * 8), dim3(256), 0, stream, m);
          WA_TRY(launched("split merge"));
        }
        continue;
      }
    }
    if constexpr (!ROPE && !CAUSAL) {
      // cross attention: one workgroup per compute unit (a multiple of 8, so
      // that each XCD gets the same share), items in a fixed order, each
      // workgroup issuing its next item's first loads before its epilogue
      const int ncu = device_cus();
      const int grid = (ncu / 8) * 8;
      if (grid >= 8 && p.total >= grid) {
        hipLaunchKernelGGL((attn_fwd_kernel<false, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
        WA_TRY(launched("cross attention"));
        continue;
      }
    }
    hipLaunchKernelGGL((attn_fwd_kernel<ROPE, CAUSAL, false, QNORM>), dim3(p.total), dim3(kThreads), 0, stream, p);
    WA_TRY(launched("attention"));
  }
  return WANATTN_OK;
}

// 3D RoPE of a whole tensor with the table(s) at `tab` (head h's table at
// tab + h * hstride); arguments already checked
wanattn_status rope3d_launch(const void* x, void* y, int32_t B, int32_t N, int32_t heads,
                             const wanattn_grid3d* grid, const float2* tab, long long hstride,
                             hipStream_t stream, const float* rms = nullptr, const void* gamma = nullptr) {
  RopeParams p;
  p.rms = rms;
  p.gamma = (const uint16_t*)gamma;
  p.x = (const u32x4*)x;
  p.y = (u32x4*)y;
  p.tab = tab;
  p.tab_hstride = hstride;
  p.tokens = (long long)B * N;
  p.N = N;
  p.heads = heads;
  p.H = grid->H;
  p.W = grid->W;
  p.f0 = grid->f0;
  p.h0 = grid->h0;
  p.w0 = grid->w0;
  p.inv_hw = 1.0 / ((double)grid->H * grid->W);
  p.inv_w = 1.0 / (double)grid->W;
  // one wave per token, 4 per workgroup; the grid-stride loop only matters
  // past 2^24 workgroups
  long long blocks = (p.tokens + 3) / 4;
  if (blocks > (1LL << 24)) blocks = 1LL << 24;
  hipLaunchKernelGGL(rope3d_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return launched("rope3d");
}

// 3D RoPE of a whole tensor on `stream` (checked arguments)
wanattn_status rope3d_checked(const void* x, void* y, int32_t B, int32_t N, int32_t heads,
                              int32_t head_dim, const wanattn_grid3d* grid, double theta,
                              hipStream_t stream) {
  t_err[0] = 0;
  if (!x || !y) return fail(WANATTN_E_INVALID, "null tensor pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  WA_TRY(check_tensor_sizes(B, N, heads, head_dim));
  WA_TRY(check_grid(grid, N));
  WA_TRY(check_theta(theta));
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  if (x != y && overlap(x, bytes, y, bytes)) return fail(WANATTN_E_INVALID, "y partially overlaps x");
  const float2* tab = nullptr;
  WA_TRY(table_for(theta, stream, &tab));
  return rope3d_launch(x, y, B, N, heads, grid, tab, 0, stream);
}

// argument checks shared by the self-attention entry points (theta checked by
// the caller); the workspace must hold ws_need bytes, of which the call uses
// ws_use (ws_need, or more where the tail split's partials fit)
wanattn_status check_self_args(const void* q, const void* k, const void* v, const void* o, int32_t B, int32_t N,
                               int32_t heads, int32_t head_dim, const wanattn_grid3d* grid, float scale,
                               wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens) {
  if (!q || !k || !v || !o) return fail(WANATTN_E_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  WA_TRY(check_tensor_sizes(B, N, heads, head_dim));
  WA_TRY(check_launch_size(B, N, heads));
  WA_TRY(check_grid(grid, N));
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(WANATTN_E_INVALID, "scale must be finite and > 0");
  if (mask != WANATTN_MASK_NONE && mask != WANATTN_MASK_BLOCK_CAUSAL)
    return fail(WANATTN_E_INVALID, "unknown mask %d", (int)mask);
  if (mask == WANATTN_MASK_BLOCK_CAUSAL && chunk_frames < 1)
    return fail(WANATTN_E_INVALID, "chunk_frames must be >= 1 for the block-causal mask");
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, bytes) || overlap(o, bytes, v, bytes))
    return fail(WANATTN_E_INVALID, "o overlaps an input");
  return check_lens(B, kv_lens, N, "kv_lens");
}

// ... and of the caller's workspace
wanattn_status check_self(const void* q, const void* k, const void* v, const void* o, int32_t B, int32_t N,
                          int32_t heads, int32_t head_dim, const wanattn_grid3d* grid, float scale,
                          wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                          const void* workspace, size_t workspace_bytes, size_t ws_need, size_t ws_use) {
  WA_TRY(check_self_args(q, k, v, o, B, N, heads, head_dim, grid, scale, mask, chunk_frames, kv_lens));
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  if (!workspace) return fail(WANATTN_E_INVALID, "workspace is NULL");
  if (!aligned16(workspace)) return fail(WANATTN_E_INVALID, "workspace must be 16-byte aligned");
  if (workspace_bytes < ws_need)
    return fail(WANATTN_E_INVALID, "workspace has %zu bytes, %zu needed", workspace_bytes, ws_need);
  if (overlap(workspace, ws_use, q, bytes) || overlap(workspace, ws_use, k, bytes) ||
      overlap(workspace, ws_use, v, bytes) || overlap(workspace, ws_use, o, bytes))
    return fail(WANATTN_E_INVALID, "workspace overlaps a tensor");
  return WANATTN_OK;
}

// keys rotated once into kprime (with head h's table at tab + h * hstride);
// the queries are rotated by the attention kernel as it loads them
// (rms, gq, gk non-null: q and k are projections before the QK-Norm, whose
// factors rms holds, q's then k's; the norm is applied as q is loaded and as k
// is rotated)
wanattn_status self_launch(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t N,
                           int32_t heads, const wanattn_grid3d* grid, float scale, wanattn_mask mask,
                           int32_t chunk_frames, const int32_t* kv_lens, void* kprime, const float2* tab,
                           long long hstride, void* part, size_t part_items, hipStream_t stream,
                           const float* rms = nullptr, const void* gq = nullptr, const void* gk = nullptr) {
  WA_TRY(rope3d_launch(k, kprime, B, N, heads, grid, tab, hstride, stream, rms ? rms + (size_t)B * N : nullptr, gk));
  AttnParams p;
  memset(&p, 0, sizeof p);
  p.q_rms = rms;
  p.gq = (const uint16_t*)gq;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)kprime;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.tab = tab;
  p.tab_hstride = hstride;
  p.N = N;
  p.Nk = N;
  p.heads = heads;
  p.qscale = scale * 1.4426950408889634f;
  p.H = grid->H;
  p.W = grid->W;
  p.f0 = grid->f0;
  p.h0 = grid->h0;
  p.w0 = grid->w0;
  p.inv_hw = 1.0 / ((double)grid->H * grid->W);
  p.inv_w = 1.0 / (double)grid->W;
  if (mask == WANATTN_MASK_BLOCK_CAUSAL) {
    long long ct = (long long)chunk_frames * grid->H * grid->W;
    p.chunk_tokens = (int)(ct < N ? ct : N);
    if (rms) return launch_attn<true, true, true>(p, B, kv_lens, stream, part, part_items);
    return launch_attn<true, true>(p, B, kv_lens, stream, part, part_items);
  }
  if (rms) return launch_attn<true, false, true>(p, B, kv_lens, stream, part, part_items);
  return launch_attn<true, false>(p, B, kv_lens, stream, part, part_items);
}

size_t jitter_table_bytes(int heads) { return (size_t)heads * kTabEntries * sizeof(float2); }

wanattn_status check_head_thetas(const double* theta_per_head, int32_t heads) {
  if (heads < 1) return fail(WANATTN_E_INVALID, "heads must be >= 1");
  if (heads > kMaxJitterHeads)
    return fail(WANATTN_E_UNSUPPORTED, "heads=%d above %d for per-head tables", heads, kMaxJitterHeads);
  if (!theta_per_head) return fail(WANATTN_E_INVALID, "theta_per_head is NULL");
  for (int h = 0; h < heads; ++h)
    if (!(theta_per_head[h] > 0.0) || !std::isfinite(theta_per_head[h]))
      return fail(WANATTN_E_INVALID, "theta_per_head[%d] must be finite and > 0", h);
  return WANATTN_OK;
}

// per-head tables for checked bases into `tab` (heads * kTabEntries entries)
wanattn_status build_head_tables(const double* theta_per_head, int32_t heads, float2* tab, hipStream_t stream) {
  TableParams tp;
  memset(&tp, 0, sizeof tp);
  tp.tab = tab;
  tp.heads = heads;
  for (int h = 0; h < heads; ++h) tp.theta[h] = theta_per_head[h];
  const long long total = (long long)heads * kTabEntries;
  long long blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, tp);
  return launched("rope_table");
}

// a caller's table set: heads tables of kTabEntries entries
wanattn_status check_tables(const void* tables, size_t tables_bytes, int32_t heads) {
  if (!tables) return fail(WANATTN_E_INVALID, "tables is NULL");
  if (!aligned16(tables)) return fail(WANATTN_E_INVALID, "tables must be 16-byte aligned");
  if (heads > kMaxJitterHeads)
    return fail(WANATTN_E_UNSUPPORTED, "heads=%d above %d for per-head tables", heads, kMaxJitterHeads);
  if (tables_bytes < jitter_table_bytes(heads))
    return fail(WANATTN_E_INVALID, "tables has %zu bytes, %zu needed for %d heads", tables_bytes,
                jitter_table_bytes(heads), heads);
  return WANATTN_OK;
}

// checks of the KV-cache streaming call (the table is checked by the caller)
wanattn_status check_kv(const void* q, const void* k_cache, const void* v_cache, const void* o, int32_t B,
                        int32_t Nq, int32_t Nkv, int32_t heads, int32_t head_dim, const wanattn_grid3d* grid_q,
                        float scale, const int32_t* kv_lens) {
  if (!q || !k_cache || !v_cache || !o) return fail(WANATTN_E_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  WA_TRY(check_tensor_sizes(B, Nq, heads, head_dim));
  WA_TRY(check_tensor_sizes(B, Nkv, heads, head_dim));
  WA_TRY(check_launch_size(B, Nq, heads));
  WA_TRY(check_grid(grid_q, Nq));
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(WANATTN_E_INVALID, "scale must be finite and > 0");
  const long long hw = (long long)grid_q->H * grid_q->W;
  if (Nkv % hw != 0) return fail(WANATTN_E_INVALID, "Nkv=%d is not whole frames of %lld tokens", Nkv, hw);
  const size_t qbytes = (size_t)B * Nq * heads * kHeadDim * 2, kbytes = (size_t)B * Nkv * heads * kHeadDim * 2;
  if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k_cache, kbytes) || overlap(o, qbytes, v_cache, kbytes))
    return fail(WANATTN_E_INVALID, "o overlaps an input");
  return check_lens(B, kv_lens, Nkv, "kv_lens");
}

// one chunk of queries against the rotated cache, head h's table at tab + h * hstride
wanattn_status kv_launch(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t B, int32_t Nq,
                         int32_t Nkv, int32_t heads, const wanattn_grid3d* grid_q, const float2* tab,
                         long long hstride, float scale, const int32_t* kv_lens, hipStream_t stream) {
  AttnParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_cache;
  p.v = (const uint16_t*)v_cache;
  p.o = (uint16_t*)o;
  p.tab = tab;
  p.tab_hstride = hstride;
  p.N = Nq;
  p.Nk = Nkv;
  p.heads = heads;
  p.qscale = scale * 1.4426950408889634f;
  p.H = grid_q->H;
  p.W = grid_q->W;
  p.f0 = grid_q->f0;
  p.h0 = grid_q->h0;
  p.w0 = grid_q->w0;
  p.inv_hw = 1.0 / ((double)grid_q->H * grid_q->W);
  p.inv_w = 1.0 / (double)grid_q->W;
  return launch_attn<true, false>(p, B, kv_lens, stream);
}

// ---- q/k/v projections: plain bf16 GEMMs in hipBLASLt ---------------------

constexpr size_t kGemmWorkspace = size_t(128) << 20;  // hipBLASLt's share of the prologue workspace
constexpr long long kMaxPrologueRows = 1ll << 24;    // B * N tokens per prologue call

hipblasLtHandle_t g_lt[kMaxDevices];

// algorithm chosen by the library's heuristic for one (device, dim, rows) shape
struct GemmPlan {
  int dev = -1, dim = 0;
  long long rows = 0;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
};
constexpr int kPlans = 32;
GemmPlan g_plans[kPlans];
int g_plan_next = 0;

#define LT_TRY(call, what)                                                        \
  do {                                                                            \
    hipblasStatus_t s_ = (call);                                                  \
    if (s_ != HIPBLAS_STATUS_SUCCESS)                                             \
      return fail(WANATTN_E_HIP, "%s: hipBLASLt status %d", what, (int)s_);      \
  } while (0)

// descriptors of out[rows, dim] = y[rows, dim] W^T + bias, all row-major bf16.
// In the library's column-major terms D = op(A) B with m = dim (output
// features), n = rows (tokens), k = dim: A is W read as a k x m matrix and
// transposed, B is y read as k x n, D is the output read as m x n, and the
// bias (length m) is broadcast over the tokens.
struct ProjDesc {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  ~ProjDesc() {
    if (d) hipblasLtMatrixLayoutDestroy(d);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
  wanattn_status init(int dim, long long rows) {
    LT_TRY(hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F), "matmul descriptor");
    const int32_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    const uint32_t epi = HIPBLASLT_EPILOGUE_BIAS;
    const int32_t bias_type = HIP_R_16BF;
    LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta), "TRANSA");
    LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb), "TRANSB");
    LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof epi), "EPILOGUE");
    LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                           sizeof bias_type), "BIAS_DATA_TYPE");
    LT_TRY(hipblasLtMatrixLayoutCreate(&a, HIP_R_16BF, dim, dim, dim), "layout A");
    LT_TRY(hipblasLtMatrixLayoutCreate(&b, HIP_R_16BF, dim, rows, dim), "layout B");
    LT_TRY(hipblasLtMatrixLayoutCreate(&d, HIP_R_16BF, dim, rows, dim), "layout D");
    return WANATTN_OK;
  }
  wanattn_status set_bias(const void* bias) {
    LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof bias),
           "BIAS_POINTER");
    return WANATTN_OK;
  }
};

// handle and algorithm for this shape on the current device (created on first use)
wanattn_status gemm_plan(ProjDesc& pd, int dim, long long rows, hipblasLtHandle_t* h, GemmPlan* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(WANATTN_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(WANATTN_E_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_lt[dev]) LT_TRY(hipblasLtCreate(&g_lt[dev]), "hipblasLtCreate");
  *h = g_lt[dev];
  for (const GemmPlan& g : g_plans)
    if (g.dev == dev && g.dim == dim && g.rows == rows) {
      *out = g;
      return WANATTN_OK;
    }
  hipblasLtMatmulPreference_t pref = nullptr;
  LT_TRY(hipblasLtMatmulPreferenceCreate(&pref), "preference");
  const uint64_t max_ws = kGemmWorkspace;
  hipblasStatus_t s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                            &max_ws, sizeof max_ws);
  // the best-ranked candidate whose workspace fits (some library builds rank
  // candidates above the workspace preference)
  constexpr int kCand = 8;
  hipblasLtMatmulHeuristicResult_t res[kCand];
  int count = 0;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulAlgoGetHeuristic(*h, pd.op, pd.a, pd.b, pd.d, pd.d, pref, kCand, res, &count);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (s != HIPBLAS_STATUS_SUCCESS) return fail(WANATTN_E_HIP, "algorithm query: hipBLASLt status %d", (int)s);
  int pick = -1;
  for (int i = 0; i < count && i < kCand && pick < 0; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kGemmWorkspace) pick = i;
  if (pick < 0)
    return fail(WANATTN_E_UNSUPPORTED, "hipBLASLt has no algorithm for a %d x %d x %lld bf16 GEMM with bias "
                "within %zu bytes of workspace", dim, dim, rows, kGemmWorkspace);
  GemmPlan& g = g_plans[g_plan_next];
  g_plan_next = (g_plan_next + 1) % kPlans;
  g.dev = dev;
  g.dim = dim;
  g.rows = rows;
  g.algo = res[pick].algo;
  g.ws = res[pick].workspaceSize;
  *out = g;
  return WANATTN_OK;
}

size_t prologue_y_bytes(long long rows, int dim) { return ((size_t)rows * dim * 2 + 255) & ~size_t(255); }

// the prologue up to the projections, then either the QK RMSNorm in place
// (rms null; gq, gk its weights) or only its per-row factors into rms
wanattn_status prologue_core(const void* x, const float* e0, const float* e1, const void* wq, const void* bq,
                             const void* wk, const void* bk, const void* wv, const void* bv, const void* gq,
                             const void* gk, void* q, void* k, void* v, float* rms, int32_t B, int32_t N,
                             int32_t dim, float eps_ln, float eps_rms, void* workspace, size_t workspace_bytes,
                             void* stream) {
  t_err[0] = 0;
  const void* ins[11] = {x, e0, e1, wq, bq, wk, bk, wv, bv, rms ? x : gq, rms ? x : gk};
  void* outs[3] = {q, k, v};
  for (const void* a : ins)
    if (!a) return fail(WANATTN_E_INVALID, "null input pointer");
  if (rms && ((uintptr_t)rms & 15u) != 0) return fail(WANATTN_E_INVALID, "rms must be 16-byte aligned");
  for (const void* a : outs)
    if (!a) return fail(WANATTN_E_INVALID, "null output pointer");
  for (const void* a : ins)
    if (!aligned16(a)) return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  for (const void* a : outs)
    if (!aligned16(a)) return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  if (B < 1 || N < 1) return fail(WANATTN_E_INVALID, "B and N must be >= 1");
  if (dim < 8 || dim % 8 != 0) return fail(WANATTN_E_INVALID, "dim=%d must be a positive multiple of 8", dim);
  if (dim > kMaxRowDim) return fail(WANATTN_E_UNSUPPORTED, "dim=%d above %d", dim, kMaxRowDim);
  const long long rows = (long long)B * N;
  if (rows > kMaxPrologueRows) return fail(WANATTN_E_UNSUPPORTED, "B*N=%lld above %lld tokens", rows, kMaxPrologueRows);
  if (!(eps_ln >= 0.0f) || !std::isfinite(eps_ln) || !(eps_rms >= 0.0f) || !std::isfinite(eps_rms))
    return fail(WANATTN_E_INVALID, "eps_ln and eps_rms must be finite and >= 0");
  const size_t act = (size_t)rows * dim * 2, mat = (size_t)dim * dim * 2, vec = (size_t)dim * 2,
               mod = (size_t)B * dim * 4;
  const size_t in_bytes[11] = {act, mod, mod, mat, vec, mat, vec, mat, vec, vec, vec};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 11; ++j)
      if (overlap(outs[i], act, ins[j], in_bytes[j])) return fail(WANATTN_E_INVALID, "an output overlaps an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], act, outs[j], act)) return fail(WANATTN_E_INVALID, "q, k and v overlap");
  }
  if (!workspace) return fail(WANATTN_E_INVALID, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(WANATTN_E_INVALID, "workspace must be 256-byte aligned");
  const size_t need = prologue_y_bytes(rows, dim) + kGemmWorkspace;
  if (workspace_bytes < need)
    return fail(WANATTN_E_INVALID, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  for (int j = 0; j < 11; ++j)
    if (overlap(workspace, need, ins[j], in_bytes[j])) return fail(WANATTN_E_INVALID, "workspace overlaps a tensor");
  for (int i = 0; i < 3; ++i)
    if (overlap(workspace, need, outs[i], act)) return fail(WANATTN_E_INVALID, "workspace overlaps a tensor");
  if (rms) {
    const size_t rbytes = (size_t)rows * 2 * sizeof(float);
    for (int j = 0; j < 11; ++j)
      if (overlap(rms, rbytes, ins[j], in_bytes[j])) return fail(WANATTN_E_INVALID, "rms overlaps an input");
    for (int i = 0; i < 3; ++i)
      if (overlap(rms, rbytes, outs[i], act)) return fail(WANATTN_E_INVALID, "rms overlaps an output");
    if (overlap(rms, rbytes, workspace, need)) return fail(WANATTN_E_INVALID, "rms overlaps the workspace");
  }

  ProjDesc pd;
  WA_TRY(pd.init(dim, rows));
  hipblasLtHandle_t h = nullptr;
  GemmPlan plan;
  WA_TRY(gemm_plan(pd, dim, rows, &h, &plan));
  const hipStream_t st = (hipStream_t)stream;
  uint16_t* y = (uint16_t*)workspace;
  void* gemm_ws = (char*)workspace + prologue_y_bytes(rows, dim);

  LnModParams lp;
  lp.x = (const uint16_t*)x;
  lp.e0 = e0;
  lp.e1 = e1;
  lp.y = y;
  lp.rows = rows;
  lp.N = N;
  lp.dim = dim;
  lp.eps = eps_ln;
  hipError_t le = launch_rows<LnModLaunch>(dim, dim3((unsigned)((rows + 3) / 4)), st, lp);
  if (le != hipSuccess) return fail(WANATTN_E_HIP, "ln_mod launch: %s", hipGetErrorString(le));

  const float one = 1.0f, zero = 0.0f;
  const void* w[3] = {wq, wk, wv};
  const void* bias[3] = {bq, bk, bv};
  for (int i = 0; i < 3; ++i) {
    WA_TRY(pd.set_bias(bias[i]));
    LT_TRY(hipblasLtMatmul(h, pd.op, &one, w[i], pd.a, y, pd.b, &zero, outs[i], pd.d, outs[i], pd.d, &plan.algo,
                           gemm_ws, plan.ws, st),
           "projection GEMM");
  }

  if (rms) {
    RmsStatParams sp;
    sp.q = (const uint16_t*)q;
    sp.k = (const uint16_t*)k;
    sp.rms = rms;
    sp.rows = rows;
    sp.dim = dim;
    sp.eps = eps_rms;
    le = launch_rows<QkRmsStatLaunch>(dim, dim3((unsigned)((2 * rows + 3) / 4)), st, sp);
    if (le != hipSuccess) return fail(WANATTN_E_HIP, "qk_rms_stats launch: %s", hipGetErrorString(le));
    return WANATTN_OK;
  }
  RmsParams rp;
  rp.q = (uint16_t*)q;
  rp.k = (uint16_t*)k;
  rp.gq = (const uint16_t*)gq;
  rp.gk = (const uint16_t*)gk;
  rp.rows = rows;
  rp.dim = dim;
  rp.eps = eps_rms;
  le = launch_rows<QkRmsLaunch>(dim, dim3((unsigned)((2 * rows + 3) / 4)), st, rp);
  if (le != hipSuccess) return fail(WANATTN_E_HIP, "qk_rmsnorm launch: %s", hipGetErrorString(le));
  return WANATTN_OK;
}

}  // namespace

extern "C" {

const char* wanattn_status_string(wanattn_status s) {
  switch (s) {
    case WANATTN_OK: return "ok";
    case WANATTN_E_INVALID: return "invalid argument";
    case WANATTN_E_UNSUPPORTED: return "unsupported";
    case WANATTN_E_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* wanattn_last_error(void) { return t_err; }

int32_t wanattn_version(void) { return WANATTN_VERSION; }

wanattn_status wanattn_prepare(double theta) {
  t_err[0] = 0;
  WA_TRY(check_theta(theta));
  const float2* tab = nullptr;
  WA_TRY(table_for(theta, nullptr, &tab));
  const hipError_t e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return fail(WANATTN_E_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  return WANATTN_OK;
}

wanattn_status wanattn_rope3d(const void* x, void* y, int32_t B, int32_t N, int32_t heads,
                              int32_t head_dim, const wanattn_grid3d* grid, double theta,
                              void* stream) {
  return rope3d_checked(x, y, B, N, heads, head_dim, grid, theta, (hipStream_t)stream);
}

size_t wanattn_self_workspace_bytes(int32_t B, int32_t N, int32_t heads, int32_t head_dim) {
  if (B < 1 || N < 1 || heads < 1 || head_dim != kHeadDim) return 0;
  return (size_t)B * N * heads * kHeadDim * 2 + split_items(B, N, heads) * kSplitItemBytes + kQueueBytes;
}

wanattn_status wanattn_self(const void* q, const void* k, const void* v, void* o, int32_t B,
                            int32_t N, int32_t heads, int32_t head_dim,
                            const wanattn_grid3d* grid, double theta, float scale,
                            wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                            void* workspace, size_t workspace_bytes, void* stream) {
  t_err[0] = 0;
  WA_TRY(check_theta(theta));
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  const size_t items = split_items(B, N, heads), full = bytes + items * kSplitItemBytes + kQueueBytes;
  const bool room = workspace_bytes >= full;
  WA_TRY(check_self(q, k, v, o, B, N, heads, head_dim, grid, scale, mask, chunk_frames, kv_lens, workspace,
                    workspace_bytes, bytes, room ? full : bytes));
  const float2* tab = nullptr;
  WA_TRY(table_for(theta, (hipStream_t)stream, &tab));
  return self_launch(q, k, v, o, B, N, heads, grid, scale, mask, chunk_frames, kv_lens, workspace, tab, 0,
                     room ? (char*)workspace + bytes : nullptr, room ? items : 0, (hipStream_t)stream);
}

wanattn_status wanattn_self_noalloc(const void* q, const void* k, const void* v, void* o, int32_t B,
                                    int32_t N, int32_t heads, int32_t head_dim,
                                    const wanattn_grid3d* grid, double theta, float scale,
                                    wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                                    void* stream) {
  t_err[0] = 0;
  WA_TRY(check_theta(theta));
  WA_TRY(check_self_args(q, k, v, o, B, N, heads, head_dim, grid, scale, mask, chunk_frames, kv_lens));
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  const size_t cap = WANATTN_NOALLOC_SCRATCH_BYTES;
  if (bytes + kQueueBytes > cap)
    return fail(WANATTN_E_UNSUPPORTED, "B*N*heads = %lld token rows need %zu bytes of scratch; the library holds %zu",
                (long long)B * N * heads, bytes + kQueueBytes, cap);
  // (the scratch is an array of its own: it cannot overlap a caller's tensor)
  unsigned char* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState* d = nullptr;
    WA_TRY(device_state(&d));
    ptr = d->scratch;
  }
  // the scratch takes the workspace's place: rotated keys, then the split's
  // partials where they fit, then the queue counters (zeroed by a kernel on
  // every call); with no room for the partials the queue follows the keys
  const size_t items = split_items(B, N, heads), full = bytes + items * kSplitItemBytes + kQueueBytes;
  const size_t room_items = full <= cap ? items : 0;
  const float2* tab = nullptr;
  WA_TRY(table_for(theta, (hipStream_t)stream, &tab));
  return self_launch(q, k, v, o, B, N, heads, grid, scale, mask, chunk_frames, kv_lens, ptr, tab, 0, ptr + bytes,
                     room_items, (hipStream_t)stream);
}

size_t wanattn_self_jitter_workspace_bytes(int32_t B, int32_t N, int32_t heads, int32_t head_dim) {
  if (B < 1 || N < 1 || heads < 1 || heads > kMaxJitterHeads || head_dim != kHeadDim) return 0;
  return jitter_table_bytes(heads) + (size_t)B * N * heads * kHeadDim * 2 + split_items(B, N, heads) * kSplitItemBytes +
         kQueueBytes;
}

wanattn_status wanattn_self_jitter(const void* q, const void* k, const void* v, void* o, int32_t B,
                                   int32_t N, int32_t heads, int32_t head_dim,
                                   const wanattn_grid3d* grid, const double* theta_per_head, float scale,
                                   wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  t_err[0] = 0;
  WA_TRY(check_tensor_sizes(B, N, heads, head_dim));
  WA_TRY(check_head_thetas(theta_per_head, heads));
  const size_t tbytes = jitter_table_bytes(heads);
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  const size_t items = split_items(B, N, heads), full = tbytes + bytes + items * kSplitItemBytes + kQueueBytes;
  const bool room = workspace_bytes >= full;
  WA_TRY(check_self(q, k, v, o, B, N, heads, head_dim, grid, scale, mask, chunk_frames, kv_lens, workspace,
                    workspace_bytes, tbytes + bytes, room ? full : tbytes + bytes));
  WA_TRY(build_head_tables(theta_per_head, heads, (float2*)workspace, (hipStream_t)stream));
  return self_launch(q, k, v, o, B, N, heads, grid, scale, mask, chunk_frames, kv_lens,
                     (char*)workspace + tbytes, (const float2*)workspace, kTabEntries,
                     room ? (char*)workspace + tbytes + bytes : nullptr, room ? items : 0, (hipStream_t)stream);
}

wanattn_status wanattn_self_kv(const void* q, const void* k_cache, const void* v_cache, void* o,
                               int32_t B, int32_t Nq, int32_t Nkv, int32_t heads, int32_t head_dim,
                               const wanattn_grid3d* grid_q, double theta, float scale,
                               const int32_t* kv_lens, void* stream) {
  t_err[0] = 0;
  WA_TRY(check_kv(q, k_cache, v_cache, o, B, Nq, Nkv, heads, head_dim, grid_q, scale, kv_lens));
  WA_TRY(check_theta(theta));
  const float2* tab = nullptr;
  WA_TRY(table_for(theta, (hipStream_t)stream, &tab));
  return kv_launch(q, k_cache, v_cache, o, B, Nq, Nkv, heads, grid_q, tab, 0, scale, kv_lens,
                   (hipStream_t)stream);
}

size_t wanattn_rope_tables_bytes(int32_t heads) {
  if (heads < 1 || heads > kMaxJitterHeads) return 0;
  return jitter_table_bytes(heads);
}

wanattn_status wanattn_rope_tables(const double* theta_per_head, int32_t heads, void* tables,
                                   size_t tables_bytes, void* stream) {
  t_err[0] = 0;
  WA_TRY(check_head_thetas(theta_per_head, heads));
  WA_TRY(check_tables(tables, tables_bytes, heads));
  return build_head_tables(theta_per_head, heads, (float2*)tables, (hipStream_t)stream);
}

wanattn_status wanattn_rope3d_tables(const void* x, void* y, int32_t B, int32_t N, int32_t heads,
                                     int32_t head_dim, const wanattn_grid3d* grid, const void* tables,
                                     size_t tables_bytes, void* stream) {
  t_err[0] = 0;
  if (!x || !y) return fail(WANATTN_E_INVALID, "null tensor pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  WA_TRY(check_tensor_sizes(B, N, heads, head_dim));
  WA_TRY(check_grid(grid, N));
  WA_TRY(check_tables(tables, tables_bytes, heads));
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2, tbytes = jitter_table_bytes(heads);
  if (x != y && overlap(x, bytes, y, bytes)) return fail(WANATTN_E_INVALID, "y partially overlaps x");
  if (overlap(tables, tbytes, y, bytes)) return fail(WANATTN_E_INVALID, "y overlaps the tables");
  return rope3d_launch(x, y, B, N, heads, grid, (const float2*)tables, kTabEntries, (hipStream_t)stream);
}

wanattn_status wanattn_self_kv_tables(const void* q, const void* k_cache, const void* v_cache, void* o,
                                      int32_t B, int32_t Nq, int32_t Nkv, int32_t heads, int32_t head_dim,
                                      const wanattn_grid3d* grid_q, const void* tables, size_t tables_bytes,
                                      float scale, const int32_t* kv_lens, void* stream) {
  t_err[0] = 0;
  WA_TRY(check_kv(q, k_cache, v_cache, o, B, Nq, Nkv, heads, head_dim, grid_q, scale, kv_lens));
  WA_TRY(check_tables(tables, tables_bytes, heads));
  const size_t qbytes = (size_t)B * Nq * heads * kHeadDim * 2;
  if (overlap(o, qbytes, tables, jitter_table_bytes(heads))) return fail(WANATTN_E_INVALID, "o overlaps the tables");
  return kv_launch(q, k_cache, v_cache, o, B, Nq, Nkv, heads, grid_q, (const float2*)tables, kTabEntries, scale,
                   kv_lens, (hipStream_t)stream);
}

wanattn_status wanattn_cross(const void* q, const void* k_ctx, const void* v_ctx, void* o,
                             int32_t B, int32_t N, int32_t M, int32_t heads, int32_t head_dim,
                             float scale, const int32_t* ctx_lens, void* stream) {
  t_err[0] = 0;
  if (!q || !k_ctx || !v_ctx || !o) return fail(WANATTN_E_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k_ctx) || !aligned16(v_ctx) || !aligned16(o))
    return fail(WANATTN_E_INVALID, "tensors must be 16-byte aligned");
  WA_TRY(check_tensor_sizes(B, N, heads, head_dim));
  WA_TRY(check_launch_size(B, N, heads));
  if (M < 1) return fail(WANATTN_E_INVALID, "M must be >= 1");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(WANATTN_E_INVALID, "scale must be finite and > 0");
  const size_t qbytes = (size_t)B * N * heads * kHeadDim * 2, cbytes = (size_t)B * M * heads * kHeadDim * 2;
  if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k_ctx, cbytes) || overlap(o, qbytes, v_ctx, cbytes))
    return fail(WANATTN_E_INVALID, "o overlaps an input");
  WA_TRY(check_lens(B, ctx_lens, M, "ctx_lens"));
  AttnParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_ctx;
  p.v = (const uint16_t*)v_ctx;
  p.o = (uint16_t*)o;
  p.tab = nullptr;
  p.N = N;
  p.Nk = M;
  p.heads = heads;
  p.qscale = scale * 1.4426950408889634f;
  p.H = 1;
  p.W = 1;
  p.inv_hw = 1.0;
  p.inv_w = 1.0;
  return launch_attn<false, false>(p, B, ctx_lens, (hipStream_t)stream);
}

size_t wanattn_prologue_workspace_bytes(int32_t B, int32_t N, int32_t dim) {
  if (B < 1 || N < 1 || dim < 8 || dim > kMaxRowDim || dim % 8 != 0) return 0;
  if ((long long)B * N > kMaxPrologueRows) return 0;
  return prologue_y_bytes((long long)B * N, dim) + kGemmWorkspace;
}

wanattn_status wanattn_prologue(const void* x, const float* e0, const float* e1, const void* wq,
                                const void* bq, const void* wk, const void* bk, const void* wv,
                                const void* bv, const void* gq, const void* gk, void* q, void* k,
                                void* v, int32_t B, int32_t N, int32_t dim, float eps_ln,
                                float eps_rms, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return prologue_core(x, e0, e1, wq, bq, wk, bk, wv, bv, gq, gk, q, k, v, nullptr, B, N, dim, eps_ln, eps_rms,
                       workspace, workspace_bytes, stream);
}

wanattn_status wanattn_prologue_rms(const void* x, const float* e0, const float* e1, const void* wq,
                                    const void* bq, const void* wk, const void* bk, const void* wv,
                                    const void* bv, void* q, void* k, void* v, float* rms, int32_t B,
                                    int32_t N, int32_t dim, float eps_ln, float eps_rms, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!rms) {
    t_err[0] = 0;
    return fail(WANATTN_E_INVALID, "rms is NULL");
  }
  return prologue_core(x, e0, e1, wq, bq, wk, bk, wv, bv, nullptr, nullptr, q, k, v, rms, B, N, dim, eps_ln,
                       eps_rms, workspace, workspace_bytes, stream);
}

wanattn_status wanattn_self_qknorm(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t N,
                                   int32_t heads, int32_t head_dim, const wanattn_grid3d* grid, double theta,
                                   float scale, wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                                   const float* rms, const void* gq, const void* gk, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  t_err[0] = 0;
  WA_TRY(check_theta(theta));
  WA_TRY(check_self_args(q, k, v, o, B, N, heads, head_dim, grid, scale, mask, chunk_frames, kv_lens));
  if (!rms || !gq || !gk) return fail(WANATTN_E_INVALID, "rms, gq and gk must be given");
  if (((uintptr_t)rms & 3u) != 0 || !aligned16(gq) || !aligned16(gk))
    return fail(WANATTN_E_INVALID, "rms must be 4-byte and gq, gk 16-byte aligned");
  const size_t bytes = (size_t)B * N * heads * kHeadDim * 2;
  const size_t rbytes = (size_t)B * N * 2 * sizeof(float), gbytes = (size_t)heads * kHeadDim * 2;
  if (overlap(o, bytes, rms, rbytes) || overlap(o, bytes, gq, gbytes) || overlap(o, bytes, gk, gbytes))
    return fail(WANATTN_E_INVALID, "o overlaps rms or a gamma");
  const size_t items = split_items(B, N, heads), full = bytes + items * kSplitItemBytes + kQueueBytes;
  const bool room = workspace_bytes >= full;
  WA_TRY(check_self(q, k, v, o, B, N, heads, head_dim, grid, scale, mask, chunk_frames, kv_lens, workspace,
                    workspace_bytes, bytes, room ? full : bytes));
  const size_t ws_use = room ? full : bytes;
  if (overlap(workspace, ws_use, rms, rbytes) || overlap(workspace, ws_use, gq, gbytes) ||
      overlap(workspace, ws_use, gk, gbytes))
    return fail(WANATTN_E_INVALID, "workspace overlaps rms or a gamma");
  const float2* tab = nullptr;
  WA_TRY(table_for(theta, (hipStream_t)stream, &tab));
  return self_launch(q, k, v, o, B, N, heads, grid, scale, mask, chunk_frames, kv_lens, workspace, tab, 0,
                     room ? (char*)workspace + bytes : nullptr, room ? items : 0, (hipStream_t)stream, rms, gq, gk);
}

}  // extern "C"
