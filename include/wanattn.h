/*
 * wanattn -- 3D-RoPE self attention and text cross attention of the Wan2.1/2.2
 * video diffusion transformer, as hand-written HIP kernels for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * Pages that define the operations (titles as published):
 *  [P1] "動画生成の勘定を明らかにする：Wan2.2 ソースコード精読" (blog.leeguoo.com)
 *       ch. 4 "DiT: 75600 token の attention" -- full 3D joint attention over all
 *       latent-frame tokens; subsection "3D RoPE" -- head dim 128 split 44/42/42
 *       over time/height/width, applied to q and k as complex multiplication;
 *       the block forward calls self_attn(x, seq_lens, grid_sizes, freqs) and
 *       cross_attn(x, context, context_lens).
 *       ch. 8 "75600² とは何か" -- the Q K^T and A V products, 4 L^2 dim FLOPs.
 *  [P2] "論文解説: Wan - 大規模オープンソース動画生成モデルのアーキテクチャと訓練"
 *       (0h-n0.github.io), section on the text encoder -- cross attention
 *       softmax(Q K_text^T / sqrt(d_k)) V_text.
 *  [P3] long-video survey (atlascloud.ai), "ルート3 · Self Forcing" --
 *       bidirectional attention replaced by causal attention over chunks;
 *       "ルート2 · LoL" -- multi-head RoPE jitter against sink collapse.
 *
 * Common conventions
 *  - Tensors are caller-owned DEVICE memory on the device that owns `stream`,
 *    bf16 bit patterns (uint16_t), contiguous [B, tokens, heads, head_dim]
 *    with head_dim fastest, and 16-byte aligned.  head_dim must be 128.
 *  - Tokens of an F x H x W latent grid are frame-major:
 *    n = (f * H + h) * W + w.  RoPE positions are (f + f0, h + h0, w + w0) and
 *    must stay below 1024 on every axis (the table length of [P1]'s
 *    rope_params(1024, .)).
 *  - Pair c of a head vector is (x[2c], x[2c+1]) = (real, imag); pairs 0..21
 *    rotate with the frame position, 22..42 with the row, 43..63 with the
 *    column; frequency k of an axis of width D is theta^(-2k/D).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work and return; success means "enqueued".  Nothing synchronises the
 *    host with the device (wanattn_prepare and the prologue's first call on a
 *    device aside).  The rotary table of a theta ([P1] builds `freqs` once,
 *    at construction) is built on the device, in fp64 rounded to fp32, by the
 *    first call that uses that theta on a device, on that call's stream;
 *    calls on other streams wait for it through an event, and a call under
 *    HIP stream capture puts its own build of the table into the graph.
 *  - Errors: arguments are checked before anything is launched.
 *    WANATTN_E_INVALID: null or misaligned pointer, sizes < 1, N != F*H*W,
 *    positions reaching 1024, an output overlapping an input, bad lengths.
 *    WANATTN_E_UNSUPPORTED: head_dim != 128, heads > WANATTN_MAX_HEADS, more
 *    distinct theta values than the library keeps tables for, an attention
 *    launch of more than 2^24 workgroups (min(B, 256) * heads * ceil(N / 256)).  WANATTN_E_HIP: a HIP call failed.
 *    wanattn_last_error() gives a thread-local text for the last failure.
 *  - Calls on different streams may run concurrently.
 */
#ifndef WANATTN_H
#define WANATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WANATTN_VERSION 1
#define WANATTN_HEAD_DIM 128
#define WANATTN_MAX_POS 1024
#define WANATTN_MAX_LEN_BATCH 256  /* batches per kernel launch (larger B: several launches) */
#define WANATTN_MAX_HEADS 65536

typedef enum wanattn_status {
  WANATTN_OK = 0,
  WANATTN_E_INVALID = 1,
  WANATTN_E_UNSUPPORTED = 2,
  WANATTN_E_HIP = 3
} wanattn_status;

/* token grid: N = F * H * W; (f0, h0, w0) are RoPE position offsets (>= 0) */
typedef struct wanattn_grid3d {
  int32_t F, H, W;
  int32_t f0, h0, w0;
} wanattn_grid3d;

typedef enum wanattn_mask {
  WANATTN_MASK_NONE = 0,         /* bidirectional, [P1] ch. 4 */
  WANATTN_MASK_BLOCK_CAUSAL = 1  /* latent-frame chunks, [P3] Self Forcing */
} wanattn_mask;

/*
 * [P1] ch. 4, 3D RoPE (rope_apply): y = x rotated by the 3D rotary embedding.
 * x, y: [B, N, heads, 128] bf16; y may equal x (in place) but must not
 * otherwise overlap it.  The rotation is done in fp32 from a table built in
 * fp64 (rounded to fp32), and rounded to bf16 (nearest even).
 */
wanattn_status wanattn_rope3d(const void* x, void* y, int32_t B, int32_t N, int32_t heads,
                              int32_t head_dim, const wanattn_grid3d* grid, double theta,
                              void* stream);

/*
 * [P1] ch. 4 and ch. 8: o = softmax(q' k'^T * scale + mask) v, per batch and
 * head, where q' and k' are q and k rotated by the 3D RoPE of their tokens.
 * q, k, v, o: [B, N, heads, 128] bf16; o must not overlap q, k or v.
 * scale: usually 1/sqrt(128).
 * mask: WANATTN_MASK_NONE (every query sees every key), or
 *   WANATTN_MASK_BLOCK_CAUSAL ([P3] Self Forcing): with C = chunk_frames
 *   latent frames per chunk counted from frame 0 of the grid, query i sees key
 *   j iff floor(f_j / C) <= floor(f_i / C).  chunk_frames is read only in
 *   that mode and must be >= 1.
 * kv_lens: HOST array [B] or NULL (= N): keys j >= kv_lens[b] are excluded
 *   ([P1] ch. 4 seq_lens; ch. 8 pads the sequence to a multiple of the
 *   sequence-parallel size), 1 <= kv_lens[b] <= N.  Every query row is still
 *   written.
 * workspace: caller-owned device memory, 16-byte aligned, not overlapping q,
 *   k, v or o, of at least B*N*heads*head_dim*2 bytes: it receives the
 *   rotated keys k' (one rotation per key, shared by every query tile).
 *   wanattn_self_workspace_bytes(B, N, heads, head_dim) adds room for fp32
 *   partial results (at most 512 * 130 KiB) and 256 bytes of work-queue
 *   counters.  With it, a launch that covers the chip at least once runs one
 *   workgroup per compute unit, drawing query tiles from one queue per XCD
 *   (its own first, then the others'), and under the bidirectional mask the
 *   last query tiles run as several work items each over ranges of the keys,
 *   whose partial softmax results a second kernel combines.  A smaller
 *   workspace runs one workgroup per query tile, without the split.  The
 *   contents after the call are unspecified.  Calls that may run
 *   concurrently need separate workspaces.
 * Accumulation is fp32; the MFMA operands (rotated and scaled q, rotated k,
 * softmax probabilities, v) are bf16; o is rounded to bf16 (nearest even).
 * Rows of split tiles are combined in a different order, so they can differ
 * from an unsplit run in the last bit; which tiles split depends on the
 * device's compute-unit count.  Repeated calls on one device give identical
 * bits.
 */
wanattn_status wanattn_self(const void* q, const void* k, const void* v, void* o, int32_t B,
                            int32_t N, int32_t heads, int32_t head_dim,
                            const wanattn_grid3d* grid, double theta, float scale,
                            wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                            void* workspace, size_t workspace_bytes, void* stream);

/* bytes of workspace for wanattn_self with these sizes, the split's room
 * included (0 for invalid sizes) */
size_t wanattn_self_workspace_bytes(int32_t B, int32_t N, int32_t heads, int32_t head_dim);

/* Bytes of scratch memory the library holds on every device it runs on, for
 * wanattn_self_noalloc (512 MiB). */
#define WANATTN_NOALLOC_SCRATCH_BYTES ((size_t)512 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * wanattn_self without a workspace argument.  Its scratch memory (the rotated
 * keys, then the key-split partials where they fit, then the work-queue
 * counters) is a module-scope device array of WANATTN_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device until the process ends; the call
 * allocates nothing.  Arguments, errors and numerics as wanattn_self, plus:
 *  - WANATTN_E_UNSUPPORTED when the rotated keys and the queue counters,
 *    B * N * heads * head_dim * 2 + 256 bytes, exceed the scratch (e.g.
 *    32,760 tokens x 40 heads fit, 75,600 x 40 do not); larger calls need
 *    wanattn_self and a caller workspace;
 *  - where the split's partials also fit, the results are bitwise those of
 *    wanattn_self with a full workspace; otherwise those of a workspace
 *    without room for the split (persistent launch, no split);
 *  - every call on a device uses that device's one scratch array: calls that
 *    may overlap on one device (different streams, or captured graphs
 *    replayed concurrently) race and give wrong results.  Serialise them.
 *    The queue counters are cleared by a kernel on every call.
 * The first call on a device sets up the library's per-device state (array
 * addresses, events) and, as for every entry point, the first use of a theta
 * enqueues the build of its rotary table on `stream`.
 */
wanattn_status wanattn_self_noalloc(const void* q, const void* k, const void* v, void* o, int32_t B,
                                    int32_t N, int32_t heads, int32_t head_dim,
                                    const wanattn_grid3d* grid, double theta, float scale,
                                    wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                                    void* stream);

#define WANATTN_MAX_JITTER_HEADS 256

/*
 * [P3] "ルート2 · LoL" multi-head RoPE jitter: wanattn_self where head h
 * rotates q and k with its own base theta_per_head[h].  [P3] describes the
 * jitter only as a random per-head perturbation of the RoPE phase, applied
 * without training; a phase offset that does not grow with position cancels
 * in q.k, so the perturbation is taken on the base (the caller draws the
 * values, e.g. theta * (1 + eps_h)).  Equal values reproduce wanattn_self.
 * theta_per_head: HOST array [heads], each finite and > 0; heads <=
 *   WANATTN_MAX_JITTER_HEADS (else WANATTN_E_UNSUPPORTED).
 * workspace: 16-byte aligned, not overlapping q, k, v or o, of at least
 *   heads * 768 KiB + B*N*heads*head_dim*2 bytes.  It receives the per-head
 *   rotary tables (built on the device in fp64 and rounded to fp32 on every
 *   call, 768 KiB per head) followed by the rotated keys;
 *   wanattn_self_jitter_workspace_bytes(...) adds the room for the tail
 *   split's partials as in wanattn_self.  Everything else, including errors
 *   and numerics, is as wanattn_self.
 */
wanattn_status wanattn_self_jitter(const void* q, const void* k, const void* v, void* o, int32_t B,
                                   int32_t N, int32_t heads, int32_t head_dim,
                                   const wanattn_grid3d* grid, const double* theta_per_head, float scale,
                                   wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* bytes of workspace for wanattn_self_jitter, the split's room included (0
 * for invalid sizes) */
size_t wanattn_self_jitter_workspace_bytes(int32_t B, int32_t N, int32_t heads, int32_t head_dim);

/*
 * [P3] Self Forcing, streamed: one chunk of queries against a key/value cache
 * of the chunks before it and itself ([P1] ch. 4 "3D RoPE" for positions).
 * q, o: [B, Nq, heads, 128] with Nq = grid_q->F * H * W; grid_q's offsets are
 *   the chunk's RoPE positions (f0 = the chunk's first latent frame).
 * k_cache: [B, Nkv, heads, 128], keys ALREADY rotated by their own positions
 *   (wanattn_rope3d with the cache's grid and offsets, once per appended
 *   chunk); v_cache: [B, Nkv, heads, 128].  Nkv must be whole frames of
 *   H x W tokens.  Every key j < kv_lens[b] is visible.
 * kv_lens: HOST array [B] or NULL (= Nkv), 1 <= kv_lens[b] <= Nkv.
 * o must not overlap the inputs.  No workspace; numerics as wanattn_self.
 */
wanattn_status wanattn_self_kv(const void* q, const void* k_cache, const void* v_cache, void* o,
                               int32_t B, int32_t Nq, int32_t Nkv, int32_t heads, int32_t head_dim,
                               const wanattn_grid3d* grid_q, double theta, float scale,
                               const int32_t* kv_lens, void* stream);

/*
 * [P3] "ルート2 · LoL" multi-head RoPE jitter in the streamed setting
 * ("ルート3 · Self Forcing"): per-head rotary tables, head h with its own
 * base theta_per_head[h] (the reading of wanattn_self_jitter), built once by
 * the caller and used by the two streaming calls below.
 *
 * wanattn_rope_tables: builds the tables of `heads` heads into `tables`
 *   (caller-owned device memory, 16-byte aligned, at least
 *   wanattn_rope_tables_bytes(heads) bytes = 768 KiB per head), in fp64 on the
 *   device, rounded to fp32; enqueued on `stream`.  theta_per_head: HOST
 *   array [heads], each finite and > 0; heads <= WANATTN_MAX_JITTER_HEADS.
 * wanattn_rope3d_tables: wanattn_rope3d with head h rotated by table h
 *   (e.g. a new chunk's keys appended to a jittered cache).
 * wanattn_self_kv_tables: wanattn_self_kv whose queries are rotated by the
 *   per-head tables; the cache keys must have been rotated with the same
 *   tables (wanattn_rope3d_tables).
 * `tables` must hold tables built for at least `heads` heads (only their
 * size can be checked) and must not overlap an output.  Errors and numerics
 * otherwise as wanattn_rope3d / wanattn_self_kv.
 */
size_t wanattn_rope_tables_bytes(int32_t heads);
wanattn_status wanattn_rope_tables(const double* theta_per_head, int32_t heads, void* tables,
                                   size_t tables_bytes, void* stream);
wanattn_status wanattn_rope3d_tables(const void* x, void* y, int32_t B, int32_t N, int32_t heads,
                                     int32_t head_dim, const wanattn_grid3d* grid, const void* tables,
                                     size_t tables_bytes, void* stream);
wanattn_status wanattn_self_kv_tables(const void* q, const void* k_cache, const void* v_cache, void* o,
                                      int32_t B, int32_t Nq, int32_t Nkv, int32_t heads, int32_t head_dim,
                                      const wanattn_grid3d* grid_q, const void* tables, size_t tables_bytes,
                                      float scale, const int32_t* kv_lens, void* stream);

/*
 * [P2] cross attention, called as cross_attn(x, context, context_lens) in
 * [P1] ch. 4: o = softmax(q k_ctx^T * scale) v_ctx, no rotary embedding.
 * q, o: [B, N, heads, 128]; k_ctx, v_ctx: [B, M, heads, 128] (M text tokens,
 * 512 after the text projection in [P1] ch. 4).  ctx_lens: HOST array [B] or
 * NULL (= M), 1 <= ctx_lens[b] <= M; text keys j >= ctx_lens[b] are excluded.
 * o must not overlap the inputs.
 */
wanattn_status wanattn_cross(const void* q, const void* k_ctx, const void* v_ctx, void* o,
                             int32_t B, int32_t N, int32_t M, int32_t heads, int32_t head_dim,
                             float scale, const int32_t* ctx_lens, void* stream);

/*
 * [P1] ch. 4, the block forward up to self_attn, and "3D RoPE" (QK-Norm):
 *   y = LayerNorm(x) * (1 + e1[b]) + e0[b]      (LayerNorm without affine
 *       parameters over dim: mean, mean squared deviation, eps_ln in the root)
 *   q = RMSNorm(y Wq^T + bq) * gq,  k = RMSNorm(y Wk^T + bk) * gk,
 *   v = y Wv^T + bv                 (RMSNorm over the whole dim, eps_rms)
 * x: [B, N, dim] bf16.  e0, e1: [B, dim] fp32 (the shift and scale of the
 * block's time modulation).  wq, wk, wv: [dim, dim] bf16, row o holding output
 * o's weights over the input columns (the nn.Linear layout).  bq, bk, bv, gq,
 * gk: [dim] bf16.  q, k, v: [B, N, dim] bf16, i.e. [B, N, heads, 128] when
 * dim = heads * 128, not yet rotated: they are wanattn_self's inputs.
 * dim: a multiple of 8 in [8, 8192].  eps_ln, eps_rms: finite, >= 0 (the
 * model uses 1e-6 for both).
 * Numerics: LayerNorm statistics and modulation in fp32, y rounded to bf16;
 * the projections are bf16 GEMMs with fp32 accumulation (hipBLASLt, bias added
 * in fp32 in the epilogue), rounded to bf16; RMSNorm in fp32 on those values,
 * rounded to bf16.  Pointers 16-byte aligned; q, k, v must not overlap each
 * other or any input.
 * workspace: caller-owned device memory of at least
 *   wanattn_prologue_workspace_bytes(B, N, dim) bytes, 256-byte aligned, not
 *   overlapping any tensor; it holds y and the GEMM library's workspace.
 *   Contents after the call are unspecified; concurrent calls need separate
 *   workspaces.
 * The first call on a device creates that device's hipBLASLt handle (which
 * may allocate device memory and synchronise), and the first call for each
 * new (dim, B * N) runs the library's algorithm query; later calls only enqueue.
 */
wanattn_status wanattn_prologue(const void* x, const float* e0, const float* e1, const void* wq,
                                const void* bq, const void* wk, const void* bk, const void* wv,
                                const void* bv, const void* gq, const void* gk, void* q, void* k,
                                void* v, int32_t B, int32_t N, int32_t dim, float eps_ln,
                                float eps_rms, void* workspace, size_t workspace_bytes,
                                void* stream);

/* bytes of workspace wanattn_prologue needs for these sizes (0 for invalid sizes) */
size_t wanattn_prologue_workspace_bytes(int32_t B, int32_t N, int32_t dim);

/*
 * [P1] ch. 4, the same prologue with the QK-Norm left to the attention call
 * that reads q and k ("3D RoPE": q and k are RMS-normalised, then rotated):
 * q and k are written as projected (before the RMSNorm), v as in
 * wanattn_prologue, and
 *   rms[t] = 1 / sqrt(mean(q[t]^2) + eps_rms),  rms[B*N + t] = the same for k
 * for every token row t (fp32, caller-owned device memory of 2*B*N floats,
 * 16-byte aligned, not overlapping any tensor or the workspace).
 * wanattn_self_qknorm then applies q * rms * gq and k * rms * gk where it
 * loads the queries and where it rotates the keys, so that q and k are not
 * written twice.  Arguments otherwise as wanattn_prologue (gq, gk are given
 * to wanattn_self_qknorm instead); the workspace is
 * wanattn_prologue_workspace_bytes(B, N, dim).
 */
wanattn_status wanattn_prologue_rms(const void* x, const float* e0, const float* e1, const void* wq,
                                    const void* bq, const void* wk, const void* bk, const void* wv,
                                    const void* bv, void* q, void* k, void* v, float* rms, int32_t B,
                                    int32_t N, int32_t dim, float eps_ln, float eps_rms, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * wanattn_self on the outputs of wanattn_prologue_rms: q and k are the
 * projections before the QK-Norm ([B, N, heads, 128] bf16), rms its factors
 * (q's B*N, then k's B*N, fp32, 4-byte aligned), gq and gk its weights
 * ([heads * 128] bf16, 16-byte aligned).  Each query element is taken as
 * q * rms * gq as it is loaded, each key element as k * rms * gk as the key
 * is rotated into the workspace, in fp32, before the rotation; the rest,
 * including the workspace (wanattn_self_workspace_bytes), errors and
 * numerics, is as wanattn_self.
 */
wanattn_status wanattn_self_qknorm(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t N,
                                   int32_t heads, int32_t head_dim, const wanattn_grid3d* grid, double theta,
                                   float scale, wanattn_mask mask, int32_t chunk_frames, const int32_t* kv_lens,
                                   const float* rms, const void* gq, const void* gk, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Build the rotary table for theta on the current device now and wait for it
 * (a blocking call on the null stream).  Optional: the first call that uses
 * theta builds it otherwise.  Up to 8 distinct theta values are kept per
 * device.
 */
wanattn_status wanattn_prepare(double theta);

const char* wanattn_status_string(wanattn_status s);
const char* wanattn_last_error(void);
int32_t wanattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WANATTN_H */
