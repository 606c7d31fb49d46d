/*
 * ORACLE -- test infrastructure only.
 *
 * A plain, slow fp64 CPU statement of what the Wan 3D-RoPE attention path
 * computes.  Only tests/, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the product path never does.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Sources (the pages these functions follow):
 *  [P1] "動画生成の勘定を明らかにする：Wan2.2 ソースコード精読" (blog.leeguoo.com),
 *       ch. 4 "DiT: 75600 token の attention":
 *         - subsection "latent から token へ": patch size (1,2,2); tokens of all
 *           latent frames form one 1-D sequence.
 *         - subsection "3D RoPE": head dim d = 128 split into rope_params(1024, 44),
 *           rope_params(1024, 42), rope_params(1024, 42) for time, height and
 *           width; each token takes the rows of its (f, h, w) coordinates,
 *           concatenates them and multiplies q and k as complex numbers, in
 *           float64; q.k then depends only on coordinate differences.
 *       ch. 8 "75600² とは何か": the core is the two products Q K^T and A V.
 *  [P2] "論文解説: Wan - 大規模オープンソース動画生成モデルのアーキテクチャと訓練"
 *       (0h-n0.github.io), "テキストエンコーダ（Qwen統合）": cross attention is
 *       softmax(Q K_text^T / sqrt(d_k)) V_text.
 *  [P3] long-video survey (atlascloud.ai), "ルート3 · Self Forcing": the
 *       bidirectional full attention is replaced by causal attention over
 *       chunks, earlier chunks acting as a KV cache; "ルート2 · LoL": a random
 *       per-head perturbation of the RoPE phase (multi-head RoPE jitter),
 *       applied without training.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - rope_params(L, D) builds, for positions p < L, the angles p * w_k with
 *    w_k = theta^(-2k/D), k < D/2 (standard RoPE per segment; theta is a
 *    parameter, 10000 in the workloads).
 *  - the complex pairs are adjacent elements (2c, 2c+1) = (real, imag).
 *  - token n of an F x H x W grid sits at f = n / (H W), h = (n / W) mod H,
 *    w = n mod W (frame-major); RoPE positions are (f + f0, h + h0, w + w0).
 *  - block-causal: key j is visible to query i iff floor(f_j / C) <=
 *    floor(f_i / C), C = chunk_frames latent frames per chunk, counted from
 *    frame 0 of the grid.
 *  - kv_len: keys j >= kv_len are excluded (all query rows still computed).
 *  - multi-head RoPE jitter: a phase offset that does not depend on position
 *    cancels in q.k (both sides turn by it), so the perturbation is taken to
 *    act on the phase rate: head h rotates with its own base theta_h (drawn
 *    by the caller, e.g. theta * (1 + eps_h)), every other step unchanged.
 *  - KV-cache streaming: a chunk of queries (first frame f0) attends to every
 *    cached key, earlier chunks and its own; the cache holds whole frames whose
 *    positions are their own frame indices (first frame kv_frame0), so a
 *    rolling window only moves positions.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* exact widening of a bf16 bit pattern */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* [P1] ch. 4, 3D RoPE: d - 4*(d//6) for time, 2*(d//6) for height and width. */
void orc_axis_dims(int head_dim, int dims[3]) {
  int s = head_dim / 6;
  dims[0] = head_dim - 4 * s;
  dims[1] = 2 * s;
  dims[2] = 2 * s;
}

/* frequency k of a segment of width D: theta^(-2k/D) (reading of rope_params) */
double orc_omega(double theta, int D, int k) { return pow(theta, -2.0 * (double)k / (double)D); }

/* [P1] ch. 4: position of token n in the frame-major (f, h, w) sequence */
void orc_decode(int n, int H, int W, int pos[3]) {
  pos[0] = n / (H * W);
  pos[1] = (n / W) % H;
  pos[2] = n % W;
}

/*
 * [P1] ch. 4, 3D RoPE: rotate one head vector x (length head_dim, fp64) of a
 * token at RoPE positions (pf, ph, pw) into y.  Pair c of the head is
 * (x[2c], x[2c+1]); the first dims[0]/2 pairs take the time angle, the next
 * dims[1]/2 the height angle, the last dims[2]/2 the width angle; the pair is
 * multiplied by e^{i * pos * w_k} as a complex number.
 */
void orc_rope_vec(const double* x, double* y, int head_dim, int pf, int ph, int pw, double theta) {
  int dims[3];
  orc_axis_dims(head_dim, dims);
  int pos[3] = {pf, ph, pw};
  int c = 0;
  for (int a = 0; a < 3; ++a) {
    for (int k = 0; k < dims[a] / 2; ++k, ++c) {
      double ang = (double)pos[a] * orc_omega(theta, dims[a], k);
      double cr = cos(ang), ci = sin(ang);
      double re = x[2 * c], im = x[2 * c + 1];
      y[2 * c] = re * cr - im * ci;
      y[2 * c + 1] = re * ci + im * cr;
    }
  }
}

/*
 * Whole-tensor RoPE: x is bf16 bits [B, N, heads, head_dim] for an F x H x W
 * grid with position offsets (f0, h0, w0); y receives fp64 values, same layout.
 */
void orc_rope3d(const uint16_t* x, double* y, int B, int N, int heads, int head_dim, int F, int H,
                int W, int f0, int h0, int w0, double theta) {
  (void)F;
  double* xin = (double*)malloc(sizeof(double) * (size_t)head_dim);
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n) {
      int pos[3];
      orc_decode(n, H, W, pos);
      for (int hd = 0; hd < heads; ++hd) {
        size_t off = (((size_t)b * N + n) * heads + hd) * head_dim;
        for (int e = 0; e < head_dim; ++e) xin[e] = bf16_value(x[off + e]);
        orc_rope_vec(xin, y + off, head_dim, pos[0] + f0, pos[1] + h0, pos[2] + w0, theta);
      }
    }
  free(xin);
}

/* [P3] Route 3: visibility of key j from query i under the block-causal mask */
static int visible(int i, int j, int HW, int mask, int chunk_frames) {
  if (!mask) return 1;
  int fi = i / HW, fj = j / HW;
  return (fj / chunk_frames) <= (fi / chunk_frames);
}

/*
 * softmax attention of one query row (fp64), two passes over the visible keys:
 * s_j = (q . k_j) * scale;  p_j = exp(s_j - max s) / sum exp(s - max s);
 * o = sum_j p_j v_j.   [P2] formula; [P1] ch. 8 (Q K^T then A V).
 */
static void attend_row(const double* qrow, const double* kmat, const double* vmat, int nkeys,
                       const unsigned char* allowed, int head_dim, double scale, double* srow,
                       double* out) {
  double m = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    if (!allowed[j]) continue;
    double s = 0.0;
    for (int e = 0; e < head_dim; ++e) s += qrow[e] * kmat[(size_t)j * head_dim + e];
    s *= scale;
    srow[j] = s;
    if (s > m) m = s;
  }
  double den = 0.0;
  for (int j = 0; j < nkeys; ++j)
    if (allowed[j]) {
      srow[j] = exp(srow[j] - m);
      den += srow[j];
    }
  for (int e = 0; e < head_dim; ++e) out[e] = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    if (!allowed[j]) continue;
    double p = srow[j] / den;
    for (int e = 0; e < head_dim; ++e) out[e] += p * vmat[(size_t)j * head_dim + e];
  }
}

typedef struct {
  /* shared */
  const uint16_t *q, *k, *v;
  int B, N, M, heads, head_dim;
  int H, W, f0, h0, w0;    /* grid and position offsets of the queries */
  int kf0, kh0, kw0;       /* position offsets of the keys (same grid H x W) */
  double theta, scale;
  const double* head_theta; /* [heads] per-head RoPE base, or NULL (= theta) */
  int rope, mask, chunk_frames;
  const int* kv_lens;
  int nrows;
  const int* rows;
  double* out;
  /* work split: (b, head) pairs [begin, end) */
  int begin, end;
  int status;
} task_t;

static void* run_task(void* arg) {
  task_t* t = (task_t*)arg;
  const int d = t->head_dim;
  const int nk = t->M; /* number of keys */
  double* kmat = (double*)malloc(sizeof(double) * (size_t)nk * d);
  double* vmat = (double*)malloc(sizeof(double) * (size_t)nk * d);
  double* qrow = (double*)malloc(sizeof(double) * d);
  double* qtmp = (double*)malloc(sizeof(double) * d);
  double* srow = (double*)malloc(sizeof(double) * (size_t)nk);
  unsigned char* allowed = (unsigned char*)malloc((size_t)nk);
  if (!kmat || !vmat || !qrow || !qtmp || !srow || !allowed) {
    t->status = 1;
    goto done;
  }
  for (int bh = t->begin; bh < t->end; ++bh) {
    int b = bh / t->heads, hd = bh % t->heads;
    int kvl = t->kv_lens ? t->kv_lens[b] : nk;
    const double th = t->head_theta ? t->head_theta[hd] : t->theta;
    /* keys and values of this (b, head), keys rotated when self attention */
    for (int j = 0; j < nk; ++j) {
      size_t off = (((size_t)b * nk + j) * t->heads + hd) * d;
      for (int e = 0; e < d; ++e) {
        qtmp[e] = bf16_value(t->k[off + e]);
        vmat[(size_t)j * d + e] = bf16_value(t->v[off + e]);
      }
      if (t->rope) {
        int pos[3];
        orc_decode(j, t->H, t->W, pos);
        orc_rope_vec(qtmp, kmat + (size_t)j * d, d, pos[0] + t->kf0, pos[1] + t->kh0, pos[2] + t->kw0, th);
      } else {
        memcpy(kmat + (size_t)j * d, qtmp, sizeof(double) * d);
      }
    }
    for (int r = 0; r < t->nrows; ++r) {
      int i = t->rows[r];
      size_t qoff = (((size_t)b * t->N + i) * t->heads + hd) * d;
      for (int e = 0; e < d; ++e) qtmp[e] = bf16_value(t->q[qoff + e]);
      if (t->rope) {
        int pos[3];
        orc_decode(i, t->H, t->W, pos);
        orc_rope_vec(qtmp, qrow, d, pos[0] + t->f0, pos[1] + t->h0, pos[2] + t->w0, th);
      } else {
        memcpy(qrow, qtmp, sizeof(double) * d);
      }
      for (int j = 0; j < nk; ++j)
        allowed[j] = (j < kvl) && visible(i, j, t->H * t->W, t->mask, t->chunk_frames);
      double* o = t->out + (((size_t)b * t->nrows + r) * t->heads + hd) * d;
      attend_row(qrow, kmat, vmat, nk, allowed, d, t->scale, srow, o);
    }
  }
done:
  free(kmat);
  free(vmat);
  free(qrow);
  free(qtmp);
  free(srow);
  free(allowed);
  return 0;
}

static int run_threads(task_t* proto, int nthreads) {
  int total = proto->B * proto->heads;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > total) nthreads = total;
  if (nthreads > 256) nthreads = 256;
  task_t* tasks = (task_t*)calloc((size_t)nthreads, sizeof(task_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  int* started = (int*)calloc((size_t)nthreads, sizeof(int));
  if (!tasks || !th || !started) {
    free(tasks);
    free(th);
    free(started);
    return 1;
  }
  for (int t = 0; t < nthreads; ++t) {
    tasks[t] = *proto;
    tasks[t].begin = (int)((long)total * t / nthreads);
    tasks[t].end = (int)((long)total * (t + 1) / nthreads);
    tasks[t].status = 0;
  }
  for (int t = 1; t < nthreads; ++t) started[t] = pthread_create(&th[t], 0, run_task, &tasks[t]) == 0;
  run_task(&tasks[0]);
  int status = tasks[0].status;
  for (int t = 1; t < nthreads; ++t) {
    if (started[t])
      pthread_join(th[t], 0);
    else
      run_task(&tasks[t]);
    status |= tasks[t].status;
  }
  free(tasks);
  free(th);
  free(started);
  return status;
}

/*
 * Self attention with 3D RoPE on the selected query rows.
 * q, k, v: bf16 bits [B, N, heads, head_dim], N = F*H*W.
 * rows[nrows]: query rows to compute (the same rows for every batch and head).
 * out: fp64 [B, nrows, heads, head_dim].
 * mask: 0 bidirectional, 1 block-causal with chunk_frames latent frames per chunk.
 * kv_lens: [B] or NULL (= N).  Returns 0 on success, 1 on bad arguments or
 * allocation failure.
 */
int orc_self_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int N, int heads,
                  int head_dim, int F, int H, int W, int f0, int h0, int w0, double theta,
                  double scale, int mask, int chunk_frames, const int* kv_lens, int nrows,
                  const int* rows, double* out, int nthreads) {
  if (B < 1 || N < 1 || heads < 1 || head_dim < 2 || (head_dim % 2) || N != F * H * W) return 1;
  if (mask && chunk_frames < 1) return 1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return 1;
  if (kv_lens)
    for (int b = 0; b < B; ++b)
      if (kv_lens[b] < 1 || kv_lens[b] > N) return 1;
  task_t t;
  memset(&t, 0, sizeof t);
  t.q = q;
  t.k = k;
  t.v = v;
  t.B = B;
  t.N = N;
  t.M = N;
  t.heads = heads;
  t.head_dim = head_dim;
  t.H = H;
  t.W = W;
  t.f0 = f0;
  t.h0 = h0;
  t.w0 = w0;
  t.kf0 = f0;
  t.kh0 = h0;
  t.kw0 = w0;
  t.theta = theta;
  t.scale = scale;
  t.rope = 1;
  t.mask = mask;
  t.chunk_frames = chunk_frames;
  t.kv_lens = kv_lens;
  t.nrows = nrows;
  t.rows = rows;
  t.out = out;
  return run_threads(&t, nthreads);
}

/*
 * Self attention with multi-head RoPE jitter ([P3] "ルート2 · LoL"): as
 * orc_self_rows, except that head h rotates q and k with its own base
 * theta_heads[h] (each finite and > 0).
 */
int orc_self_rows_heads(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int N, int heads,
                        int head_dim, int F, int H, int W, int f0, int h0, int w0,
                        const double* theta_heads, double scale, int mask, int chunk_frames,
                        const int* kv_lens, int nrows, const int* rows, double* out, int nthreads) {
  if (!theta_heads || heads < 1) return 1;
  for (int h = 0; h < heads; ++h)
    if (!(theta_heads[h] > 0.0) || !isfinite(theta_heads[h])) return 1;
  if (B < 1 || N < 1 || head_dim < 2 || (head_dim % 2) || N != F * H * W) return 1;
  if (mask && chunk_frames < 1) return 1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return 1;
  if (kv_lens)
    for (int b = 0; b < B; ++b)
      if (kv_lens[b] < 1 || kv_lens[b] > N) return 1;
  task_t t;
  memset(&t, 0, sizeof t);
  t.q = q;
  t.k = k;
  t.v = v;
  t.B = B;
  t.N = N;
  t.M = N;
  t.heads = heads;
  t.head_dim = head_dim;
  t.H = H;
  t.W = W;
  t.f0 = f0;
  t.h0 = h0;
  t.w0 = w0;
  t.kf0 = f0;
  t.kh0 = h0;
  t.kw0 = w0;
  t.head_theta = theta_heads;
  t.scale = scale;
  t.rope = 1;
  t.mask = mask;
  t.chunk_frames = chunk_frames;
  t.kv_lens = kv_lens;
  t.nrows = nrows;
  t.rows = rows;
  t.out = out;
  return run_threads(&t, nthreads);
}

/*
 * Attention of one chunk of queries to a key/value cache ([P3] "ルート3 · Self
 * Forcing": a new chunk attends to the chunks generated before it and to
 * itself; [P1] ch. 4 "3D RoPE" for the positions).  Queries q [B, Nq, heads,
 * head_dim] form a frame-major Fq x H x W grid whose positions are shifted by
 * (qf0, h0, w0); keys and values [B, Nkv, heads, head_dim] are Nkv / (H W)
 * whole frames at positions shifted by (kf0, h0, w0).  Both are rotated here
 * from the raw inputs; every key j < kv_lens[b] is visible.
 * out: fp64 [B, nrows, heads, head_dim].
 */
static int kv_rows_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int Nq, int Nkv,
                        int heads, int head_dim, int Fq, int H, int W, int qf0, int kf0, int h0, int w0,
                        double theta, const double* head_thetas, double scale, const int* kv_lens,
                        int nrows, const int* rows, double* out, int nthreads) {
  if (B < 1 || Nq < 1 || Nkv < 1 || heads < 1 || head_dim < 2 || (head_dim % 2)) return 1;
  if (H < 1 || W < 1 || Nq != Fq * H * W || Nkv % (H * W)) return 1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= Nq) return 1;
  if (kv_lens)
    for (int b = 0; b < B; ++b)
      if (kv_lens[b] < 1 || kv_lens[b] > Nkv) return 1;
  task_t t;
  memset(&t, 0, sizeof t);
  t.q = q;
  t.k = k;
  t.v = v;
  t.B = B;
  t.N = Nq;
  t.M = Nkv;
  t.heads = heads;
  t.head_dim = head_dim;
  t.H = H;
  t.W = W;
  t.f0 = qf0;
  t.h0 = h0;
  t.w0 = w0;
  t.kf0 = kf0;
  t.kh0 = h0;
  t.kw0 = w0;
  t.theta = theta;
  t.head_theta = head_thetas;
  t.scale = scale;
  t.rope = 1;
  t.mask = 0;
  t.chunk_frames = 1;
  t.kv_lens = kv_lens;
  t.nrows = nrows;
  t.rows = rows;
  t.out = out;
  return run_threads(&t, nthreads);
}

int orc_kv_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int Nq, int Nkv,
                int heads, int head_dim, int Fq, int H, int W, int qf0, int kf0, int h0, int w0,
                double theta, double scale, const int* kv_lens, int nrows, const int* rows,
                double* out, int nthreads) {
  return kv_rows_impl(q, k, v, B, Nq, Nkv, heads, head_dim, Fq, H, W, qf0, kf0, h0, w0, theta, 0, scale,
                      kv_lens, nrows, rows, out, nthreads);
}

/*
 * orc_kv_rows with multi-head RoPE jitter ([P3] "ルート2 · LoL", applied to
 * the streamed, autoregressive setting it targets): head h rotates its
 * queries and cached keys with its own base theta_heads[h] (finite, > 0).
 */
int orc_kv_rows_heads(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int Nq, int Nkv,
                      int heads, int head_dim, int Fq, int H, int W, int qf0, int kf0, int h0, int w0,
                      const double* theta_heads, double scale, const int* kv_lens, int nrows,
                      const int* rows, double* out, int nthreads) {
  if (!theta_heads || heads < 1) return 1;
  for (int h = 0; h < heads; ++h)
    if (!(theta_heads[h] > 0.0) || !isfinite(theta_heads[h])) return 1;
  return kv_rows_impl(q, k, v, B, Nq, Nkv, heads, head_dim, Fq, H, W, qf0, kf0, h0, w0, 0.0, theta_heads,
                      scale, kv_lens, nrows, rows, out, nthreads);
}

/*
 * Cross attention ([P2] formula): queries q [B, N, heads, head_dim], text keys
 * and values [B, M, heads, head_dim], no rotary embedding, keys j >= ctx_len
 * excluded.  out: fp64 [B, nrows, heads, head_dim].
 */
int orc_cross_rows(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int B, int N, int M,
                   int heads, int head_dim, double scale, const int* ctx_lens, int nrows,
                   const int* rows, double* out, int nthreads) {
  if (B < 1 || N < 1 || M < 1 || heads < 1 || head_dim < 1) return 1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return 1;
  if (ctx_lens)
    for (int b = 0; b < B; ++b)
      if (ctx_lens[b] < 1 || ctx_lens[b] > M) return 1;
  task_t t;
  memset(&t, 0, sizeof t);
  t.q = q;
  t.k = kc;
  t.v = vc;
  t.B = B;
  t.N = N;
  t.M = M;
  t.heads = heads;
  t.head_dim = head_dim;
  t.H = 1;
  t.W = 1;
  t.scale = scale;
  t.rope = 0;
  t.mask = 0;
  t.chunk_frames = 1;
  t.kv_lens = ctx_lens;
  t.nrows = nrows;
  t.rows = rows;
  t.out = out;
  return run_threads(&t, nthreads);
}

/*
 * The self-attention prologue of one block ([P1] ch. 4, "1つの block の完全な
 * forward" and "3D RoPE"): the input of self_attn is norm1(x) * (1 + e1) + e0
 * with the modulation in fp32; inside it q, k, v are linear projections of
 * that input, and q and k each pass an RMSNorm (QK-Norm) before RoPE.
 * Readings (the pages do not print these layers): norm1 is a LayerNorm over
 * dim without affine parameters, eps_ln inside the square root; the RMSNorm
 * runs over the whole projection width dim with a learned weight (gamma),
 * eps_rms inside the square root; projections are y W^T + b with W [dim, dim]
 * (out, in) and b [dim].
 * x: bf16 [B, N, dim]; e0, e1: fp32 [B, dim]; wq, wk, wv: bf16 [dim, dim];
 * bq, bk, bv, gq, gk: bf16 [dim].  Outputs fp64 [B, nrows, dim] for the rows
 * requested (q and k RMS-normalised, v as projected), before any rotation.
 */
static void linear_row(const double* y, const uint16_t* w, const uint16_t* b, int dim, double* out) {
  for (int o = 0; o < dim; ++o) {
    double acc = bf16_value(b[o]);
    const uint16_t* wr = w + (size_t)o * dim;
    for (int i = 0; i < dim; ++i) acc += y[i] * bf16_value(wr[i]);
    out[o] = acc;
  }
}

static void rms_norm_row(double* x, const uint16_t* g, int dim, double eps) {
  double ss = 0.0;
  for (int i = 0; i < dim; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / sqrt(ss / dim + eps);
  for (int i = 0; i < dim; ++i) x[i] = x[i] * inv * bf16_value(g[i]);
}

typedef struct {
  const uint16_t *x, *wq, *wk, *wv, *bq, *bk, *bv, *gq, *gk;
  const float *e0, *e1;
  int B, N, dim, nrows;
  const int* rows;
  double eps_ln, eps_rms;
  double *oq, *ok, *ov;
  int begin, end; /* flat (b, row) range */
  int status;
} pro_task_t;

static void* run_pro_task(void* arg) {
  pro_task_t* t = (pro_task_t*)arg;
  const int dim = t->dim;
  double* y = (double*)malloc(sizeof(double) * dim);
  if (!y) {
    t->status = 1;
    return 0;
  }
  for (int br = t->begin; br < t->end; ++br) {
    const int b = br / t->nrows, r = br % t->nrows;
    const uint16_t* xr = t->x + ((size_t)b * t->N + t->rows[r]) * dim;
    double mean = 0.0, var = 0.0;
    for (int i = 0; i < dim; ++i) mean += bf16_value(xr[i]);
    mean /= dim;
    for (int i = 0; i < dim; ++i) {
      const double d = bf16_value(xr[i]) - mean;
      var += d * d;
    }
    var /= dim;
    const double inv = 1.0 / sqrt(var + t->eps_ln);
    for (int i = 0; i < dim; ++i)
      y[i] = (bf16_value(xr[i]) - mean) * inv * (1.0 + (double)t->e1[(size_t)b * dim + i]) +
             (double)t->e0[(size_t)b * dim + i];
    const size_t off = ((size_t)b * t->nrows + r) * dim;
    linear_row(y, t->wq, t->bq, dim, t->oq + off);
    linear_row(y, t->wk, t->bk, dim, t->ok + off);
    linear_row(y, t->wv, t->bv, dim, t->ov + off);
    rms_norm_row(t->oq + off, t->gq, dim, t->eps_rms);
    rms_norm_row(t->ok + off, t->gk, dim, t->eps_rms);
  }
  free(y);
  return 0;
}

int orc_prologue_rows(const uint16_t* x, const float* e0, const float* e1, const uint16_t* wq,
                      const uint16_t* bq, const uint16_t* wk, const uint16_t* bk, const uint16_t* wv,
                      const uint16_t* bv, const uint16_t* gq, const uint16_t* gk, int B, int N, int dim,
                      double eps_ln, double eps_rms, int nrows, const int* rows, double* oq, double* ok,
                      double* ov, int nthreads) {
  if (B < 1 || N < 1 || dim < 1 || nrows < 1 || !(eps_ln >= 0.0) || !(eps_rms >= 0.0)) return 1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return 1;
  const int total = B * nrows;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > total) nthreads = total;
  if (nthreads > 256) nthreads = 256;
  pro_task_t* tasks = (pro_task_t*)calloc((size_t)nthreads, sizeof(pro_task_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  int* started = (int*)calloc((size_t)nthreads, sizeof(int));
  if (!tasks || !th || !started) {
    free(tasks);
    free(th);
    free(started);
    return 1;
  }
  for (int k = 0; k < nthreads; ++k) {
    pro_task_t* t = &tasks[k];
    t->x = x; t->wq = wq; t->wk = wk; t->wv = wv; t->bq = bq; t->bk = bk; t->bv = bv;
    t->gq = gq; t->gk = gk; t->e0 = e0; t->e1 = e1;
    t->B = B; t->N = N; t->dim = dim; t->nrows = nrows; t->rows = rows;
    t->eps_ln = eps_ln; t->eps_rms = eps_rms; t->oq = oq; t->ok = ok; t->ov = ov;
    t->begin = (int)((long)total * k / nthreads);
    t->end = (int)((long)total * (k + 1) / nthreads);
  }
  for (int k = 1; k < nthreads; ++k) started[k] = pthread_create(&th[k], 0, run_pro_task, &tasks[k]) == 0;
  run_pro_task(&tasks[0]);
  int status = tasks[0].status;
  for (int k = 1; k < nthreads; ++k) {
    if (started[k])
      pthread_join(th[k], 0);
    else
      run_pro_task(&tasks[k]);
    status |= tasks[k].status;
  }
  free(tasks);
  free(th);
  free(started);
  return status;
}

/*
 * [P1] ch. 2 "VAE" (vae_stride (4, 8, 8), the latent-shape expression and
 * "4n+1 の由来") and ch. 4 "latent から token へ" (patch (1, 2, 2)): a clip of
 * `frames` frames (4n+1) at height x width pixels becomes (frames-1)/4+1 latent frames of
 * (height/8) x (width/8) latents; patch size (1,2,2) then gives a token grid
 * of (frames-1)/4+1 x height/16 x width/16.
 */
void orc_token_grid(int frames, int height, int width, int grid[3]) {
  grid[0] = (frames - 1) / 4 + 1;
  grid[1] = (height / 8) / 2;
  grid[2] = (width / 8) / 2;
}
