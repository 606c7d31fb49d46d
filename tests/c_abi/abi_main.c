/*
 * The C ABI used from plain C (no Python, no torch): device buffers from the
 * HIP runtime, the library's entry points, and the fp64 oracle (test
 * infrastructure, linked here only as the checker) on the same seeded inputs.
 *
 * Cases: bidirectional self attention with 3D RoPE (Wan2.2 source reading
 * (blog.leeguoo.com), ch. 4 "3D RoPE"); block-causal with per-batch kv_lens
 * (long-video survey (atlascloud.ai), "ルート3 · Self Forcing"); cross
 * attention with ctx_lens (Wan paper explainer (0h-n0.github.io), text-encoder
 * section); one chunk against a rotated key/value cache; an argument error.
 * Gates: max |err| <= 2e-2, mean |err| <= 2e-3, rms(err)/rms(ref) <= 1e-2.
 * Exit status 0 when every case passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wanattn.h"

/* seeded inputs (video_diffusion_transformer_wanattn_amd/seeded/seeded.c) */
int seeded_normal_bf16(uint16_t* out, float* out_f32, uint64_t n, uint64_t seed, uint64_t stream, double sigma,
                       int nthreads);
/* the oracle (oracle/wanattn_oracle.c) */
int orc_self_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int N, int heads, int head_dim,
                  int F, int H, int W, int f0, int h0, int w0, double theta, double scale, int mask,
                  int chunk_frames, const int* kv_lens, int nrows, const int* rows, double* out, int nthreads);
int orc_cross_rows(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int B, int N, int M, int heads,
                   int head_dim, double scale, const int* ctx_lens, int nrows, const int* rows, double* out,
                   int nthreads);
int orc_kv_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int Nq, int Nkv, int heads,
                int head_dim, int Fq, int H, int W, int qf0, int kf0, int h0, int w0, double theta, double scale,
                const int* kv_lens, int nrows, const int* rows, double* out, int nthreads);

#define HEADS 2
#define D 128
#define THETA 10000.0

static int failures = 0;

#define HIP_CHECK(x)                                                                  \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(2);                                                                        \
    }                                                                                 \
  } while (0)

static double widen(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static uint16_t* gen(size_t n, uint64_t stream, double sigma) {
  uint16_t* h = (uint16_t*)malloc(n * sizeof(uint16_t));
  if (!h || seeded_normal_bf16(h, NULL, n, 11, stream, sigma, 4) != 0) {
    fprintf(stderr, "input generation failed\n");
    exit(2);
  }
  return h;
}

static void* to_dev(const uint16_t* h, size_t n) {
  void* d = NULL;
  HIP_CHECK(hipMalloc(&d, n * sizeof(uint16_t)));
  HIP_CHECK(hipMemcpy(d, h, n * sizeof(uint16_t), hipMemcpyHostToDevice));
  return d;
}

static void compare(const char* what, const void* dev_out, const double* ref, size_t n) {
  uint16_t* got = (uint16_t*)malloc(n * sizeof(uint16_t));
  HIP_CHECK(hipMemcpy(got, dev_out, n * sizeof(uint16_t), hipMemcpyDeviceToHost));
  double max_abs = 0.0, sum_abs = 0.0, sum_d2 = 0.0, sum_r2 = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double d = widen(got[i]) - ref[i];
    if (!isfinite(d)) max_abs = INFINITY;
    if (fabs(d) > max_abs) max_abs = fabs(d);
    sum_abs += fabs(d);
    sum_d2 += d * d;
    sum_r2 += ref[i] * ref[i];
  }
  const double mean_abs = sum_abs / (double)n, rel = sqrt(sum_d2 / (sum_r2 > 0 ? sum_r2 : 1e-300));
  const int ok = max_abs <= 2e-2 && mean_abs <= 2e-3 && rel <= 1e-2;
  printf("%-34s max %.3e mean %.3e rel_rms %.3e %s\n", what, max_abs, mean_abs, rel, ok ? "ok" : "FAIL");
  if (!ok) ++failures;
  free(got);
}

static void status(const char* what, wanattn_status s) {
  if (s != WANATTN_OK) {
    printf("%s: %s (%s)\n", what, wanattn_status_string(s), wanattn_last_error());
    exit(1);
  }
}

int main(void) {
  const int F = 3, H = 5, W = 7, N = F * H * W, B = 2, M = 33;
  const size_t n = (size_t)B * N * HEADS * D, nc = (size_t)B * M * HEADS * D;
  const float scale = (float)(1.0 / sqrt((double)D));
  int rows[F * H * W];
  for (int i = 0; i < N; ++i) rows[i] = i;
  uint16_t *q = gen(n, 1, 1.0), *k = gen(n, 2, 1.0), *v = gen(n, 3, 0.5);
  uint16_t *kc = gen(nc, 4, 0.5), *vc = gen(nc, 5, 0.5);
  void *dq = to_dev(q, n), *dk = to_dev(k, n), *dv = to_dev(v, n), *dkc = to_dev(kc, nc), *dvc = to_dev(vc, nc);
  void *dout = NULL, *ws = NULL;
  HIP_CHECK(hipMalloc(&dout, n * sizeof(uint16_t)));
  const size_t ws_bytes = wanattn_self_workspace_bytes(B, N, HEADS, D);
  HIP_CHECK(hipMalloc(&ws, ws_bytes));
  hipStream_t st;
  HIP_CHECK(hipStreamCreate(&st));
  double* ref = (double*)malloc(n * sizeof(double));
  const wanattn_grid3d grid = {F, H, W, 0, 0, 0};

  /* bidirectional self attention */
  status("wanattn_self", wanattn_self(dq, dk, dv, dout, B, N, HEADS, D, &grid, THETA, scale, WANATTN_MASK_NONE, 1,
                                      NULL, ws, ws_bytes, st));
  HIP_CHECK(hipStreamSynchronize(st));
  if (orc_self_rows(q, k, v, B, N, HEADS, D, F, H, W, 0, 0, 0, THETA, scale, 0, 1, NULL, N, rows, ref, 4)) return 2;
  compare("self, bidirectional", dout, ref, n);

  /* block-causal (chunks of 1 frame) with per-batch key lengths */
  const int lens[2] = {N, 61};
  status("wanattn_self causal", wanattn_self(dq, dk, dv, dout, B, N, HEADS, D, &grid, THETA, scale,
                                             WANATTN_MASK_BLOCK_CAUSAL, 1, lens, ws, ws_bytes, st));
  HIP_CHECK(hipStreamSynchronize(st));
  if (orc_self_rows(q, k, v, B, N, HEADS, D, F, H, W, 0, 0, 0, THETA, scale, 1, 1, lens, N, rows, ref, 4)) return 2;
  compare("self, block-causal + kv_lens", dout, ref, n);

  /* cross attention with per-batch text lengths */
  const int clens[2] = {M, 9};
  status("wanattn_cross", wanattn_cross(dq, dkc, dvc, dout, B, N, M, HEADS, D, scale, clens, st));
  HIP_CHECK(hipStreamSynchronize(st));
  if (orc_cross_rows(q, kc, vc, B, N, M, HEADS, D, scale, clens, N, rows, ref, 4)) return 2;
  compare("cross + ctx_lens", dout, ref, n);

  /* the last frame as a chunk against the cache of all three frames */
  const int HW = H * W;
  const size_t nq = (size_t)B * HW * HEADS * D;
  uint16_t* qc = (uint16_t*)malloc(nq * sizeof(uint16_t));
  for (int b = 0; b < B; ++b)
    memcpy(qc + (size_t)b * HW * HEADS * D, q + ((size_t)b * N + 2 * HW) * HEADS * D,
           (size_t)HW * HEADS * D * sizeof(uint16_t));
  void* dqc = to_dev(qc, nq);
  void* dcache = NULL;
  HIP_CHECK(hipMalloc(&dcache, n * sizeof(uint16_t)));
  status("wanattn_rope3d", wanattn_rope3d(dk, dcache, B, N, HEADS, D, &grid, THETA, st));
  const wanattn_grid3d gq = {1, H, W, 2, 0, 0};
  status("wanattn_self_kv", wanattn_self_kv(dqc, dcache, dv, dout, B, HW, N, HEADS, D, &gq, THETA, scale, NULL, st));
  HIP_CHECK(hipStreamSynchronize(st));
  if (orc_kv_rows(qc, k, v, B, HW, N, HEADS, D, 1, H, W, 2, 0, 0, 0, THETA, scale, NULL, HW, rows, ref, 4)) return 2;
  compare("kv-cache chunk", dout, ref, nq);

  /* an argument error is reported before anything is launched */
  const wanattn_grid3d bad = {F, H, W + 1, 0, 0, 0};
  const wanattn_status s = wanattn_self(dq, dk, dv, dout, B, N, HEADS, D, &bad, THETA, scale, WANATTN_MASK_NONE, 1,
                                        NULL, ws, ws_bytes, st);
  const int err_ok = s == WANATTN_E_INVALID && strlen(wanattn_last_error()) > 0;
  printf("%-34s %s: %s\n", "N != F*H*W rejected", err_ok ? "ok" : "FAIL", wanattn_last_error());
  if (!err_ok) ++failures;

  HIP_CHECK(hipStreamDestroy(st));
  hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dkc), hipFree(dvc), hipFree(dout), hipFree(ws);
  hipFree(dqc), hipFree(dcache);
  free(q), free(k), free(v), free(kc), free(vc), free(qc), free(ref);
  printf("%s (library version %d)\n", failures ? "FAILED" : "all cases passed", wanattn_version());
  return failures ? 1 : 0;
}
