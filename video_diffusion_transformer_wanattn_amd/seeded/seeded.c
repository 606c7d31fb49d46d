/*
 * Seeded synthetic inputs shared by the oracle side and the HIP side.
 *
 * This file holds no attention or rotary arithmetic: it only turns
 * (seed, stream, element index) into bf16 bit patterns of N(0,1)*sigma
 * samples.  Both sides of every parity check read the same bits.
 *
 * Generator (counter based, so any element can be produced on its own):
 *   gamma = 0x9E3779B97F4A7C15
 *   key   = mix64(seed ^ (stream << 32))
 *   word_k = mix64(key + (k + 1) * gamma)                 (uint64, wraps)
 *   mix64(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *             z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
 *   (the SplitMix64 output function of Steele, Lea and Flood, 2014).
 *   u1 = ((word_k >> 32)        + 0.5) * 2^-32,  u2 = ((word_k & 0xffffffff) + 0.5) * 2^-32
 *   r = sqrt(-2 ln u1);  element 2k = r cos(2 pi u2) * sigma,  element 2k+1 = r sin(2 pi u2) * sigma
 *   (Box and Muller, 1958), evaluated in double, rounded to float (RNE),
 *   then to bfloat16 with round-to-nearest-even.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

/* float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN. */
uint16_t seeded_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

uint64_t seeded_word(uint64_t seed, uint64_t stream, uint64_t k) {
  uint64_t key = mix64(seed ^ (stream << 32));
  return mix64(key + (k + 1) * kGamma);
}

static void normal_pair(uint64_t w, double* z0, double* z1) {
  const double two_m32 = 2.3283064365386963e-10; /* 2^-32 */
  double u1 = ((double)(w >> 32) + 0.5) * two_m32;
  double u2 = ((double)(w & 0xffffffffull) + 0.5) * two_m32;
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586 * u2;
  *z0 = r * cos(a);
  *z1 = r * sin(a);
}

typedef struct {
  uint16_t* out;
  uint64_t begin, end; /* element range [begin, end) */
  uint64_t seed, stream;
  double sigma;
  float* out_f32; /* optional: the float value before bf16 rounding */
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  uint64_t key = mix64(j->seed ^ (j->stream << 32));
  uint64_t e = j->begin;
  while (e < j->end) {
    uint64_t k = e >> 1;
    double z[2];
    normal_pair(mix64(key + (k + 1) * kGamma), &z[0], &z[1]);
    for (int t = (int)(e & 1); t < 2 && e < j->end; ++t, ++e) {
      float f = (float)(z[t] * j->sigma);
      j->out[e] = seeded_f32_to_bf16(f);
      if (j->out_f32) j->out_f32[e] = f;
    }
  }
  return 0;
}

/*
 * Fill out[0..n) with the bf16 bits of elements [0, n) of stream `stream`.
 * out_f32 may be NULL; when given it receives the float values before the
 * bf16 rounding (for tests of the rounding step).  Returns 0 on success.
 */
int seeded_normal_bf16(uint16_t* out, float* out_f32, uint64_t n, uint64_t seed, uint64_t stream,
                       double sigma, int nthreads) {
  if (n == 0) return 0;
  if (!out) return 1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < (1u << 16)) nthreads = 1;
  pthread_t th[64];
  job_t jobs[64];
  /* split on even boundaries so that a Box-Muller pair never straddles threads */
  uint64_t pairs = (n + 1) / 2;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t pb = pairs * (uint64_t)t / (uint64_t)nthreads;
    uint64_t pe = pairs * (uint64_t)(t + 1) / (uint64_t)nthreads;
    jobs[t].out = out;
    jobs[t].out_f32 = out_f32;
    jobs[t].begin = 2 * pb;
    jobs[t].end = 2 * pe < n ? 2 * pe : n;
    jobs[t].seed = seed;
    jobs[t].stream = stream;
    jobs[t].sigma = sigma;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], 0, run_job, &jobs[t]) != 0) break;
    started = t;
  }
  run_job(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], 0);
  for (int t = started + 1; t < nthreads; ++t) run_job(&jobs[t]);
  return 0;
}
