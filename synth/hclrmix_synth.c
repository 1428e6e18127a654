/*
 * Seeded synthetic input generator for the HyperConnectionLowRankMix block.
 *
 * This file produces input bytes only. It holds none of the block's
 * arithmetic, and both the GPU tests and the CPU oracle consume the same
 * buffers it writes.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-based: the
 * value for counter c under seed s is mix64(s + c * 0x9E3779B97F4A7C15), so
 * any element can be produced independently and threads split the index
 * range without changing a single output.
 *
 * Uniform doubles: u = ((x >> 11) + 0.5) * 2^-53, which lies in (0, 1).
 * Normals: Box-Muller, cosine branch, from the uniforms at counters 2i+1 and
 * 2i+2 for element i, computed in double and cast to float.
 */
#include <math.h>
#include <stdint.h>
#include <pthread.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double sm_uniform(uint64_t seed, uint64_t counter) {
  uint64_t x = sm_mix(seed + counter * SM_GAMMA);
  return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

typedef struct {
  float* out;
  int64_t begin, end;
  uint64_t seed;
  double a, b;
  int kind; /* 0 normal(mean a, std b), 1 uniform(a, b) */
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t i = j->begin; i < j->end; ++i) {
    if (j->kind == 0) {
      double u1 = sm_uniform(j->seed, 2 * (uint64_t)i + 1);
      double u2 = sm_uniform(j->seed, 2 * (uint64_t)i + 2);
      double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
      j->out[i] = (float)(j->a + j->b * z);
    } else {
      double u = sm_uniform(j->seed, (uint64_t)i + 1);
      j->out[i] = (float)(j->a + (j->b - j->a) * u);
    }
  }
  return 0;
}

static void fill(float* out, int64_t n, uint64_t seed, double a, double b, int kind, int threads) {
  if (n <= 0) return;
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if (n < 65536) threads = 1;
  job_t jobs[64];
  pthread_t tid[64];
  int joined[64] = {0};
  int64_t per = (n + threads - 1) / threads;
  int used = 0;
  for (int t = 0; t < threads; ++t) {
    int64_t lo = (int64_t)t * per, hi = lo + per;
    if (lo >= n) break;
    if (hi > n) hi = n;
    jobs[t].out = out; jobs[t].begin = lo; jobs[t].end = hi; jobs[t].seed = seed;
    jobs[t].a = a; jobs[t].b = b; jobs[t].kind = kind;
    used = t + 1;
    if (t == 0) continue;
    if (pthread_create(&tid[t], 0, run_job, &jobs[t]) == 0) joined[t] = 1;
    else run_job(&jobs[t]);
  }
  run_job(&jobs[0]);
  for (int t = 1; t < used; ++t) if (joined[t]) pthread_join(tid[t], 0);
}

/* out[i] ~ N(mean, std^2), i in [0, n). */
void hcs_fill_normal(float* out, int64_t n, uint64_t seed, double mean, double std, int threads) {
  fill(out, n, seed, mean, std, 0, threads);
}

/* out[i] ~ U(lo, hi), i in [0, n). */
void hcs_fill_uniform(float* out, int64_t n, uint64_t seed, double lo, double hi, int threads) {
  fill(out, n, seed, lo, hi, 1, threads);
}

/* Raw SplitMix64 output for counter c (used by tests against published values). */
uint64_t hcs_splitmix64(uint64_t seed, uint64_t counter) { return sm_mix(seed + counter * SM_GAMMA); }
