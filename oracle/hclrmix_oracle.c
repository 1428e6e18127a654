/*
 * CPU oracle for the HyperConnectionLowRankMix block.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product path (the HIP library)
 * never calls it and shares no code with it.
 *
 * What it computes: the block defined in onnxruntime PR #33384
 * ("com.microsoft.HyperConnectionLowRankMix"), section "Schema summary":
 *
 *   S          = streams + prev_post_gate * prev_block_output   (optional prologue)
 *   hn         = S / sqrt(mean_h(S^2) + epsilon) * norm_scale   (per branch)
 *   d          = ScaledSiLU(hn @ down_weight, silu_alpha)
 *   g          = sigmoid(d @ up_weight)
 *   pre_output = reduction_scale * sum_c(hn * g)
 *   post_gate  = sigmoid((hn @ inject_weight) / gate_div) * gate_mul
 *
 * with the section "Numerics contract" of the same page: every matrix product
 * and reduction accumulates in fp32, and each step's result is rounded once to
 * the element type T at the points S, hn, down, Z, SG, hidden, up, g,
 * pre_output, inject and post_gate; the sigmoid is 1/(1+exp(-x)) in fp32 with
 * an accurate expf, rounded once. The oracle therefore is that composition,
 * one row at a time, every sum taken in ascending index order, built with
 * -ffp-contract=off so no multiply-add is fused.
 *
 * Readings where the pages leave a step open (each is listed with its reason
 * in the design notes of this repository):
 *  - ScaledSiLU(x, a) = x * sigmoid(a * x), evaluated as Z = a*x, SG =
 *    sigmoid(Z), hidden = x * SG. The pages give only the name and the rounding
 *    points Z, SG, hidden in that order; Z before SG makes Z the sigmoid's
 *    scaled argument. At a = 1 every candidate reading is SiLU. For a != 1
 *    the ScaledSiLU step is "parity unpinned" beyond this reading.
 *  - norm_scale has C*H entries (one per stream and feature); streams are
 *    flattened branch-major, k = c*H + h.
 *  - The prologue broadcasts S[c,h] = s[c,h] + q[c] * p[h].
 *  - RMS: fp32 sum of squares in ascending h, ss/H + eps, IEEE sqrtf and
 *    division, then * norm_scale, rounded once.
 *  - Gate and pre-mix: one rounding at each listed point, fp32 in between;
 *    pre_output = rT(rs * sum_c(hn*g)), post_gate = rT(sigmoid(inject/gd)*gm).
 *  - Rounding to T is round-to-nearest-even, NaN stays NaN, no flush to zero.
 *
 * Element types use the ONNX TensorProto codes: 1 float, 10 float16,
 * 16 bfloat16. 16-bit values travel as raw uint16 bit patterns.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_F32 1
#define ORA_F16 10
#define ORA_BF16 16

/* ------------------------------------------------------------------------ */
/* Element codecs, written from the IEEE 754 / bfloat16 format definitions. */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 is the top half of a binary32: widening appends 16 zero bits. */
static float bf16_widen(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float f16_widen(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);                    /* zero / subnormal */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);                /* (1.m) * 2^(e-15) */
  if (e == 31 && m) return bits_f32(sign ? 0xFFC00000u : 0x7FC00000u);
  return (float)(sign ? -v : v);
}

/* Round a binary32 value to bfloat16, nearest, ties to even. The two
 * candidates are the truncation t (toward zero) and its successor in
 * magnitude; the 16 discarded bits decide. */
static uint16_t bf16_round(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN: keep sign, quiet */
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t t = u >> 16, rem = u & 0xFFFFu;
  if (rem > 0x8000u || (rem == 0x8000u && (t & 1u))) t += 1; /* may carry into inf: correct */
  return (uint16_t)t;
}

/* Round a binary32 value to binary16, nearest, ties to even, computed on the
 * value: find the spacing q of binary16 numbers around |x|, round |x|/q to an
 * integer (ties to even), and re-encode. Overflow goes to infinity. */
static uint16_t f16_round(float f) {
  uint32_t u = f32_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if ((u & 0x7F800000u) == 0x7F800000u) {
    if (u & 0x007FFFFFu) return (uint16_t)(sign | 0x7E00u);  /* NaN */
    return (uint16_t)(sign | 0x7C00u);                      /* inf */
  }
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);                     /* a = fr * 2^e2, fr in [0.5, 1): binade [2^(e2-1), 2^e2) */
  int ulp_exp = (e2 - 1) - 10;       /* spacing of normal binary16 numbers in that binade */
  if (ulp_exp < -24) ulp_exp = -24;  /* subnormal spacing 2^-24 */
  double n = ldexp(a, -ulp_exp);     /* exact */
  double fl = floor(n), frac = n - fl;
  double r = fl;
  if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
  double v = ldexp(r, ulp_exp);
  if (v >= 65536.0) return (uint16_t)(sign | 0x7C00u);      /* above the largest finite 65504 */
  if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(v, 24));   /* subnormal */
  int ev;
  frexp(v, &ev);
  int E = ev - 1;                                           /* v in [2^E, 2^(E+1)) */
  uint16_t mant = (uint16_t)(ldexp(v, 10 - E) - 1024.0);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | mant);
}

/* f(x): widen a stored element to fp32 (exact). */
static float widen(int dt, const void* p, int64_t i) {
  if (dt == ORA_F32) return ((const float*)p)[i];
  if (dt == ORA_BF16) return bf16_widen(((const uint16_t*)p)[i]);
  return f16_widen(((const uint16_t*)p)[i]);
}

/* rT(x): round an fp32 value to T and return it widened back to fp32. */
static float rT(int dt, float x) {
  if (dt == ORA_F32) return x;
  if (dt == ORA_BF16) return bf16_widen(bf16_round(x));
  return f16_widen(f16_round(x));
}

static void store(int dt, void* p, int64_t i, float x) {
  if (dt == ORA_F32) ((float*)p)[i] = x;
  else if (dt == ORA_BF16) ((uint16_t*)p)[i] = bf16_round(x);
  else ((uint16_t*)p)[i] = f16_round(x);
}

/* "Numerics contract": accurate fp32 expf-based sigmoid. */
static float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

/* ScaledSiLU under the reading stated in the header: Z, SG and hidden are
 * each rounded once to T. */
static float scaled_silu(int dt, float down, float alpha) {
  float Z = rT(dt, alpha * down);
  float SG = rT(dt, sigmoid_f32(Z));
  return rT(dt, down * SG);
}

/* ------------------------------------------------------------------------ */
/* The block, one row.                                                      */
/* ------------------------------------------------------------------------ */

typedef struct {
  int dt;
  int64_t rows, C, H, R;
  const void *streams, *norm_scale, *down_w, *up_w, *inject_w, *prev_out, *prev_gate;
  void *pre_output, *post_gate, *streams_out;
  float eps, rs, alpha, gate_div, gate_mul;
  /* weights widened once to fp32 (exact) */
  const float *ns_f, *wd_f, *wu_f, *wi_f;
  /* optional trace of one row's intermediates (all fp32 holding T values) */
  int64_t trace_row;
  float* trace;
  /* optional [rows, H]: |reduction_scale| * sum_c |hn * g|, the magnitude that
   * feeds the rounding of pre_output (a diagnostic for tolerances near
   * cancellation; it does not change any output) */
  float* pre_mag;
} block_t;

/* Trace layout for one row (floats): S[K] hn[K] down[R] inject[C] Z[R] SG[R]
 * hidden[R] up[K] g[K] pre[H] post[C] ss[C]. */
static int64_t trace_floats(int64_t C, int64_t H, int64_t R) {
  int64_t K = C * H;
  return 4 * K + 4 * R + 3 * C + H;
}

typedef struct {
  float *S, *hn, *down, *inject, *hidden, *up, *g;
} row_scratch_t;

static void block_row(const block_t* b, int64_t m, row_scratch_t* w) {
  const int dt = b->dt;
  const int64_t C = b->C, H = b->H, R = b->R, K = C * H;
  float* tr = (b->trace && m == b->trace_row) ? b->trace : 0;
  float *tS = 0, *thn = 0, *tdown = 0, *tinj = 0, *tZ = 0, *tSG = 0, *thid = 0, *tup = 0, *tg = 0,
        *tpre = 0, *tpost = 0, *tss = 0;
  if (tr) {
    tS = tr; thn = tS + K; tdown = thn + K; tinj = tdown + R; tZ = tinj + C; tSG = tZ + R;
    thid = tSG + R; tup = thid + R; tg = tup + K; tpre = tg + K; tpost = tpre + H; tss = tpost + C;
  }

  /* Step 1, prologue ("Schema summary": S = streams + prev_post_gate * prev_block_output),
   * rounded to T at S. Without the prologue S is streams itself. */
  for (int64_t c = 0; c < C; ++c) {
    for (int64_t h = 0; h < H; ++h) {
      int64_t k = c * H + h;
      float s = widen(dt, b->streams, m * K + k);
      if (b->prev_out) {
        float q = widen(dt, b->prev_gate, m * C + c);
        float p = widen(dt, b->prev_out, m * H + h);
        float prod = q * p;
        s = rT(dt, s + prod);
      }
      w->S[k] = s;
    }
  }
  /* Step 2, streams_out = S (a copy of streams without the prologue). */
  if (b->streams_out)
    for (int64_t k = 0; k < K; ++k) store(dt, b->streams_out, m * K + k, w->S[k]);

  /* Step 3, per-branch weighted RMS norm, rounded at hn. */
  for (int64_t c = 0; c < C; ++c) {
    float ss = 0.0f;
    for (int64_t h = 0; h < H; ++h) {
      float x = w->S[c * H + h];
      ss = ss + x * x;
    }
    float den = sqrtf(ss / (float)H + b->eps);
    for (int64_t h = 0; h < H; ++h) {
      int64_t k = c * H + h;
      w->hn[k] = rT(dt, (w->S[k] / den) * b->ns_f[k]);
    }
    if (tss) tss[c] = ss;
  }

  /* Step 4, down = hn @ down_weight ([K, R] row-major), ascending k, rounded at down.
   * Step 5, inject = hn @ inject_weight ([K, C] row-major), rounded at inject.
   * The k-outer loop keeps one fp32 accumulator per output column; each
   * accumulator still adds its terms in ascending k. */
  for (int64_t n = 0; n < R; ++n) w->down[n] = 0.0f;
  for (int64_t c = 0; c < C; ++c) w->inject[c] = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    const float hk = w->hn[k];
    const float* wd = b->wd_f + k * R;
    for (int64_t n = 0; n < R; ++n) w->down[n] = w->down[n] + hk * wd[n];
    const float* wi = b->wi_f + k * C;
    for (int64_t c = 0; c < C; ++c) w->inject[c] = w->inject[c] + hk * wi[c];
  }
  for (int64_t n = 0; n < R; ++n) w->down[n] = rT(dt, w->down[n]);
  for (int64_t c = 0; c < C; ++c) w->inject[c] = rT(dt, w->inject[c]);

  /* Step 6, ScaledSiLU (rounded at Z, SG, hidden). */
  for (int64_t n = 0; n < R; ++n) {
    w->hidden[n] = scaled_silu(dt, w->down[n], b->alpha);
    if (tr) {
      tZ[n] = rT(dt, b->alpha * w->down[n]);
      tSG[n] = rT(dt, sigmoid_f32(tZ[n]));
    }
  }

  /* Step 7, up = hidden @ up_weight ([R, K] row-major), ascending n, rounded at
   * up; g = sigmoid(up), rounded at g. */
  for (int64_t j = 0; j < K; ++j) w->up[j] = 0.0f;
  for (int64_t n = 0; n < R; ++n) {
    const float hv = w->hidden[n];
    const float* wu = b->wu_f + n * K;
    for (int64_t j = 0; j < K; ++j) w->up[j] = w->up[j] + hv * wu[j];
  }
  for (int64_t j = 0; j < K; ++j) {
    w->up[j] = rT(dt, w->up[j]);
    w->g[j] = rT(dt, sigmoid_f32(w->up[j]));
  }

  /* Step 8, pre_output = reduction_scale * sum_c(hn * g), branches ascending,
   * rounded once at pre_output. */
  for (int64_t h = 0; h < H; ++h) {
    float acc = 0.0f;
    for (int64_t c = 0; c < C; ++c) acc = acc + w->hn[c * H + h] * w->g[c * H + h];
    float v = rT(dt, b->rs * acc);
    store(dt, b->pre_output, m * H + h, v);
    if (tpre) tpre[h] = v;
    if (b->pre_mag) {
      float mag = 0.0f;
      for (int64_t c = 0; c < C; ++c) mag = mag + fabsf(w->hn[c * H + h] * w->g[c * H + h]);
      b->pre_mag[m * H + h] = fabsf(b->rs) * mag;
    }
  }

  /* Step 9, post_gate = sigmoid(inject / gate_div) * gate_mul, rounded once. */
  for (int64_t c = 0; c < C; ++c) {
    float v = rT(dt, sigmoid_f32(w->inject[c] / b->gate_div) * b->gate_mul);
    store(dt, b->post_gate, m * C + c, v);
    if (tpost) tpost[c] = v;
  }

  if (tr) {
    memcpy(tS, w->S, K * 4); memcpy(thn, w->hn, K * 4); memcpy(tdown, w->down, R * 4);
    memcpy(tinj, w->inject, C * 4); memcpy(thid, w->hidden, R * 4); memcpy(tup, w->up, K * 4);
    memcpy(tg, w->g, K * 4);
  }
}

typedef struct {
  const block_t* b;
  int64_t lo, hi;
  int status;
} row_job_t;

static void* row_job(void* p) {
  row_job_t* j = (row_job_t*)p;
  const block_t* b = j->b;
  int64_t K = b->C * b->H;
  row_scratch_t w;
  float* mem = (float*)malloc(sizeof(float) * (size_t)(5 * K + 3 * b->R + b->C));
  if (!mem) { j->status = -1; return 0; }
  w.S = mem; w.hn = w.S + K; w.up = w.hn + K; w.g = w.up + K;
  w.down = w.g + K; w.hidden = w.down + b->R; w.inject = w.hidden + b->R;
  for (int64_t m = j->lo; m < j->hi; ++m) block_row(b, m, &w);
  free(mem);
  j->status = 0;
  return 0;
}

static float* widen_all(int dt, const void* p, int64_t n) {
  float* out = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  if (!out) return 0;
  for (int64_t i = 0; i < n; ++i) out[i] = widen(dt, p, i);
  return out;
}

static int run_block(block_t* b, int threads) {
  if (b->dt != ORA_F32 && b->dt != ORA_F16 && b->dt != ORA_BF16) return -2;
  if (b->C < 1 || b->H < 1 || b->R < 1 || b->rows < 0) return -3;
  if ((b->prev_out == 0) != (b->prev_gate == 0)) return -4;
  const int64_t K = b->C * b->H;
  float* ns = widen_all(b->dt, b->norm_scale, K);
  float* wd = widen_all(b->dt, b->down_w, K * b->R);
  float* wu = widen_all(b->dt, b->up_w, b->R * K);
  float* wi = widen_all(b->dt, b->inject_w, K * b->C);
  int rc = 0;
  if (!ns || !wd || !wu || !wi) { rc = -1; goto done; }
  b->ns_f = ns; b->wd_f = wd; b->wu_f = wu; b->wi_f = wi;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > b->rows) threads = (int)(b->rows > 0 ? b->rows : 1);
  {
    row_job_t jobs[256];
    pthread_t tid[256];
    int joined[256] = {0};
    int64_t per = b->rows > 0 ? (b->rows + threads - 1) / threads : 0;
    for (int t = 0; t < threads; ++t) {
      jobs[t].b = b;
      jobs[t].lo = (int64_t)t * per;
      jobs[t].hi = jobs[t].lo + per < b->rows ? jobs[t].lo + per : b->rows;
      if (jobs[t].lo > jobs[t].hi) jobs[t].lo = jobs[t].hi;
      jobs[t].status = 0;
    }
    for (int t = 1; t < threads; ++t)
      if (pthread_create(&tid[t], 0, row_job, &jobs[t]) == 0) joined[t] = 1;
      else row_job(&jobs[t]);
    row_job(&jobs[0]);
    for (int t = 1; t < threads; ++t) if (joined[t]) pthread_join(tid[t], 0);
    for (int t = 0; t < threads; ++t) if (jobs[t].status) rc = jobs[t].status;
  }
done:
  free(ns); free(wd); free(wu); free(wi);
  return rc;
}

/* Runs the block over all rows with T-rounding at the contract's points.
 * Inputs and outputs are host buffers of element type dtype, row-major,
 * leading dims flattened into rows. prev_out/prev_gate are both NULL (no
 * prologue) or both set. streams_out may be NULL. threads splits rows.
 * Returns 0 on success, negative on bad arguments or allocation failure. */
int hclrmix_oracle_run_mag(int dtype, int64_t rows, int64_t C, int64_t H, int64_t R,
                           const void* streams, const void* norm_scale, const void* down_w,
                           const void* up_w, const void* inject_w, const void* prev_out,
                           const void* prev_gate, void* pre_output, void* post_gate,
                           void* streams_out, float eps, float rs, float alpha, float gate_div,
                           float gate_mul, int threads, float* pre_mag);

int hclrmix_oracle_run(int dtype, int64_t rows, int64_t C, int64_t H, int64_t R,
                       const void* streams, const void* norm_scale, const void* down_w,
                       const void* up_w, const void* inject_w, const void* prev_out,
                       const void* prev_gate, void* pre_output, void* post_gate,
                       void* streams_out, float eps, float rs, float alpha, float gate_div,
                       float gate_mul, int threads) {
  return hclrmix_oracle_run_mag(dtype, rows, C, H, R, streams, norm_scale, down_w, up_w, inject_w,
                                prev_out, prev_gate, pre_output, post_gate, streams_out, eps, rs,
                                alpha, gate_div, gate_mul, threads, 0);
}

/* hclrmix_oracle_run that also writes pre_mag [rows, H] when it is not NULL. */
int hclrmix_oracle_run_mag(int dtype, int64_t rows, int64_t C, int64_t H, int64_t R,
                           const void* streams, const void* norm_scale, const void* down_w,
                           const void* up_w, const void* inject_w, const void* prev_out,
                           const void* prev_gate, void* pre_output, void* post_gate,
                           void* streams_out, float eps, float rs, float alpha, float gate_div,
                           float gate_mul, int threads, float* pre_mag) {
  block_t b;
  memset(&b, 0, sizeof b);
  b.dt = dtype; b.rows = rows; b.C = C; b.H = H; b.R = R;
  b.streams = streams; b.norm_scale = norm_scale; b.down_w = down_w; b.up_w = up_w;
  b.inject_w = inject_w; b.prev_out = prev_out; b.prev_gate = prev_gate;
  b.pre_output = pre_output; b.post_gate = post_gate; b.streams_out = streams_out;
  b.eps = eps; b.rs = rs; b.alpha = alpha; b.gate_div = gate_div; b.gate_mul = gate_mul;
  b.trace_row = -1;
  b.pre_mag = pre_mag;
  return run_block(&b, threads);
}

/* Same as hclrmix_oracle_run, and also writes the intermediates of row
 * trace_row into trace (hclrmix_oracle_trace_floats(C,H,R) floats). */
int hclrmix_oracle_trace(int dtype, int64_t rows, int64_t C, int64_t H, int64_t R,
                         const void* streams, const void* norm_scale, const void* down_w,
                         const void* up_w, const void* inject_w, const void* prev_out,
                         const void* prev_gate, void* pre_output, void* post_gate,
                         void* streams_out, float eps, float rs, float alpha, float gate_div,
                         float gate_mul, int64_t trace_row, float* trace) {
  block_t b;
  memset(&b, 0, sizeof b);
  b.dt = dtype; b.rows = rows; b.C = C; b.H = H; b.R = R;
  b.streams = streams; b.norm_scale = norm_scale; b.down_w = down_w; b.up_w = up_w;
  b.inject_w = inject_w; b.prev_out = prev_out; b.prev_gate = prev_gate;
  b.pre_output = pre_output; b.post_gate = post_gate; b.streams_out = streams_out;
  b.eps = eps; b.rs = rs; b.alpha = alpha; b.gate_div = gate_div; b.gate_mul = gate_mul;
  b.trace_row = trace_row; b.trace = trace;
  return run_block(&b, 1);
}

int64_t hclrmix_oracle_trace_floats(int64_t C, int64_t H, int64_t R) { return trace_floats(C, H, R); }

/* ------------------------------------------------------------------------ */
/* fp64 reference without any rounding to T: the same algebra in double.    */
/* Inputs are element type dtype (widened exactly); outputs are double.     */
/* ------------------------------------------------------------------------ */

static double sigmoid_f64(double x) { return 1.0 / (1.0 + exp(-x)); }

int hclrmix_oracle_fp64(int dtype, int64_t rows, int64_t C, int64_t H, int64_t R,
                        const void* streams, const void* norm_scale, const void* down_w,
                        const void* up_w, const void* inject_w, const void* prev_out,
                        const void* prev_gate, double* pre_output, double* post_gate,
                        double* streams_out, double eps, double rs, double alpha,
                        double gate_div, double gate_mul) {
  if (dtype != ORA_F32 && dtype != ORA_F16 && dtype != ORA_BF16) return -2;
  if ((prev_out == 0) != (prev_gate == 0)) return -4;
  const int64_t K = C * H;
  double* S = (double*)malloc(sizeof(double) * (size_t)(3 * K + 2 * R + C));
  if (!S) return -1;
  double *hn = S + K, *g = hn + K, *down = g + K, *hid = down + R, *inj = hid + R;
  for (int64_t m = 0; m < rows; ++m) {
    for (int64_t c = 0; c < C; ++c)
      for (int64_t h = 0; h < H; ++h) {
        int64_t k = c * H + h;
        double s = widen(dtype, streams, m * K + k);
        if (prev_out) s += (double)widen(dtype, prev_gate, m * C + c) * widen(dtype, prev_out, m * H + h);
        S[k] = s;
        if (streams_out) streams_out[m * K + k] = s;
      }
    for (int64_t c = 0; c < C; ++c) {
      double ss = 0;
      for (int64_t h = 0; h < H; ++h) ss += S[c * H + h] * S[c * H + h];
      double den = sqrt(ss / (double)H + eps);
      for (int64_t h = 0; h < H; ++h) hn[c * H + h] = S[c * H + h] / den * widen(dtype, norm_scale, c * H + h);
    }
    for (int64_t n = 0; n < R; ++n) {
      double a = 0;
      for (int64_t k = 0; k < K; ++k) a += hn[k] * widen(dtype, down_w, k * R + n);
      down[n] = a;
      hid[n] = a * sigmoid_f64(alpha * a);
    }
    for (int64_t c = 0; c < C; ++c) {
      double a = 0;
      for (int64_t k = 0; k < K; ++k) a += hn[k] * widen(dtype, inject_w, k * C + c);
      inj[c] = a;
      post_gate[m * C + c] = sigmoid_f64(a / gate_div) * gate_mul;
    }
    for (int64_t j = 0; j < K; ++j) {
      double a = 0;
      for (int64_t n = 0; n < R; ++n) a += hid[n] * widen(dtype, up_w, n * K + j);
      g[j] = sigmoid_f64(a);
    }
    for (int64_t h = 0; h < H; ++h) {
      double a = 0;
      for (int64_t c = 0; c < C; ++c) a += hn[c * H + h] * g[c * H + h];
      pre_output[m * H + h] = rs * a;
    }
  }
  free(S);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Codec entry points (for exhaustive checks of the rounding definitions).  */
/* ------------------------------------------------------------------------ */

/* out[i] = bits of rT(in[i]) for T in {10 float16, 16 bfloat16}. */
void hclrmix_oracle_round(int dtype, const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = dtype == ORA_BF16 ? bf16_round(in[i]) : f16_round(in[i]);
}

/* Same over a range of fp32 bit patterns [first, first+n). */
void hclrmix_oracle_round_bits(int dtype, uint32_t first, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    float f = bits_f32(first + (uint32_t)i);
    out[i] = dtype == ORA_BF16 ? bf16_round(f) : f16_round(f);
  }
}

/* out[i] = f(in[i]), the exact fp32 value of a stored 16-bit element. */
void hclrmix_oracle_widen(int dtype, const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = dtype == ORA_BF16 ? bf16_widen(in[i]) : f16_widen(in[i]);
}

/* The oracle's fp32 sigmoid, exposed for pins. */
float hclrmix_oracle_sigmoid(float x) { return sigmoid_f32(x); }

/* ------------------------------------------------------------------------ */
/* inv_rms (TEST INFRASTRUCTURE ONLY, like everything in this file).          */
/*                                                                          */
/* FreeToken PR #101, "compute the hyper-connection pre-norm in one kernel",  */
/* section "The problem": one value per row, the reciprocal square root of    */
/* the row's mean square plus eps, from the 16-bit source (section "The       */
/* change": the widening is exact, so the squares are those of the source).  */
/* Reading: the value is taken in fp64 -- a 16-bit value's square is exact in */
/* fp64 and the ascending sum of up to 2^20 of them has relative error below  */
/* 2^-32 -- and rounded once to fp32 (nearest even). That is the reference    */
/* the page's section "Accuracy" measures every fp32 form against.            */
/* ------------------------------------------------------------------------ */
static double inv_rms_row64(int dt, const void* x, int64_t row, int64_t dim, double eps) {
  double ss = 0.0;
  for (int64_t d = 0; d < dim; ++d) {
    const double v = (double)widen(dt, x, row * dim + d);
    ss = ss + v * v;
  }
  return 1.0 / sqrt(ss / (double)dim + eps);
}

int hclrmix_oracle_inv_rms64(int dtype, int64_t rows, int64_t dim, const void* x, double eps, double* out) {
  if (rows < 0 || dim < 1 || (rows > 0 && (!x || !out))) return 1;
  for (int64_t r = 0; r < rows; ++r) out[r] = inv_rms_row64(dtype, x, r, dim, eps);
  return 0;
}

int hclrmix_oracle_inv_rms(int dtype, int64_t rows, int64_t dim, const void* x, double eps, float* out) {
  if (rows < 0 || dim < 1 || (rows > 0 && (!x || !out))) return 1;
  for (int64_t r = 0; r < rows; ++r) out[r] = (float)inv_rms_row64(dtype, x, r, dim, eps);
  return 0;
}
