// Generic vector-ALU path of the HyperConnectionLowRankMix block: any element
// type, any shape, any row count. It serves fp32 and shapes outside the
// matrix-core envelope. Every sum is taken in an order fixed by the shape
// alone, so a row's bits do not depend on the row count.
//
// Four kernels, following onnxruntime PR #33384 "Schema summary":
//   rms   : prologue, streams_out, per-branch reciprocal RMS   (one workgroup per row and branch)
//   down  : hn @ [down | inject] over one part of K            (64 columns x 4 rows per workgroup)
//   fin   : the K parts in order, ScaledSiLU, post_gate        (one thread per output)
//   up    : hidden @ up, sigmoid, pre-mix                      (64 features x 4 rows per workgroup)
// or, for tiny problems, all four in one workgroup (tiny), in the same orders.
#include "hc_device.h"
#include "hc_internal.h"

namespace hc {

// S[m, c*H + h] recomputed from the inputs; identical to what rms writes.
template <DT D>
__device__ __forceinline__ float S_recompute(const Args& a, int64_t m, int c, int h) {
  float s = ld<D>(a.streams, m * a.K + (int64_t)c * a.H + h);
  if (a.prev_out) s = prologue<D>(s, ld<D>(a.prev_gate, m * a.C + c), ld<D>(a.prev_out, m * a.H + h));
  return s;
}

template <DT D>
__device__ __forceinline__ float S_load(const Args& a, int64_t m, int c, int h) {
  if (a.streams_out) return ld<D>(a.streams_out, m * a.K + (int64_t)c * a.H + h);
  return S_recompute<D>(a, m, c, h);
}

// One workgroup per (row, branch): wave i plays quarter i of the canonical
// sum of squares' 256 virtual lanes (lane L: virtual lane 64 i + L), writes
// streams_out for the elements it visits, and the four quarter sums are
// combined in their fixed order.
template <DT D>
__global__ __launch_bounds__(256) void k_generic_rms(Args a, float* __restrict__ rinv) {
  __shared__ float qs[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NQ = (a.H + 7) >> 3;
  for (int64_t pair = blockIdx.x; pair < a.M * a.C; pair += gridDim.x) {
    const int64_t m = pair / a.C;
    const int c = (int)(pair - m * a.C);
    float acc = 0.0f;
    for (int q = 64 * wave + lane; q < NQ; q += 256)
      for (int e = 0; e < 8; ++e) {
        const int h = 8 * q + e;
        if (h < a.H) {
          const float x = S_recompute<D>(a, m, c, h);
          if (a.streams_out) st<D>(a.streams_out, m * a.K + (int64_t)c * a.H + h, x);
          acc = acc + x * x;
        }
      }
    const float t = wave_allsum(acc);
    if (lane == 0) qs[wave] = t;
    __syncthreads();
    if (threadIdx.x == 0) rinv[pair] = rinv_from_ss(ss_combine(qs[0], qs[1], qs[2], qs[3]), a.H, a.eps);
    __syncthreads();  // qs is reused by the next pair
  }
}

// down (eight waves) and up (sixteen): one workgroup per block of 64 output
// columns (or features) and GEN_RB rows. down also splits K into
// P = generic_parts(K) contiguous parts over the grid's y dimension. Inside a
// workgroup the waves split their reduction range (the K part for down, R for
// up) into one contiguous piece each, summed in ascending order by a lane that
// owns one column; the pieces are then added in order, and down's K parts in
// order by k_generic_down_fin. The order depends only on K and R, so a row's
// bits do not depend on the row count.
constexpr int GEN_W = 8;     // waves per down workgroup
constexpr int GEN_WU = 16;   // waves per up workgroup
constexpr int GEN_RB = 4;    // rows per workgroup
constexpr int GEN_KC = 128;  // hn values per wave and row staged in LDS at a time
constexpr int GEN_CC = 8;    // branches whose up partials are combined at a time

// Piece w of [lo0, lo0 + n) split in W contiguous pieces.
template <int W>
__device__ __forceinline__ void gen_part(int lo0, int n, int w, int& lo, int& hi) {
  const int len = (n + W - 1) / W;
  lo = lo0 + min(n, w * len);
  hi = lo0 + min(n, min(n, w * len) + len);
}

// partial[p][m][n] (n < R + C): column n of row m summed over K part p.
template <DT D>
__global__ __launch_bounds__(512) void k_generic_down(Args a, const float* __restrict__ rinv,
                                                      float* __restrict__ partial) {
  __shared__ float hn_s[GEN_W][GEN_RB][GEN_KC];
  __shared__ float part[GEN_W][GEN_RB][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 64 + lane, NC = a.R + a.C;
  const bool is_down = n < a.R, is_inj = n >= a.R && n < NC;
  // This lane's weight column, read without a branch (a lane past the last
  // column reads column 0 of down_weight; its sums are never stored), so that
  // the loads of several k can be in flight at once.
  const void* wsrc = is_inj ? a.wi : a.wd;
  const int64_t wstr = is_inj ? a.C : a.R, wcol = is_down ? n : is_inj ? n - a.R : 0;
  const int p = blockIdx.y, KP = (a.K + gridDim.y - 1) / gridDim.y;
  const int kp_lo = min(a.K, p * KP), kp_hi = min(a.K, kp_lo + KP);
  int k_lo, k_hi;
  gen_part<GEN_W>(kp_lo, kp_hi - kp_lo, wave, k_lo, k_hi);
  for (int64_t m0 = (int64_t)blockIdx.z * GEN_RB; m0 < a.M; m0 += (int64_t)gridDim.z * GEN_RB) {
    const int nr = (int)min((int64_t)GEN_RB, a.M - m0);
    float acc[GEN_RB];
#pragma unroll
    for (int r = 0; r < GEN_RB; ++r) acc[r] = 0.0f;
    for (int k0 = k_lo; k0 < k_hi; k0 += GEN_KC) {
      const int kn = min(GEN_KC, k_hi - k0);
      // this wave's hn chunk for the workgroup's rows (only this wave reads it)
      for (int i = lane; i < GEN_RB * kn; i += 64) {
        const int r = i / kn, kk = i - r * kn, k = k0 + kk, c = k / a.H, h = k - c * a.H;
        const int64_t m = m0 + min(r, nr - 1);
        hn_s[wave][r][kk] = hnorm<D>(S_load<D>(a, m, c, h), rinv[m * a.C + c], ld<D>(a.ns, k));
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll 8
      for (int kk = 0; kk < kn; ++kk) {
        const float wv = ld<D>(wsrc, (int64_t)(k0 + kk) * wstr + wcol);
#pragma unroll
        for (int r = 0; r < GEN_RB; ++r) acc[r] = acc[r] + hn_s[wave][r][kk] * wv;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
#pragma unroll
    for (int r = 0; r < GEN_RB; ++r) part[wave][r][lane] = acc[r];
    __syncthreads();
    // the eight pieces in order
    if (threadIdx.x < GEN_RB * 64) {
      const int r = threadIdx.x >> 6, l = threadIdx.x & 63, nn = blockIdx.x * 64 + l;
      if (r < nr && nn < NC) {
        float tot = 0.0f;
        for (int w = 0; w < GEN_W; ++w) tot = tot + part[w][r][l];
        partial[((int64_t)p * a.M + m0 + r) * NC + nn] = tot;
      }
    }
    __syncthreads();  // part is reused by the next row block
  }
}

// The K parts of each (row, column) in order, then ScaledSiLU -> hidden or
// the inject gate.
template <DT D>
__global__ __launch_bounds__(256) void k_generic_down_fin(Args a, int P, const float* __restrict__ partial,
                                                          void* __restrict__ hidden) {
  const int NC = a.R + a.C;
  const int64_t total = a.M * NC, stride = (int64_t)gridDim.x * 256;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < total; gi += stride) {
    const int64_t m = gi / NC;
    const int n = (int)(gi - m * NC);
    float tot = 0.0f;
    for (int q = 0; q < P; ++q) tot = tot + partial[((int64_t)q * a.M + m) * NC + n];
    if (n < a.R) st<D>(hidden, m * a.R + n, scaled_silu<D>(rT<D>(tot), a.alpha));
    else st<D>(a.post, m * a.C + (n - a.R), post_gate<D>(rT<D>(tot), a.gate_div, a.gate_mul));
  }
}

constexpr int GEN_RMAX = 8192;

// Workgroup (64 features, GEN_RB rows, GEN_WU waves): wave w sums piece w of
// R for every branch; for each branch the pieces are added in order, then g,
// hn and the pre-mix over branches in ascending c.
template <DT D>
__global__ __launch_bounds__(64 * GEN_WU) void k_generic_up(Args a, const float* __restrict__ rinv,
                                                            const void* __restrict__ hidden) {
  __shared__ float part[GEN_WU][GEN_CC][GEN_RB][64];
  __shared__ float mix[GEN_RB][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 64 + lane;
  int r_lo, r_hi;
  gen_part<GEN_WU>(0, a.R, wave, r_lo, r_hi);
  for (int64_t m0 = (int64_t)blockIdx.y * GEN_RB; m0 < a.M; m0 += (int64_t)gridDim.y * GEN_RB) {
    const int nr = (int)min((int64_t)GEN_RB, a.M - m0);
    if (threadIdx.x < GEN_RB * 64) mix[threadIdx.x >> 6][threadIdx.x & 63] = 0.0f;
    for (int c0 = 0; c0 < a.C; c0 += GEN_CC) {
      const int cn = min(GEN_CC, a.C - c0);
      for (int cc = 0; cc < cn; ++cc) {
        float up[GEN_RB];
#pragma unroll
        for (int r = 0; r < GEN_RB; ++r) up[r] = 0.0f;
        if (h < a.H) {
          const int64_t j = (int64_t)(c0 + cc) * a.H + h;
#pragma unroll 4
          for (int n = r_lo; n < r_hi; ++n) {
            const float wv = ld<D>(a.wu, (int64_t)n * a.K + j);
#pragma unroll
            for (int r = 0; r < GEN_RB; ++r)
              up[r] = up[r] + ld<D>(hidden, (m0 + min(r, nr - 1)) * a.R + n) * wv;
          }
        }
#pragma unroll
        for (int r = 0; r < GEN_RB; ++r) part[wave][cc][r][lane] = up[r];
      }
      __syncthreads();
      // branches of this group in ascending c: parts in order, g, hn, pre-mix
      if (threadIdx.x < GEN_RB * 64) {
        const int r = threadIdx.x >> 6, l = threadIdx.x & 63, hh = blockIdx.x * 64 + l;
        if (r < nr && hh < a.H) {
          const int64_t m = m0 + r;
          float acc = mix[r][l];
          for (int cc = 0; cc < cn; ++cc) {
            float u = 0.0f;
            for (int w = 0; w < GEN_WU; ++w) u = u + part[w][cc][r][l];
            const int c = c0 + cc;
            const float g = up_gate<D>(u);
            const float hn = hnorm<D>(S_load<D>(a, m, c, hh), rinv[m * a.C + c], ld<D>(a.ns, (int64_t)c * a.H + hh));
            acc = acc + hn * g;
          }
          mix[r][l] = acc;
        }
      }
      __syncthreads();
    }
    if (threadIdx.x < GEN_RB * 64) {
      const int r = threadIdx.x >> 6, l = threadIdx.x & 63, hh = blockIdx.x * 64 + l;
      if (r < nr && hh < a.H) st<D>(a.pre, (m0 + r) * a.H + hh, rT<D>(a.rs * mix[r][l]));
    }
  }
}

// The whole block in one workgroup, for problems small enough that the four
// kernels' launches would cost more than their work: the same values in the
// same orders as rms, down, fin and up above. Each piece of a sum that those
// kernels give to one wave or lane is summed by one thread here, and the
// pieces are added in the same order, so a row's bits do not depend on which
// of the two runs it. Every operand is first brought into LDS (as fp32) by
// loads that do not depend on each other; S is recomputed from the inputs
// (the same bits as streams_out).
constexpr int TINY_THREADS = 1024;
constexpr int TINY_LDS = 32768;  // fp32 values of LDS the whole problem must fit in
bool generic_tiny(int64_t M, int C, int H, int R) {
  const int64_t K = (int64_t)C * H, P = generic_parts(K);
  const int64_t need = M * K + M * R + K * R + K * C + R * K + K + M * C + 16 + M * (R + C) * P * GEN_W +
                       M * K * GEN_WU;
  return M >= 1 && need <= TINY_LDS && M * K * (2 * (int64_t)R + C) <= ((int64_t)1 << 21);
}

template <DT D>
__global__ __launch_bounds__(TINY_THREADS) void k_generic_tiny(Args a, int P, void* __restrict__ hidden) {
  __shared__ float sm[TINY_LDS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int M = (int)a.M, C = a.C, H = a.H, R = a.R, K = a.K, NC = R + C;
  float* S_s = sm;               // [M][K]: S, then hn
  float* hid_s = S_s + M * K;    // [M][R]
  float* wd_s = hid_s + M * R;   // [K][R]
  float* wi_s = wd_s + K * R;    // [K][C]
  float* wu_s = wi_s + K * C;    // [R][K]
  float* ns_s = wu_s + R * K;    // [K]
  float* rinv_s = ns_s + K;      // [M][C]
  float* qs = rinv_s + M * C;    // [16]
  float* pd_s = qs + 16;         // [M][P][GEN_W][R + C]: down pieces
  float* pu_s = pd_s + M * NC * P * GEN_W;  // [M][GEN_WU][K]: up pieces of (row, branch, feature)
  // 0. Operands into LDS; S (and streams_out). The loops are unrolled so that
  //    a thread's loads go out before it waits for the first.
#pragma unroll 8
  for (int i = tid; i < K * R; i += TINY_THREADS) wd_s[i] = ld<D>(a.wd, i);
#pragma unroll 8
  for (int i = tid; i < K * C; i += TINY_THREADS) wi_s[i] = ld<D>(a.wi, i);
#pragma unroll 8
  for (int i = tid; i < R * K; i += TINY_THREADS) wu_s[i] = ld<D>(a.wu, i);
#pragma unroll 4
  for (int i = tid; i < K; i += TINY_THREADS) ns_s[i] = ld<D>(a.ns, i);
#pragma unroll 4
  for (int i = tid; i < M * K; i += TINY_THREADS) {
    const int m = i / K, k = i - m * K, c = k / H;
    const float x = S_recompute<D>(a, m, c, k - c * H);
    S_s[i] = x;
    if (a.streams_out) st<D>(a.streams_out, i, x);
  }
  __syncthreads();
  // 1. rms: four waves per (row, branch), wave i playing quarter i of the
  //    canonical virtual lanes (as k_generic_rms), four pairs at a time.
  const int NQ = (H + 7) >> 3;
  for (int pb = 0; pb < M * C; pb += 4) {
    const int pair = pb + (wave >> 2), wq = wave & 3;
    float acc = 0.0f;
    if (pair < M * C) {
      const float* row = S_s + pair * H;  // (row m, branch c) = pair m C + c: S_s + m K + c H
      for (int q = 64 * wq + lane; q < NQ; q += 256)
        for (int e = 0; e < 8; ++e) {
          const int h = 8 * q + e;
          if (h < H) acc = acc + row[h] * row[h];
        }
    }
    const float t = wave_allsum(acc);
    if (lane == 0) qs[wave] = t;
    __syncthreads();
    if (tid < 4 && pb + tid < M * C)
      rinv_s[pb + tid] = rinv_from_ss(ss_combine(qs[4 * tid], qs[4 * tid + 1], qs[4 * tid + 2], qs[4 * tid + 3]), H,
                                      a.eps);
    __syncthreads();
  }
  // 2. hn of every row, in place.
  for (int i = tid; i < M * K; i += TINY_THREADS) {
    const int m = i / K, k = i - m * K;
    S_s[i] = hnorm<D>(S_s[i], rinv_s[m * C + k / H], ns_s[k]);
  }
  __syncthreads();
  // 3. down and inject (as k_generic_down then k_generic_down_fin): per
  //    output, the K parts in order, each the sum of its GEN_W pieces in
  //    order, each piece k ascending from zero; then ScaledSiLU or the gate.
  const int KP = (K + P - 1) / P;  // P = generic_parts(K)
  // (Items are ordered column fastest, so neighbouring threads read
  //  neighbouring weights and the same hn value: no LDS bank conflicts.)
  // (A thread's item index i = r NC + n, r = (m P + p) GEN_W + w, advances by
  //  TINY_THREADS = dq NC + dr: n and r are stepped with a carry, not divided.)
  {
    const int dq = TINY_THREADS / NC, dr = TINY_THREADS - dq * NC;
    int n = tid % NC, r = tid / NC;
    for (int i = tid; i < M * NC * P * GEN_W; i += TINY_THREADS) {  // piece (m, p, w, n)
      const int w = r % GEN_W, mp = r / GEN_W, p = mp % P, m = mp / P;
      const float* hn = S_s + m * K;
      const float* wcol = n < R ? wd_s + n : wi_s + (n - R);
      const int ws = n < R ? R : C;
      const int kp_lo = min(K, p * KP), kp_hi = min(K, kp_lo + KP);
      int lo, hi;
      gen_part<GEN_W>(kp_lo, kp_hi - kp_lo, w, lo, hi);
      float acc = 0.0f;
#pragma unroll 8
      for (int k = lo; k < hi; ++k) acc = acc + hn[k] * wcol[k * ws];
      pd_s[i] = acc;
      n += dr;
      r += dq;
      if (n >= NC) {
        n -= NC;
        ++r;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < M * NC; i += TINY_THREADS) {
    const int m = i / NC, n = i - m * NC;
    float tot = 0.0f;
    for (int p = 0; p < P; ++p) {
      float part = 0.0f;
      for (int w = 0; w < GEN_W; ++w) part = part + pd_s[((m * P + p) * GEN_W + w) * NC + n];
      tot = tot + part;
    }
    if (n < R) {
      const float hv = rT<D>(scaled_silu<D>(rT<D>(tot), a.alpha));
      hid_s[m * R + n] = hv;
      st<D>(hidden, (int64_t)m * R + n, hv);
    } else {
      st<D>(a.post, (int64_t)m * C + (n - R), post_gate<D>(rT<D>(tot), a.gate_div, a.gate_mul));
    }
  }
  __syncthreads();
  // 4. up and pre-mix (as k_generic_up): per (row, feature), branches
  //    ascending; per branch the GEN_WU pieces of R in order, each n ascending
  //    from zero; g, hn and the pre-mix term.
  {
    const int dq = TINY_THREADS / K, dr = TINY_THREADS - dq * K;  // the item index stepped as above
    int j = tid % K, mw = tid / K;
    for (int i = tid; i < M * K * GEN_WU; i += TINY_THREADS) {  // piece (m, w, j = c H + h), j fastest
      const int w = mw % GEN_WU, m = mw / GEN_WU;
      int lo, hi;
      gen_part<GEN_WU>(0, R, w, lo, hi);
      float up = 0.0f;
      for (int n = lo; n < hi; ++n) up = up + hid_s[m * R + n] * wu_s[n * K + j];
      pu_s[i] = up;
      j += dr;
      mw += dq;
      if (j >= K) {
        j -= K;
        ++mw;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < M * H; i += TINY_THREADS) {
    const int m = i / H, h = i - m * H;
    float mix = 0.0f;
    for (int c = 0; c < C; ++c) {
      const int j = c * H + h;
      float u = 0.0f;
      for (int w = 0; w < GEN_WU; ++w) u = u + pu_s[(m * GEN_WU + w) * K + j];
      const float g = up_gate<D>(u);
      mix = mix + S_s[m * K + j] * g;
    }
    st<D>(a.pre, (int64_t)m * H + h, rT<D>(a.rs * mix));
  }
}

template <DT D>
static hipError_t run_generic(const Args& a, char* ws, const Workspace& w, hipStream_t s, Marks* mk) {
  float* rinv = (float*)(ws + w.rinv);
  void* hidden = ws + w.hidden;
  float* partial = (float*)(ws + w.partial);
  const int64_t pairs = a.M * a.C;
  const int64_t rb = (a.M + GEN_RB - 1) / GEN_RB;
  const int P = generic_parts(a.K);
  if (a.R > GEN_RMAX) return hipErrorInvalidValue;
  if (generic_tiny(a.M, a.C, a.H, a.R))
    return launch(mk, k_generic_tiny<D>, dim3(1), dim3(TINY_THREADS), 0, s, a, P, hidden);
  hipError_t e = launch(mk, k_generic_rms<D>, dim3((unsigned)(pairs < (1 << 20) ? pairs : (1 << 20))), dim3(256), 0,
                        s, a, rinv);  // pairs strided beyond that
  if (e != hipSuccess) return e;
  e = launch(mk, k_generic_down<D>, dim3((unsigned)((a.R + a.C + 63) / 64), (unsigned)P,
                                         (unsigned)(rb < 65535 ? rb : 65535)),  // row blocks, strided beyond
             dim3(64 * GEN_W), 0, s, a, (const float*)rinv, partial);
  if (e != hipSuccess) return e;
  const int64_t fb = (a.M * (a.R + a.C) + 255) / 256;
  e = launch(mk, k_generic_down_fin<D>, dim3((unsigned)(fb < 65536 ? fb : 65536)), dim3(256), 0, s, a, P,
             (const float*)partial, hidden);
  if (e != hipSuccess) return e;
  const unsigned gy = (unsigned)(rb < 32768 ? rb : 32768);  // row blocks, strided beyond that
  return launch(mk, k_generic_up<D>, dim3((unsigned)((a.H + 63) / 64), gy), dim3(64 * GEN_WU), 0, s, a,
                (const float*)rinv, (const void*)hidden);
}

hipError_t launch_generic(const Args& a, int dtype, char* ws, const Workspace& w, hipStream_t s, Marks* mk) {
  switch (dtype) {
    case 1: return run_generic<DT::F32>(a, ws, w, s, mk);
    case 10: return run_generic<DT::F16>(a, ws, w, s, mk);
    case 16: return run_generic<DT::BF16>(a, ws, w, s, mk);
  }
  return hipErrorInvalidValue;
}

}  // namespace hc
