// Decode path (few rows) of the HyperConnectionLowRankMix block on gfx950.
//
// The time goes into streaming the three weight matrices once from HBM
// (13.2 MB for 4 x 2560, rank 320, bf16). Each kernel therefore issues all of a
// workgroup's weight loads before anything else, as 16-byte coalesced loads,
// then stages them in LDS and reads matrix-core fragments with transposing LDS
// reads (the weights stay row-major [K, N] and are used in place, as in
// onnxruntime PR #33384, "Motivation and Context").
//
//   hc_down   grid (slice x tile group, row group): prologue + per-branch RMS
//             of its rows, hn of its K slice, one matrix-core chain per 16
//             output columns of [down | inject], fp32 partial sums per slice.
//   hc_mid    fixed-order reduction of the partials (slices within a branch,
//             then branches), ScaledSiLU -> hidden, inject -> post_gate.
//   hc_uppre  grid (16 features, row group), one wave per branch: up chain over
//             R, sigmoid, hn recomputed, pre-mix over branches in ascending c.
//
// Rows are taken in groups of 16 (one matrix-core tile); rows beyond the
// batch are zero and never stored. The split of the work follows the "CUDA
// implementation" section of the PR (split-K partials, then a consumer that
// reduces them in a fixed order); the tiles and fragments are gfx950's.
#include "hc_mfma_common.h"

namespace hc {

constexpr int KSMAX = 256;          // largest slice length
constexpr int HN_LD = KSMAX + 8;    // padded LDS row of hn (elements)

template <DT D>
__global__ __launch_bounds__(256) void k_hc_down(Args a, Geometry g, float* __restrict__ partial,
                                                 float* __restrict__ rinv_out) {
  __shared__ __attribute__((aligned(16))) uint16_t hn_lds[16 * HN_LD];
  __shared__ __attribute__((aligned(16))) uint16_t w_lds[4 * KSMAX * 16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NG = (g.NT + 3) >> 2;
  const int s = blockIdx.x / NG, b = blockIdx.x - s * NG;
  const int c = s / g.SPB, s_in = s - c * g.SPB;
  const int KS = g.KS, h_lo = s_in * KS;
  const int64_t kbase = (int64_t)c * a.H + h_lo;

  // 1. Weight tile of this workgroup: rows kbase .. kbase+KS of columns
  //    [64b, 64b+64) of [down | inject | 0]; eight threads per row, 16 bytes each.
  uint4 wreg[KSMAX / 32];
  const int col8 = 64 * b + 8 * (tid & 7);
  const uint16_t* wd = (const uint16_t*)a.wd;
  const uint16_t* wi = (const uint16_t*)a.wi;
#pragma unroll
  for (int p = 0; p < KSMAX / 32; ++p) {
    wreg[p] = make_uint4(0u, 0u, 0u, 0u);
    const int rr = 32 * p + (tid >> 3);
    if (rr < KS) {
      const int64_t k = kbase + rr;
      if (col8 + 8 <= a.R) {
        wreg[p] = *(const uint4*)(wd + k * a.R + col8);
      } else if (col8 == a.R) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < a.C) w[e >> 1] |= (uint32_t)wi[k * a.C + e] << (16 * (e & 1));
        wreg[p] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  bool wstored = false;
  for (int64_t rg = blockIdx.y; rg * 16 < a.M; rg += gridDim.y) {
    const int64_t m0 = rg * 16;
    // 2. Per-branch RMS of each row (one wave per row), hn of this slice into LDS.
    for (int r = wave; r < 16; r += 4) {
      const int64_t m = m0 + r;
      uint16_t* hrow = hn_lds + r * HN_LD;
      if (m >= a.M) {
        for (int i = lane; i < KS / 8; i += 64) *(uint4*)(hrow + 8 * i) = make_uint4(0u, 0u, 0u, 0u);
        continue;
      }
      const SRow sr = s_row<D>(a, m, c);
      const float rv = rinv_from_ss(branch_sumsq_vec<D>(sr, a.H, lane), a.H, a.eps);
      if (b == 0 && s_in == 0 && lane == 0) rinv_out[m * a.C + c] = rv;
      for (int i = lane; i < KS / 8; i += 64) {
        const int ch = (h_lo >> 3) + i;
        float x[8];
        load_S8<D>(sr.s, sr.p, sr.q, ch, x);
        if (b == 0 && a.streams_out)
          *(uint4*)((uint16_t*)a.streams_out + m * a.K + (int64_t)c * a.H + 8 * ch) = pack8<D>(x);
        float nsv[8], hv[8];
        unpack8<D>(*(const uint4*)((const uint16_t*)a.ns + (int64_t)c * a.H + 8 * ch), nsv);
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = hnorm<D>(x[e], rv, nsv[e]);
        *(uint4*)(hrow + 8 * i) = pack8<D>(hv);
      }
    }
    // 3. Weights to LDS, one [KS][16] tile per wave.
    if (!wstored) {
#pragma unroll
      for (int p = 0; p < KSMAX / 32; ++p) {
        const int rr = 32 * p + (tid >> 3);
        if (rr < KS) {
          const int j = tid & 7;
          *(uint4*)(w_lds + (j >> 1) * (KSMAX * 16) + rr * 16 + 8 * (j & 1)) = wreg[p];
        }
      }
      wstored = true;
    }
    __syncthreads();
    // 4. One matrix-core chain over the slice for output tile t = 4b + wave.
    const int t = 4 * b + wave;
    if (t < g.NT) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* tile = w_lds + wave * (KSMAX * 16);
      for (int k0 = 0; k0 < KS; k0 += 32)
        acc = mfma<D>(lds_afrag(hn_lds, HN_LD, k0, lane), lds_bfrag(tile, k0, lane), acc);
      const int n = 16 * t + (lane & 15);
      if (n < a.R + a.C) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + 4 * (lane >> 4) + r;
          if (m < a.M) partial[((int64_t)s * a.M + m) * g.NP + n] = acc[r];
        }
      }
    }
    __syncthreads();
  }
}

// Reduction of fp32 partials laid out [C * spb][M][NP] in the canonical order
// (slices within a branch, then branches), then the down/inject epilogue.
// Decode passes spb = slices per branch; prefill passes spb = 1 (one partial
// per branch, already summed over its slices in the same order).
template <DT D>
__global__ __launch_bounds__(256) void k_hc_mid(Args a, int spb, int NP, const float* __restrict__ partial,
                                                void* __restrict__ hidden) {
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  if (n >= a.R + a.C) return;
  for (int64_t m = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6); m < a.M; m += (int64_t)gridDim.y * 4) {
    float tot = 0.0f;
    for (int c = 0; c < a.C; ++c) {
      float br = 0.0f;
      for (int si = 0; si < spb; ++si) br = br + partial[((int64_t)(c * spb + si) * a.M + m) * NP + n];
      tot = tot + br;
    }
    finish_down_inject<D>(a, m, n, tot, hidden);
  }
}

// up = hidden @ up_weight for 16 features h of every branch (one wave per
// branch c), then g, hn and the pre-mix over branches.
template <DT D>
__global__ __launch_bounds__(512) void k_hc_uppre(Args a, const float* __restrict__ rinv,
                                                  const void* __restrict__ hidden) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int R = a.R, HLD = R + 8;
  uint16_t* hid_lds = (uint16_t*)smem;                 // [16][R + 8]
  uint16_t* wu_lds = hid_lds + 16 * HLD;               // [C][R][16]
  float* e_lds = (float*)(wu_lds + a.C * R * 16);      // [C][16][16]
  const int tid = threadIdx.x, c = tid >> 6, lane = tid & 63;
  const int nthreads = blockDim.x;
  const int h0 = blockIdx.x * 16;

  // Wu tile of branch c: rows 0..R-1, columns c*H + h0 .. +16; two lanes per row.
  uint4 wreg[16];
  const uint16_t* wu = (const uint16_t*)a.wu;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int n = 32 * p + (lane >> 1);
    wreg[p] = make_uint4(0u, 0u, 0u, 0u);
    if (n < R) wreg[p] = *(const uint4*)(wu + (int64_t)n * a.K + (int64_t)c * a.H + h0 + 8 * (lane & 1));
  }

  bool wstored = false;
  const int R8 = R >> 3;
  for (int64_t rg = blockIdx.y; rg * 16 < a.M; rg += gridDim.y) {
    const int64_t m0 = rg * 16;
    for (int i = tid; i < 16 * R8; i += nthreads) {
      const int r = i / R8, j = i - r * R8;
      const int64_t m = m0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < a.M) v = *(const uint4*)((const uint16_t*)hidden + m * R + 8 * j);
      *(uint4*)(hid_lds + r * HLD + 8 * j) = v;
    }
    if (!wstored) {
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int n = 32 * p + (lane >> 1);
        if (n < R) *(uint4*)(wu_lds + ((int64_t)c * R + n) * 16 + 8 * (lane & 1)) = wreg[p];
      }
      wstored = true;
    }
    __syncthreads();
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* tile = wu_lds + c * R * 16;
    for (int k0 = 0; k0 < R; k0 += 32)
      acc = mfma<D>(lds_afrag(hid_lds, HLD, k0, lane), lds_bfrag(tile, k0, lane), acc);
    const int h = h0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 4 * (lane >> 4) + r;
      const int64_t m = m0 + rr;
      float e = 0.0f;
      if (m < a.M) e = premix_term<D>(a, rinv, m, c, h, acc[r]);
      e_lds[c * 256 + rr * 16 + (lane & 15)] = e;
    }
    __syncthreads();
    for (int i = tid; i < 256; i += nthreads) {
      const int rr = i >> 4, hh = i & 15;
      const int64_t m = m0 + rr;
      if (m < a.M) {
        float sum = 0.0f;
        for (int cc = 0; cc < a.C; ++cc) sum = sum + e_lds[cc * 256 + i];
        st<D>(a.pre, m * a.H + h0 + hh, rT<D>(a.rs * sum));
      }
    }
    __syncthreads();
  }
}

hipError_t launch_mid(const Args& a, int dtype, int spb, int NP, const float* partial, void* hidden,
                      hipStream_t s);

size_t uppre_lds_bytes(int C, int R) {
  return (size_t)16 * (R + 8) * 2 + (size_t)C * R * 16 * 2 + (size_t)C * 256 * 4;
}

template <DT D>
static hipError_t run_decode(const Args& a, char* ws, const Workspace& w, const Geometry& g, hipStream_t s,
                             Marks* mk) {
  float* rinv = (float*)(ws + w.rinv);
  void* hidden = ws + w.hidden;
  float* partial = (float*)(ws + w.partial);
  const int NG = (g.NT + 3) / 4;
  const int64_t rgroups = (a.M + 15) / 16;
  const unsigned gy = (unsigned)(rgroups < 65535 ? rgroups : 65535);
  const size_t lds = uppre_lds_bytes(a.C, a.R);
  hipError_t e = allow_dynamic_lds((const void*)k_hc_uppre<D>, D == DT::BF16 ? 0 : 1, lds);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_hc_down<D>, dim3((unsigned)(g.NS * NG), gy), dim3(256), 0, s, a, g, partial, rinv);
  if ((e = mark(mk, s)) != hipSuccess) return e;
  e = launch_mid(a, (int)D, g.SPB, g.NP, partial, hidden, s);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_hc_uppre<D>, dim3((unsigned)(a.H / 16), gy), dim3(64 * a.C), lds, s, a,
                     (const float*)rinv, (const void*)hidden);
  if ((e = mark(mk, s)) != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_decode(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                         hipStream_t s, Marks* mk) {
  if (dtype == 16) return run_decode<DT::BF16>(a, ws, w, g, s, mk);
  if (dtype == 10) return run_decode<DT::F16>(a, ws, w, g, s, mk);
  return hipErrorInvalidValue;
}

// The prefill path ends its down projection with the same reduction kernel.
hipError_t launch_mid(const Args& a, int dtype, int spb, int NP, const float* partial, void* hidden,
                      hipStream_t s) {
  const int64_t mq = (a.M + 3) / 4;
  const dim3 grid((unsigned)((a.R + a.C + 63) / 64), (unsigned)(mq < 65535 ? mq : 65535));
  if (dtype == 16) hipLaunchKernelGGL(k_hc_mid<DT::BF16>, grid, dim3(256), 0, s, a, spb, NP, partial, hidden);
  else if (dtype == 10) hipLaunchKernelGGL(k_hc_mid<DT::F16>, grid, dim3(256), 0, s, a, spb, NP, partial, hidden);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hc
