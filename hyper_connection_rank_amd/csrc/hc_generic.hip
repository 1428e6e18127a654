// Generic vector-ALU path of the HyperConnectionLowRankMix block: any element
// type, any shape, any row count. It serves fp32 and shapes outside the
// matrix-core envelope. Every output is computed by one thread in a fixed
// sequential order, so a row's bits do not depend on the row count.
//
// Three kernels, following onnxruntime PR #33384 "Schema summary":
//   rms   : prologue, streams_out, per-branch reciprocal RMS   (one wave per row and branch)
//   down  : hn @ [down | inject], ScaledSiLU, post_gate       (one thread per output column)
//   up    : hidden @ up, sigmoid, pre-mix                      (one thread per feature h)
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

// One wave per (row, branch): canonical sum of squares, rinv, streams_out.
template <DT D>
__global__ __launch_bounds__(256) void k_generic_rms(Args a, float* __restrict__ rinv) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= a.M * a.C) return;  // wave-uniform
  const int64_t m = pair / a.C;
  const int c = (int)(pair - m * a.C);
  const float ss = branch_sumsq(a.H, lane, [&](int h) { return S_recompute<D>(a, m, c, h); });
  if (lane == 0) rinv[pair] = rinv_from_ss(ss, a.H, a.eps);
  if (a.streams_out)
    for (int h = lane; h < a.H; h += 64)
      st<D>(a.streams_out, m * a.K + (int64_t)c * a.H + h, S_recompute<D>(a, m, c, h));
}

constexpr int GEN_KCHUNK = 8192;  // hn values staged in LDS per pass (32 KB)

// Block (column block, row): hn of the row staged through LDS in chunks of
// GEN_KCHUNK; thread n accumulates its column over k ascending.
template <DT D>
__global__ __launch_bounds__(256) void k_generic_down(Args a, const float* __restrict__ rinv,
                                                      void* __restrict__ hidden) {
  __shared__ float hn_s[GEN_KCHUNK];
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool is_down = n < a.R, is_inj = n >= a.R && n < a.R + a.C;
  for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
    float acc = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += GEN_KCHUNK) {
      const int kn = min(GEN_KCHUNK, a.K - k0);
      __syncthreads();
      for (int i = threadIdx.x; i < kn; i += 256) {
        const int k = k0 + i, c = k / a.H, h = k - c * a.H;
        hn_s[i] = hnorm<D>(S_load<D>(a, m, c, h), rinv[m * a.C + c], ld<D>(a.ns, k));
      }
      __syncthreads();
      if (is_down) {
        for (int i = 0; i < kn; ++i) acc = acc + hn_s[i] * ld<D>(a.wd, (int64_t)(k0 + i) * a.R + n);
      } else if (is_inj) {
        for (int i = 0; i < kn; ++i)
          acc = acc + hn_s[i] * ld<D>(a.wi, (int64_t)(k0 + i) * a.C + (n - a.R));
      }
    }
    if (is_down) {
      st<D>(hidden, m * a.R + n, scaled_silu<D>(rT<D>(acc), a.alpha));
    } else if (is_inj) {
      st<D>(a.post, m * a.C + (n - a.R), post_gate<D>(rT<D>(acc), a.gate_div, a.gate_mul));
    }
  }
}

constexpr int GEN_RMAX = 8192;

// Block (feature block, row): thread h computes up for every branch c, then
// g, hn and the pre-mix sum over branches in ascending c.
template <DT D>
__global__ __launch_bounds__(256) void k_generic_up(Args a, const float* __restrict__ rinv,
                                                    const void* __restrict__ hidden) {
  __shared__ float hid_s[GEN_RMAX];
  const int h = blockIdx.x * 256 + threadIdx.x;
  for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
    __syncthreads();
    for (int i = threadIdx.x; i < a.R; i += 256) hid_s[i] = ld<D>(hidden, m * a.R + i);
    __syncthreads();
    if (h < a.H) {
      float acc = 0.0f;
      for (int c = 0; c < a.C; ++c) {
        const int64_t j = (int64_t)c * a.H + h;
        float up = 0.0f;
        for (int n = 0; n < a.R; ++n) up = up + hid_s[n] * ld<D>(a.wu, (int64_t)n * a.K + j);
        const float g = up_gate<D>(up);
        const float hn = hnorm<D>(S_load<D>(a, m, c, h), rinv[m * a.C + c], ld<D>(a.ns, j));
        acc = acc + hn * g;
      }
      st<D>(a.pre, m * a.H + h, rT<D>(a.rs * acc));
    }
  }
}

template <DT D>
static hipError_t run_generic(const Args& a, char* ws, const Workspace& w, hipStream_t s, Marks* mk) {
  float* rinv = (float*)(ws + w.rinv);
  void* hidden = ws + w.hidden;
  const int64_t pairs = a.M * a.C;
  const unsigned gy = (unsigned)(a.M < 32768 ? a.M : 32768);
  hipError_t e = launch(mk, k_generic_rms<D>, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, a, rinv);
  if (e != hipSuccess) return e;
  e = launch(mk, k_generic_down<D>, dim3((unsigned)((a.R + a.C + 255) / 256), gy), dim3(256), 0, s, a,
             (const float*)rinv, hidden);
  if (e != hipSuccess) return e;
  return launch(mk, k_generic_up<D>, dim3((unsigned)((a.H + 255) / 256), gy), dim3(256), 0, s, a,
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
