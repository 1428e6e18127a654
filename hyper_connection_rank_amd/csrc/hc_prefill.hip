// Prefill path (many rows) of the HyperConnectionLowRankMix block on gfx950:
// down/inject and up become dense GEMMs on the matrix cores (the general path
// of onnxruntime PR #33384, "CUDA implementation", done with our own kernels
// and always with fp32 accumulation).
//
//   pf_down   grid (64-row tile, branch c): per-branch RMS of its rows
//             (streams_out written here), then hn @ [down | inject] over the
//             branch's K range, one matrix-core chain per slice, slices added
//             in order; writes one fp32 partial per branch.
//   branch_reduce  adds the branch partials in ascending c and applies
//             ScaledSiLU / the inject gate (the same order as the decode path's
//             ticket reduction: slices within a branch, then branches).
//   pf_uppre  grid (64-row tile, 16 features): up chain over R per branch,
//             sigmoid, hn recomputed, pre-mix over branches.
//
// Every arithmetic step is the same function, in the same order, as in the
// decode kernels, so a row's bits match the decode path's.
#include "hc_mfma_common.h"

namespace hc {


constexpr int PF_BM = 64;        // rows per workgroup
constexpr int PF_ALD = 40;       // padded LDS row of the hn chunk (elements)

template <DT D, int TPW>
__global__ __launch_bounds__(256) void k_pf_down(Args a, Geometry g, float* __restrict__ bpart,
                                                 float* __restrict__ rinv_out) {
  __shared__ float rinv_s[PF_BM];
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[PF_BM * PF_ALD];
  __shared__ __attribute__((aligned(16))) uint16_t b_lds[4 * TPW * 32 * 16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t m0 = (int64_t)blockIdx.x * PF_BM;
  const int c = blockIdx.y;

  // Pass 1: per-branch RMS of the 64 rows (one wave per row), streams_out.
  for (int r = wave; r < PF_BM; r += 4) {
    const int64_t m = m0 + r;
    float rv = 0.0f;
    if (m < a.M) {
      const SRow sr = s_row<D>(a, m, c);
      uint16_t* so = a.streams_out ? (uint16_t*)a.streams_out + m * a.K + (int64_t)c * a.H : nullptr;
      rv = rinv_from_ss(branch_sumsq_vec<D>(sr, a.H, lane, so), a.H, a.eps);
      if (lane == 0) rinv_out[m * a.C + c] = rv;
    }
    if (lane == 0) rinv_s[r] = rv;
  }
  __syncthreads();

  // Pass 2: the branch's K range in slices; per slice one chain per tile.
  f32x4 br[TPW][4], sl[TPW][4];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) br[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* wd = (const uint16_t*)a.wd;
  const uint16_t* wi = (const uint16_t*)a.wi;
  const int NP8 = g.NP / 8;
  for (int s_in = 0; s_in < g.SPB; ++s_in) {
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sl[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kk = 0; kk < g.KS; kk += 32) {
      const int hk = s_in * g.KS + kk;               // branch-local k of the chunk
      const int64_t kg = (int64_t)c * a.H + hk;      // global k
      {  // hn chunk [64 rows][32 k]: thread -> row tid/4, eight k at 8*(tid%4)
        const int r = tid >> 2, q = tid & 3;
        const int64_t m = m0 + r;
        float hv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (m < a.M) {
          const SRow sr = s_row<D>(a, m, c);
          float x[8], nsv[8];
          load_S8<D>(sr.s, sr.p, sr.q, (hk >> 3) + q, x);
          unpack8<D>(*(const uint4*)((const uint16_t*)a.ns + kg + 8 * q), nsv);
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = hnorm<D>(x[e], rinv_s[r], nsv[e]);
        }
        *(uint4*)(a_lds + r * PF_ALD + 8 * q) = pack8<D>(hv);
      }
      // [down | inject | 0] rows kg .. kg+31 into per-tile [32][16] LDS tiles.
      for (int i = tid; i < 32 * NP8; i += 256) {
        const int rr = i / NP8, j = i - rr * NP8, col8 = 8 * j;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (col8 + 8 <= a.R) v = *(const uint4*)(wd + (kg + rr) * a.R + col8);
        *(uint4*)(b_lds + (col8 >> 4) * 512 + rr * 16 + 8 * ((col8 >> 3) & 1)) = v;
      }
      const uint4 injw = inject_word(wi, a.C, kg, 32, tid);
      __syncthreads();  // the zero chunks of the inject tile are written
      inject_scatter(b_lds + (a.R >> 4) * 512, a.C, 32, tid, injw);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = wave + 4 * i;
        if (t < g.NT) {
          const s16x8 bf = lds_bfrag(b_lds + t * 512, 0, lane);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            sl[i][rt] = mfma<D>(lds_afrag(a_lds + rt * 16 * PF_ALD, PF_ALD, 0, lane), bf, sl[i][rt]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) br[i][rt] = br[i][rt] + sl[i][rt];
  }
  // Branch partials: bpart[c][m][n].
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + 4 * i;
    const int n = 16 * t + (lane & 15);
    if (t < g.NT && n < a.R + a.C) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + 16 * rt + 4 * (lane >> 4) + r;
          if (m < a.M) bpart[((int64_t)c * a.M + m) * g.NP + n] = br[i][rt][r];
        }
    }
  }
}

// up = hidden @ up_weight for 64 rows x 16 features of every branch (one wave
// per branch c, four row tiles), chunks of 32 along R, then the pre-mix.
template <DT D>
__global__ __launch_bounds__(512) void k_pf_uppre(Args a, const float* __restrict__ rinv,
                                                  const void* __restrict__ hidden) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int R = a.R, HLD = R + 8;
  uint16_t* hid_lds = (uint16_t*)smem;              // [64][R + 8]
  uint16_t* wu_lds = hid_lds + PF_BM * HLD;         // [C][32][16]
  float* e_lds = (float*)(wu_lds + a.C * 512);      // [C][64][16]
  const int tid = threadIdx.x, c = tid >> 6, lane = tid & 63;
  const int nthreads = blockDim.x;
  const int64_t m0 = (int64_t)blockIdx.x * PF_BM;
  const int h0 = blockIdx.y * 16;
  const int R8 = R >> 3;
  for (int i = tid; i < PF_BM * R8; i += nthreads) {
    const int r = i / R8, j = i - r * R8;
    const int64_t m = m0 + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (m < a.M) v = *(const uint4*)((const uint16_t*)hidden + m * R + 8 * j);
    *(uint4*)(hid_lds + r * HLD + 8 * j) = v;
  }
  const uint16_t* wu = (const uint16_t*)a.wu;
  f32x4 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < R; k0 += 32) {
    {
      const int n = k0 + (lane >> 1);
      *(uint4*)(wu_lds + c * 512 + (lane >> 1) * 16 + 8 * (lane & 1)) =
          *(const uint4*)(wu + (int64_t)n * a.K + (int64_t)c * a.H + h0 + 8 * (lane & 1));
    }
    __syncthreads();
    const s16x8 bf = lds_bfrag(wu_lds + c * 512, 0, lane);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      acc[rt] = mfma<D>(lds_afrag(hid_lds + rt * 16 * HLD, HLD, k0, lane), bf, acc[rt]);
    __syncthreads();
  }
  const int h = h0 + (lane & 15);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rt + 4 * (lane >> 4) + r;
      const int64_t m = m0 + row;
      float e = 0.0f;
      if (m < a.M) e = premix_term<D>(a, rinv, m, c, h, acc[rt][r]);
      e_lds[(c * PF_BM + row) * 16 + (lane & 15)] = e;
    }
  __syncthreads();
  for (int i = tid; i < PF_BM * 16; i += nthreads) {
    const int row = i >> 4, hh = i & 15;
    const int64_t m = m0 + row;
    if (m < a.M) {
      float sum = 0.0f;
      for (int cc = 0; cc < a.C; ++cc) sum = sum + e_lds[(cc * PF_BM + row) * 16 + hh];
      st<D>(a.pre, m * a.H + h0 + hh, rT<D>(a.rs * sum));
    }
  }
}

static size_t pf_uppre_lds_bytes(int C, int R) {
  return (size_t)PF_BM * (R + 8) * 2 + (size_t)C * 512 * 2 + (size_t)C * PF_BM * 16 * 4;
}

template <DT D, int TPW>
static void launch_pf_down(const Args& a, const Geometry& g, float* bpart, float* rinv, hipStream_t s) {
  const dim3 grid((unsigned)((a.M + PF_BM - 1) / PF_BM), (unsigned)a.C);
  hipLaunchKernelGGL((k_pf_down<D, TPW>), grid, dim3(256), 0, s, a, g, bpart, rinv);
}

template <DT D>
static hipError_t run_prefill(const Args& a, char* ws, const Workspace& w, const Geometry& g, hipStream_t s,
                              Marks* mk) {
  float* rinv = (float*)(ws + w.rinv);
  void* hidden = ws + w.hidden;
  float* bpart = (float*)(ws + w.partial);
  const int tpw = (g.NT + 3) / 4;
  const size_t lds = pf_uppre_lds_bytes(a.C, a.R);
  hipError_t e = allow_dynamic_lds((const void*)k_pf_uppre<D>, D == DT::BF16 ? 4 : 5, lds);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  switch (tpw) {
    case 1: launch_pf_down<D, 1>(a, g, bpart, rinv, s); break;
    case 2: launch_pf_down<D, 2>(a, g, bpart, rinv, s); break;
    case 3: launch_pf_down<D, 3>(a, g, bpart, rinv, s); break;
    case 4: launch_pf_down<D, 4>(a, g, bpart, rinv, s); break;
    case 5: launch_pf_down<D, 5>(a, g, bpart, rinv, s); break;
    case 6: launch_pf_down<D, 6>(a, g, bpart, rinv, s); break;
    case 7: launch_pf_down<D, 7>(a, g, bpart, rinv, s); break;
    case 8: launch_pf_down<D, 8>(a, g, bpart, rinv, s); break;
    case 9: launch_pf_down<D, 9>(a, g, bpart, rinv, s); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  e = launch_branch_reduce(a, (int)D, g.NP, bpart, hidden, s);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  const dim3 grid((unsigned)((a.M + PF_BM - 1) / PF_BM), (unsigned)(a.H / 16));
  hipLaunchKernelGGL(k_pf_uppre<D>, grid, dim3(64 * a.C), lds, s, a, (const float*)rinv, (const void*)hidden);
  if ((e = mark(mk, s)) != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_prefill(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                          hipStream_t s, Marks* mk) {
  if (dtype == 16) return run_prefill<DT::BF16>(a, ws, w, g, s, mk);
  if (dtype == 10) return run_prefill<DT::F16>(a, ws, w, g, s, mk);
  return hipErrorInvalidValue;
}

}  // namespace hc
