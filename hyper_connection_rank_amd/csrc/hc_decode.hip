// Decode path (at most 16 rows: one matrix-core row tile) of the
// HyperConnectionLowRankMix block on gfx950.
//
// The time goes into streaming the weights once from HBM (13.2 MB for
// 4 x 2560, rank 320, bf16) and into latency: a graph-launched kernel costs
// about 1.6 us on MI355X before it does anything, and one trip to memory
// about 1 us. So the block is two kernels, and every workgroup issues all of
// its global loads before it waits on any of them -- the small loads needed
// first, then the weight stream -- so the compiler's in-order load counters
// let the early work overlap the stream. Weights stay row-major [K, N] and
// are used in place (onnxruntime PR #33384, "Motivation and Context"); they
// are read with coalesced 16-byte loads, staged in LDS and turned into
// matrix-core fragments by transposing LDS reads.
//
//   hc_down   grid: K slice x 64-column tile group. Prologue and per-branch RMS
//             of every row (one wave per row), hn of its slice, one 16x16x32
//             matrix-core chain per 16 output columns of [down | inject], fp32
//             partial sums per slice.
//   hc_uppre  grid: 16 features, one wave per branch. For one or two rows each
//             workgroup adds the slice partials itself (fixed order) while its
//             up_weight loads are in flight; for more rows the last hc_down
//             workgroup of each tile group does it (an arrival counter) and
//             writes hidden. Then the up chain over R, sigmoid, hn and the
//             pre-mix over branches in ascending c.
//
// The split mirrors the PR's "CUDA implementation" (split-K partials, then a
// fixed-order consumer); where the consumer runs never changes the bits.
#include "hc_mfma_common.h"

namespace hc {

constexpr int KSMAX = 256;             // largest slice length
constexpr int HN_LD = KSMAX + 8;       // padded LDS row of hn (elements)
constexpr int MAXQ = 16;               // 8-element chunks per lane of one branch (H <= 8192)
constexpr int CMAX = 8;                // branches on the matrix-core paths
constexpr int K2_REDUCE_MAX_ROWS = 2;  // up to this many rows hc_uppre reduces the partials itself
constexpr int SB = 16;                 // slices whose partials one thread loads at once

// Agent-coherent (sc1) store and load: visible to workgroups on every XCD
// without writing back or invalidating a whole L2, which is what a
// device-scope fence costs on this chip (microseconds per workgroup).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const float* p) {
  return __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this thread's stores have completed (vmcnt(0)).
__device__ __forceinline__ void wait_stores() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// --------------------------------------------------------------- RMS, in two phases

struct RmsLoads {
  uint4 sv[MAXQ];  // streams chunks (lane's chunks L, L+64, ...)
  uint4 pv[MAXQ];  // prev_block_output chunks
  uint4 nsraw;     // norm_scale of the lane's chunk inside the slice, if any
  uint32_t qraw;   // prev_post_gate[m, c] (raw; widened where it is used)
};

// Issue the loads of (row m, branch c); [q_lo, q_hi) is the slice in chunks
// (fewer than 64 chunks, so a lane holds at most one of them).
template <DT D>
__device__ __forceinline__ void rms_issue(const Args& a, int64_t m, int c, int lane, int q_lo, int q_hi,
                                          RmsLoads& L) {
  const uint16_t* srow = (const uint16_t*)a.streams + m * a.K + (int64_t)c * a.H;
  const uint16_t* prow = a.prev_out ? (const uint16_t*)a.prev_out + m * a.H : nullptr;
#pragma unroll
  for (int i = 0; i < MAXQ; ++i) {
    const int q = lane + 64 * i;
    if (8 * q < a.H) {
      L.sv[i] = *(const uint4*)(srow + 8 * q);
      if (prow) L.pv[i] = *(const uint4*)(prow + 8 * q);
    }
  }
  const int i0 = q_lo > lane ? (q_lo - lane + 63) >> 6 : 0;
  const int qs = lane + 64 * i0;
  L.nsraw = make_uint4(0u, 0u, 0u, 0u);
  if (qs < q_hi && 8 * qs < a.H) L.nsraw = *(const uint4*)((const uint16_t*)a.ns + (int64_t)c * a.H + 8 * qs);
  L.qraw = ((const uint16_t*)(prow ? a.prev_gate : a.ns))[prow ? m * a.C + c : 0];
}

// Canonical sum of squares (lane L owns chunks L, L+64, ... in ascending h;
// see branch_sumsq()), rinv, then hn of the slice into hrow and optionally S
// of the slice to streams_out. Returns rinv.
template <DT D>
__device__ __forceinline__ float rms_finish(const Args& a, int64_t m, int c, int lane, int q_lo, int q_hi,
                                            const RmsLoads& L, uint16_t* hrow, bool write_so) {
  const bool pro = a.prev_out != nullptr;
  const float gate = widen<D>(L.qraw);
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXQ; ++i) {
    const int q = lane + 64 * i;
    if (8 * q < a.H) {
      float x[8];
      unpack8<D>(L.sv[i], x);
      if (pro) {
        float p[8];
        unpack8<D>(L.pv[i], p);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], gate, p[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ss + x[e] * x[e];
    }
  }
  const float rv = rinv_from_ss(wave_allsum(ss), a.H, a.eps);
  uint16_t* so = write_so ? (uint16_t*)a.streams_out + m * a.K + (int64_t)c * a.H : nullptr;
#pragma unroll
  for (int i = 0; i < MAXQ; ++i) {
    const int q = lane + 64 * i;
    if (8 * q < a.H && q >= q_lo && q < q_hi) {
      float x[8], nsv[8], hv[8];
      unpack8<D>(L.sv[i], x);
      if (pro) {
        float p[8];
        unpack8<D>(L.pv[i], p);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], gate, p[e]);
      }
      if (so) *(uint4*)(so + 8 * q) = pack8<D>(x);
      unpack8<D>(L.nsraw, nsv);  // q is this lane's slice chunk
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = hnorm<D>(x[e], rv, nsv[e]);
      *(uint4*)(hrow + 8 * (q - q_lo)) = pack8<D>(hv);
    }
  }
  return rv;
}

// --------------------------------------------------------------- hc_down

template <DT D, bool TICKET>
__global__ __launch_bounds__(256) void k_hc_down(Args a, Geometry g, float* __restrict__ partial,
                                                 float* __restrict__ rinv_out, void* __restrict__ hidden,
                                                 unsigned* __restrict__ tickets) {
  __shared__ __attribute__((aligned(16))) uint16_t hn_lds[16 * HN_LD];
  __shared__ __attribute__((aligned(16))) uint16_t w_lds[4 * KSMAX * 16];
  __shared__ float br_lds[TICKET ? 16 * CMAX * 64 : 1];
  __shared__ int is_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NG = (g.NT + 3) >> 2;
  const int s = blockIdx.x / NG, b = blockIdx.x - s * NG;
  const int c = s / g.SPB, s_in = s - c * g.SPB;
  const int KS = g.KS, h_lo = s_in * KS, q_lo = h_lo >> 3, q_hi = (h_lo + KS) >> 3;
  const int64_t kbase = (int64_t)c * a.H + h_lo;
  const bool write_so = b == 0 && a.streams_out != nullptr;

  // 1. The RMS inputs of this wave's first row: small, needed first.
  RmsLoads L;
  if (wave < a.M) rms_issue<D>(a, wave, c, lane, q_lo, q_hi, L);

  // 2. The weight tile: rows kbase .. kbase+KS of columns [64b, 64b+64) of
  //    [down | inject | 0], eight threads per row, 16 bytes each. The inject
  //    columns (C <= 8 from column R) are KS*C contiguous values of
  //    inject_weight, loaded as flat words by the workgroup that holds R.
  uint4 wreg[KSMAX / 32];
  const int col8 = 64 * b + 8 * (tid & 7);
  const uint16_t* wd = (const uint16_t*)a.wd;
#pragma unroll
  for (int p = 0; p < KSMAX / 32; ++p) {
    const int rr = 32 * p + (tid >> 3);
    wreg[p] = make_uint4(0u, 0u, 0u, 0u);
    if (rr < KS && col8 + 8 <= a.R) wreg[p] = *(const uint4*)(wd + (kbase + rr) * a.R + col8);
  }
  const bool inj_wg = a.R >= 64 * b && a.R < 64 * b + 64;
  const uint4 injw = inj_wg ? inject_word((const uint16_t*)a.wi, a.C, kbase, KS, tid) : make_uint4(0u, 0u, 0u, 0u);

  // 3. RMS of each row (one wave per row); hn of this slice into LDS.
  for (int r = wave; r < 16; r += 4) {
    uint16_t* hrow = hn_lds + r * HN_LD;
    if (r >= a.M) {
      for (int i = lane; i < KS / 8; i += 64) *(uint4*)(hrow + 8 * i) = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    if (r != wave) rms_issue<D>(a, r, c, lane, q_lo, q_hi, L);
    const float rv = rms_finish<D>(a, r, c, lane, q_lo, q_hi, L, hrow, write_so);
    if (b == 0 && s_in == 0 && lane == 0) rinv_out[r * a.C + c] = rv;
  }

  // 4. Weights to LDS, one [KS][16] tile per wave.
#pragma unroll
  for (int p = 0; p < KSMAX / 32; ++p) {
    const int rr = 32 * p + (tid >> 3);
    if (rr < KS) {
      const int j = tid & 7;
      *(uint4*)(w_lds + (j >> 1) * (KSMAX * 16) + rr * 16 + 8 * (j & 1)) = wreg[p];
    }
  }
  if (inj_wg) {
    __syncthreads();  // the zero chunks of the inject tile are in place
    inject_scatter(w_lds + ((a.R - 64 * b) >> 4) * (KSMAX * 16), a.C, KS, tid, injw);
  }
  __syncthreads();

  // 5. One matrix-core chain over the slice for output tile t = 4b + wave.
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
        const int m = 4 * (lane >> 4) + r;
        if (m >= a.M) continue;
        float* dst = partial + ((int64_t)s * a.M + m) * g.NP + n;
        if (TICKET) st_agent(dst, acc[r]);
        else *dst = acc[r];
      }
    }
  }
  if (!TICKET) return;

  // 6. Arrival counter: the last of the NS slice workgroups of tile group b
  //    adds the partials. They went out as agent-coherent stores; once those
  //    have completed, one relaxed device-scope increment publishes them.
  wait_stores();
  __syncthreads();
  unsigned* ticket = tickets + b;
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(g.NS - 1);
  __syncthreads();
  if (!is_last) return;
  const int rows = (int)a.M;
  // Branch sums (slices ascending) for item = (row, branch, column pair);
  // four items per thread with every load issued before the additions.
  const int items = rows * a.C * 32;
  const int64_t step = a.M * g.NP;
  for (int it0 = tid; it0 < items; it0 += 4 * 256) {
    uint64_t v[4][SB];
    float2 br[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) br[u] = make_float2(0.0f, 0.0f);
    for (int s0 = 0; s0 < g.SPB; s0 += SB) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int it = it0 + 256 * u;
        const int np = it & 31, rc = it >> 5, r = rc / a.C, cc = rc - r * a.C;
        const int n = 64 * b + 2 * np;
        const bool ok = it < items && n < a.R + a.C;
        const float* p = partial + (((int64_t)cc * g.SPB) * a.M + r) * g.NP + n;
#pragma unroll
        for (int i = 0; i < SB; ++i) v[u][i] = (ok && s0 + i < g.SPB) ? ld_agent64(p + (s0 + i) * step) : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (s0 + i < g.SPB) {
            br[u].x = br[u].x + __uint_as_float((uint32_t)v[u][i]);
            br[u].y = br[u].y + __uint_as_float((uint32_t)(v[u][i] >> 32));
          }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = it0 + 256 * u;
      if (it < items) {
        const int np = it & 31, rc = it >> 5, r = rc / a.C, cc = rc - r * a.C;
        br_lds[(r * CMAX + cc) * 64 + 2 * np] = br[u].x;
        br_lds[(r * CMAX + cc) * 64 + 2 * np + 1] = br[u].y;
      }
    }
  }
  __syncthreads();
  for (int it = tid; it < rows * 64; it += 256) {
    const int r = it >> 6, nl = it & 63, n = 64 * b + nl;
    if (n < a.R + a.C) {
      float tot = 0.0f;
      for (int cc = 0; cc < a.C; ++cc) tot = tot + br_lds[(r * CMAX + cc) * 64 + nl];
      finish_down_inject<D>(a, r, n, tot, hidden);
    }
  }
  if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // zero for the next call
}

// --------------------------------------------------------------- hc_uppre

constexpr int HIDMAX = 16;  // hidden chunks per thread (16 rows x R/8 chunks over 64*C threads)

template <DT D, bool REDUCE>
__global__ __launch_bounds__(512) void k_hc_uppre(Args a, Geometry g, const float* __restrict__ rinv,
                                                  const void* __restrict__ hidden,
                                                  const float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int R = a.R, HLD = R + 8, R8 = R >> 3;
  uint16_t* hid_lds = (uint16_t*)smem;                 // [16][R + 8]
  uint16_t* wu_lds = hid_lds + 16 * HLD;               // [C][R][16]
  float* e_lds = (float*)(wu_lds + a.C * R * 16);      // [C][16][16]
  float* br_lds = e_lds + a.C * 256;                   // [rows][C][NP] (REDUCE only)
  const int tid = threadIdx.x, c = tid >> 6, lane = tid & 63;
  const int nthreads = blockDim.x;
  // Workgroups on one XCD (blockIdx.x mod 8) take adjacent feature blocks, so
  // the 128-byte lines of up_weight they share come from HBM once per XCD.
  const int nhb = a.H >> 4;
  const int hb = (nhb & 7) == 0 ? (int)(blockIdx.x & 7) * (nhb >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int h0 = hb * 16, h = h0 + (lane & 15);
  const int64_t kc = (int64_t)c * a.H + h;

  // 1. Inputs of hn for this lane's four outputs (rows 4*(lane/16) + r).
  //    Loads are unconditional (rows clamped into the batch, and without a
  //    prologue they re-read streams), so no branch merges a loaded register;
  //    values of rows beyond the batch are never stored.
  const bool from_so = a.streams_out != nullptr, pro = !from_so && a.prev_out != nullptr;
  const uint16_t* sp = (const uint16_t*)(from_so ? a.streams_out : a.streams);
  const uint16_t* pp = (const uint16_t*)(pro ? a.prev_out : a.streams);
  const uint16_t* qp = (const uint16_t*)(pro ? a.prev_gate : a.streams);
  uint32_t sraw[4], praw[4], qraw[4];
  float rvv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t m = min(4 * (lane >> 4) + r, (int)a.M - 1);
    sraw[r] = sp[m * a.K + kc];
    praw[r] = pp[pro ? m * a.H + h : m * a.K + kc];
    qraw[r] = qp[pro ? m * a.C + c : m * a.K + kc];
    rvv[r] = rinv[m * a.C + c];
  }
  const uint32_t nsraw = ((const uint16_t*)a.ns)[kc];

  // 2. Either the slice partials of this thread's first item (REDUCE; item =
  //    row, branch, 8 columns) or its chunks of the hidden tile.
  const int NP8 = g.NP >> 3;
  const int items = REDUCE ? (int)a.M * a.C * NP8 : 0;
  const int64_t step = a.M * g.NP;
  float4 pv[SB][2];
  uint4 hreg[HIDMAX];
  if (REDUCE) {
    const int it = min(tid, items - 1);  // clamped: every thread loads a valid item
    const int j8 = it % NP8, rc = it / NP8, r = rc / a.C, cc = rc - r * a.C;
    const float* p = partial + (((int64_t)cc * g.SPB) * a.M + r) * g.NP + 8 * j8;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (i < g.SPB) {
        pv[i][0] = *(const float4*)(p + i * step);
        pv[i][1] = *(const float4*)(p + i * step + 4);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < HIDMAX; ++i) {
      const int ch = min(tid + i * nthreads, 16 * R8 - 1), r = min(ch / R8, (int)a.M - 1), j = ch % R8;
      if (i * nthreads < 16 * R8) hreg[i] = *(const uint4*)((const uint16_t*)hidden + (int64_t)r * R + 8 * j);
    }
  }

  // 3. The up_weight tile of branch c: rows 0..R-1, columns c*H + h0 .. +16.
  uint4 wreg[16];
  const uint16_t* wu = (const uint16_t*)a.wu;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int n = 32 * p + (lane >> 1);
    wreg[p] = make_uint4(0u, 0u, 0u, 0u);
    if (n < R) wreg[p] = *(const uint4*)(wu + (int64_t)n * a.K + (int64_t)c * a.H + h0 + 8 * (lane & 1));
  }

  // 4. hn (independent of up), exactly as S_at / hnorm compute it.
  float hnv[4];
  const float nsv = widen<D>(nsraw);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float S = widen<D>(sraw[r]);
    if (pro) S = prologue<D>(S, widen<D>(qraw[r]), widen<D>(praw[r]));
    hnv[r] = hnorm<D>(S, rvv[r], nsv);
  }

  // 5. The hidden tile [16][R] in LDS (rows beyond the batch zero).
  if (!REDUCE) {
#pragma unroll
    for (int i = 0; i < HIDMAX; ++i) {
      const int ch = tid + i * nthreads, r = ch / R8, j = ch - r * R8;
      if (i * nthreads < 16 * R8 && ch < 16 * R8)
        *(uint4*)(hid_lds + r * HLD + 8 * j) = r < a.M ? hreg[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    const int rows = (int)a.M;
    for (int it = tid; it < items; it += nthreads) {
      const int j8 = it % NP8, rc = it / NP8, r = rc / a.C, cc = rc - r * a.C;
      const float* p = partial + (((int64_t)cc * g.SPB) * a.M + r) * g.NP + 8 * j8;
      float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      for (int s0 = 0; s0 < g.SPB; s0 += SB) {
        if (it != tid || s0 != 0) {  // the first batch of the first item is already loaded
#pragma unroll
          for (int i = 0; i < SB; ++i) {
            const bool ok = s0 + i < g.SPB;
            pv[i][0] = ok ? *(const float4*)(p + (s0 + i) * step) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            pv[i][1] = ok ? *(const float4*)(p + (s0 + i) * step + 4) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          }
        }
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (s0 + i < g.SPB) {
            sum[0] = sum[0] + pv[i][0].x; sum[1] = sum[1] + pv[i][0].y;
            sum[2] = sum[2] + pv[i][0].z; sum[3] = sum[3] + pv[i][0].w;
            sum[4] = sum[4] + pv[i][1].x; sum[5] = sum[5] + pv[i][1].y;
            sum[6] = sum[6] + pv[i][1].z; sum[7] = sum[7] + pv[i][1].w;
          }
      }
      float* dst = br_lds + (r * a.C + cc) * g.NP + 8 * j8;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = sum[e];
    }
    for (int i = tid; i < 16 * R8; i += nthreads) {
      const int r = i / R8, j = i - r * R8;
      if (r >= rows) *(uint4*)(hid_lds + r * HLD + 8 * j) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    // Totals over branches (ascending); ScaledSiLU into the hidden tile;
    // workgroup 0 also writes post_gate.
    for (int i = tid; i < rows * (R + a.C); i += nthreads) {
      const int r = i / (R + a.C), n = i - r * (R + a.C);
      float tot = 0.0f;
      for (int cc = 0; cc < a.C; ++cc) tot = tot + br_lds[(r * a.C + cc) * g.NP + n];
      if (n < R) hid_lds[r * HLD + n] = (uint16_t)to_bits<D>(scaled_silu<D>(rT<D>(tot), a.alpha));
      else if (blockIdx.x == 0) finish_down_inject<D>(a, r, n, tot, nullptr);
    }
  }

  // 6. up_weight to LDS; the up chain; g; the pre-mix over branches.
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int n = 32 * p + (lane >> 1);
    if (n < R) *(uint4*)(wu_lds + ((int64_t)c * R + n) * 16 + 8 * (lane & 1)) = wreg[p];
  }
  __syncthreads();
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* tile = wu_lds + c * R * 16;
  for (int k0 = 0; k0 < R; k0 += 32)
    acc = mfma<D>(lds_afrag(hid_lds, HLD, k0, lane), lds_bfrag(tile, k0, lane), acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 4 * (lane >> 4) + r;
    e_lds[c * 256 + rr * 16 + (lane & 15)] = hnv[r] * up_gate<D>(acc[r]);
  }
  __syncthreads();
  for (int i = tid; i < 256; i += nthreads) {
    const int rr = i >> 4, hh = i & 15;
    if (rr < a.M) {
      float sum = 0.0f;
      for (int cc = 0; cc < a.C; ++cc) sum = sum + e_lds[cc * 256 + i];
      st<D>(a.pre, (int64_t)rr * a.H + h0 + hh, rT<D>(a.rs * sum));
    }
  }
}

// --------------------------------------------------------------- prefill helper

// Fixed-order reduction of per-branch fp32 partials [C][M][NP] (one partial
// per branch, each already summed over its slices in order) + the down/inject
// epilogue. Used by the prefill path.
template <DT D>
__global__ __launch_bounds__(256) void k_branch_reduce(Args a, int NP, const float* __restrict__ partial,
                                                       void* __restrict__ hidden) {
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  if (n >= a.R + a.C) return;
  for (int64_t m = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6); m < a.M; m += (int64_t)gridDim.y * 4) {
    float v[CMAX];
#pragma unroll
    for (int cc = 0; cc < CMAX; ++cc) v[cc] = cc < a.C ? partial[((int64_t)cc * a.M + m) * NP + n] : 0.0f;
    float tot = 0.0f;
#pragma unroll
    for (int cc = 0; cc < CMAX; ++cc)
      if (cc < a.C) tot = tot + v[cc];
    finish_down_inject<D>(a, m, n, tot, hidden);
  }
}

// --------------------------------------------------------------- launchers

size_t uppre_lds_bytes(int C, int R) {
  return (size_t)16 * (R + 8) * 2 + (size_t)C * R * 16 * 2 + (size_t)C * 256 * 4;
}

static size_t uppre_reduce_lds_bytes(int C, int R, int NP, int rows) {
  return uppre_lds_bytes(C, R) + (size_t)rows * C * NP * 4;
}

// hc_uppre adds the partials itself for one or two rows (when its LDS allows).
static bool k2_reduces(const Args& a, const Geometry& g) {
  return a.M <= K2_REDUCE_MAX_ROWS && uppre_reduce_lds_bytes(a.C, a.R, g.NP, (int)a.M) <= 160 * 1024;
}

template <DT D>
static hipError_t run_decode(const Args& a, char* ws, const Workspace& w, const Geometry& g, hipStream_t s,
                             Marks* mk) {
  float* rinv = (float*)(ws + w.rinv);
  void* hidden = ws + w.hidden;
  float* partial = (float*)(ws + w.partial);
  unsigned* tickets = (unsigned*)(ws + w.tickets);
  const int NG = (g.NT + 3) / 4;
  const bool k2r = k2_reduces(a, g);
  const size_t lds = k2r ? uppre_reduce_lds_bytes(a.C, a.R, g.NP, (int)a.M) : uppre_lds_bytes(a.C, a.R);
  const int slot = (D == DT::BF16 ? 0 : 1) + (k2r ? 2 : 0);
  const void* k2 = k2r ? (const void*)k_hc_uppre<D, true> : (const void*)k_hc_uppre<D, false>;
  hipError_t e = allow_dynamic_lds(k2, slot, lds);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  const dim3 g1((unsigned)(g.NS * NG)), g2((unsigned)(a.H / 16));
  if (k2r) {
    hipLaunchKernelGGL((k_hc_down<D, false>), g1, dim3(256), 0, s, a, g, partial, rinv, hidden, tickets);
    if ((e = mark(mk, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_hc_uppre<D, true>), g2, dim3(64 * a.C), lds, s, a, g, (const float*)rinv,
                       (const void*)hidden, (const float*)partial);
  } else {
    hipLaunchKernelGGL((k_hc_down<D, true>), g1, dim3(256), 0, s, a, g, partial, rinv, hidden, tickets);
    if ((e = mark(mk, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_hc_uppre<D, false>), g2, dim3(64 * a.C), lds, s, a, g, (const float*)rinv,
                       (const void*)hidden, (const float*)partial);
  }
  if ((e = mark(mk, s)) != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_decode(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                         hipStream_t s, Marks* mk) {
  if (a.M > 16) return hipErrorInvalidValue;
  if (dtype == 16) return run_decode<DT::BF16>(a, ws, w, g, s, mk);
  if (dtype == 10) return run_decode<DT::F16>(a, ws, w, g, s, mk);
  return hipErrorInvalidValue;
}

hipError_t launch_branch_reduce(const Args& a, int dtype, int NP, const float* partial, void* hidden,
                                hipStream_t s) {
  const int64_t mq = (a.M + 3) / 4;
  const dim3 grid((unsigned)((a.R + a.C + 63) / 64), (unsigned)(mq < 65535 ? mq : 65535));
  if (dtype == 16) hipLaunchKernelGGL(k_branch_reduce<DT::BF16>, grid, dim3(256), 0, s, a, NP, partial, hidden);
  else if (dtype == 10) hipLaunchKernelGGL(k_branch_reduce<DT::F16>, grid, dim3(256), 0, s, a, NP, partial, hidden);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hc
