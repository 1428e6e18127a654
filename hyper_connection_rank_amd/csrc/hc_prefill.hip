// Prefill path (many rows) of the HyperConnectionLowRankMix block on gfx950:
// down/inject and up become dense GEMMs on the matrix cores (the general path
// of onnxruntime PR #33384, "CUDA implementation", done with our own kernels
// and always with fp32 accumulation).
//
//   pf_down   grid (64-row tile, branch c, column group). Pass 1: the branch
//             sum of squares of its rows (two rows in flight per wave),
//             rinv, streams_out. Pass 2: hn @ [down | inject] over the
//             branch's K range in double-buffered chunks of 32; one 16x16x32
//             matrix-core chain per slice, slices added in order; one fp32
//             partial per branch. Two workgroups fit a CU, so one streams its
//             rows while the other keeps the matrix cores busy.
//   branch_reduce  adds the branch partials in ascending c and applies
//             ScaledSiLU / the inject gate (the decode path's order: slices
//             within a branch, then branches).
//   pf_uppre  grid (64-row tile, 64 features). up = hidden @ up_weight for
//             every branch of those features (chunks of 32 along R), rounded
//             to T into LDS; then per 8 features of a row: hn recomputed,
//             sigmoid, the pre-mix over branches in ascending c.
//
// Every arithmetic step is the same function, in the same order, as in the
// decode kernels, so a row's bits match the decode path's.
#include "hc_mfma_common.h"

namespace hc {

constexpr int PF_BM = 64;      // rows per workgroup (four 16-row matrix-core tiles)
constexpr int PF_ALD = 40;     // padded LDS row of an hn chunk (32 + 8 elements)
constexpr int PF_TPW = 3;      // [down | inject] output tiles per wave
constexpr int PF_TPG = 24;     // output tiles per column group (8 waves x PF_TPW)
constexpr int PF_RQ = 8;       // 16-byte chunks per lane of a row that pass 1 loads at once
constexpr int PF_BITEMS = 3;   // weight chunks per thread per k-chunk (PF_TPG * 2 * 32 / 512)
constexpr int PF_BF = 64;      // features per pf_uppre workgroup

// --------------------------------------------------------------- pf_down

// FROM_SO: hn is rebuilt from streams_out (written in pass 1) instead of from
// streams, prev_block_output and prev_post_gate.
template <DT D, bool FROM_SO>
__global__ __launch_bounds__(512) void k_pf_down(Args a, Geometry g, float* __restrict__ bpart,
                                                 float* __restrict__ rinv_out) {
  __shared__ float rinv_s[PF_BM];
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][PF_BM * PF_ALD];
  __shared__ __attribute__((aligned(16))) uint16_t b_lds[2][PF_TPG * 32 * 16];
  __shared__ __attribute__((aligned(16))) uint16_t inj_lds[2][32 * 8];  // inject values [32][C] of a chunk
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c = blockIdx.y, cg = blockIdx.z;
  const int64_t m0 = (int64_t)blockIdx.x * PF_BM;
  const int M = (int)min((int64_t)PF_BM, a.M - m0);  // rows of this tile
  const bool pro = a.prev_out != nullptr;
  const int t_lo = PF_TPG * cg, t_hi = min(g.NT, t_lo + PF_TPG);  // this group's output tiles

  // ---- Pass 1: rows 2*wave + 16i and 2*wave + 16i + 1 of the tile, every
  //      load of both rows issued before either is used. Lane L plays the
  //      virtual lanes L + 64 q (chunk L + 64 t falls in quarter t mod 4).
  const int NQ = a.H >> 3;
  for (int rp = 2 * wave; rp < PF_BM; rp += 16) {
    float acc[2][4] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    float gate[2];
    const uint16_t* sr[2];
    const uint16_t* pr[2];
    uint16_t* so[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t m = m0 + min(rp + u, M - 1);
      sr[u] = (const uint16_t*)a.streams + m * a.K + (int64_t)c * a.H;
      pr[u] = pro ? (const uint16_t*)a.prev_out + m * a.H : sr[u];
      gate[u] = pro ? ld<D>(a.prev_gate, m * a.C + c) : 0.0f;
      so[u] = a.streams_out && cg == 0 && rp + u < M ? (uint16_t*)a.streams_out + m * a.K + (int64_t)c * a.H
                                                     : nullptr;
    }
    for (int t0 = 0; 64 * t0 < NQ; t0 += PF_RQ) {
      uint4 sv[2][PF_RQ], pv[2][PF_RQ];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < PF_RQ; ++i) {
          const int q = min(lane + 64 * (t0 + i), NQ - 1);
          sv[u][i] = *(const uint4*)(sr[u] + 8 * q);
          if (pro) pv[u][i] = *(const uint4*)(pr[u] + 8 * q);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < PF_RQ; ++i) {
          const int q = lane + 64 * (t0 + i);
          if (q < NQ) {
            float x[8];
            unpack8<D>(sv[u][i], x);
            if (pro) {
              float p[8];
              unpack8<D>(pv[u][i], p);
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], gate[u], p[e]);
            }
            if (so[u]) *(uint4*)(so[u] + 8 * q) = pack8<D>(x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[u][(t0 + i) & 3] = acc[u][(t0 + i) & 3] + x[e] * x[e];
          }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float ss = ss_combine(wave_allsum(acc[u][0]), wave_allsum(acc[u][1]), wave_allsum(acc[u][2]),
                                  wave_allsum(acc[u][3]));
      const float rv = rinv_from_ss(ss, a.H, a.eps);
      if (lane == 0) {
        rinv_s[rp + u] = rv;
        if (cg == 0 && rp + u < M) rinv_out[(m0 + rp + u) * a.C + c] = rv;
      }
    }
  }
  __syncthreads();

  // ---- Pass 2. Per k-chunk of 32: hn [64 rows][32] (threads 0..255: row
  //      tid/4, eight k) and the weight rows [32][this group's columns] go through
  //      registers into one of two LDS buffers; the next chunk's loads are in
  //      flight while the matrix cores work on this one.
  const int KSC = g.KS >> 5;  // chunks per slice
  const int nch = a.H >> 5;   // chunks of the branch
  const int hr = (tid & 255) >> 2, hq = tid & 3;
  const int64_t hm = m0 + min(hr, M - 1);
  const uint16_t* hs = (const uint16_t*)(FROM_SO ? a.streams_out : a.streams) + hm * a.K + (int64_t)c * a.H + 8 * hq;
  const uint16_t* hp = pro ? (const uint16_t*)a.prev_out + hm * a.H + 8 * hq : hs;
  const float hgate = (!FROM_SO && pro) ? ld<D>(a.prev_gate, hm * a.C + c) : 0.0f;
  const uint16_t* hns = (const uint16_t*)a.ns + (int64_t)c * a.H + 8 * hq;
  // Weight chunks of this thread: item idx = tid + 256 i -> row rr = idx / ncw,
  // 8-column chunk j = idx % ncw of the group's columns below R.
  const int ncw = (min(16 * t_hi, a.R) - 16 * t_lo) >> 3;  // 8-column chunks below R in this group
  int b_goff[PF_BITEMS], b_loff[PF_BITEMS];
#pragma unroll
  for (int i = 0; i < PF_BITEMS; ++i) {
    const int idx = tid + 512 * i;
    const int rr = ncw > 0 ? idx / ncw : 0, j = ncw > 0 ? idx - rr * ncw : 0;
    const bool ok = ncw > 0 && rr < 32;
    b_goff[i] = ok ? rr * a.R + 16 * t_lo + 8 * j : -1;
    b_loff[i] = ok ? (j >> 1) * 512 + rr * 16 + 8 * (j & 1) : 0;
  }
  const int t_inj = a.R >> 4;  // tile holding the inject columns
  const bool inj_here = t_inj >= t_lo && t_inj < t_hi;
  const uint16_t* wd = (const uint16_t*)a.wd + (int64_t)c * a.H * a.R;
  const uint16_t* wi = (const uint16_t*)a.wi + (int64_t)c * a.H * a.C;

  // The inject values of a chunk's 32 rows are 32*C contiguous values: 4C
  // flat 16-byte words (threads past the last word load it again).
  const int iw_idx = min(tid, 4 * a.C - 1);
  // Staging registers are native vectors: arrays of the uint4 struct carried
  // across loop iterations end up in scratch memory.
  u32x4 sa, pa, na, wb[PF_BITEMS], iw;
  const bool a_wave = wave < 4;  // waves 0..3 build the hn chunk
  auto fetch = [&](int ch) {
    if (a_wave) {
      sa = *(const u32x4*)(hs + 32 * ch);
      if (!FROM_SO && pro) pa = *(const u32x4*)(hp + 32 * ch);
      na = *(const u32x4*)(hns + 32 * ch);
    }
#pragma unroll
    for (int i = 0; i < PF_BITEMS; ++i)
      wb[i] = *(const u32x4*)(wd + (int64_t)32 * ch * a.R + max(b_goff[i], 0));
    if (inj_here) iw = *(const u32x4*)(wi + (int64_t)32 * ch * a.C + 8 * iw_idx);
  };

  f32x4 sl[PF_TPW][4], br[PF_TPW][4];
#pragma unroll
  for (int i = 0; i < PF_TPW; ++i)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      sl[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      br[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  fetch(0);
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    if (a_wave) {  // stage the hn chunk
      float x[8], nsv[8], hv[8];
      unpack8<D>(to_uint4(sa), x);
      if (!FROM_SO && pro) {
        float p[8];
        unpack8<D>(to_uint4(pa), p);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], hgate, p[e]);
      }
      unpack8<D>(to_uint4(na), nsv);
      const float rv = rinv_s[hr];
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = hr < M ? hnorm<D>(x[e], rv, nsv[e]) : 0.0f;
      *(uint4*)(a_lds[buf] + hr * PF_ALD + 8 * hq) = pack8<D>(hv);
    }
    {  // stage the weight chunk
#pragma unroll
      for (int i = 0; i < PF_BITEMS; ++i)
        if (b_goff[i] >= 0) *(u32x4*)(b_lds[buf] + b_loff[i]) = wb[i];
      if (inj_here && tid < 4 * a.C) *(u32x4*)(inj_lds[buf] + 8 * tid) = iw;
    }
    __syncthreads();
    fetch(min(ch + 1, nch - 1));  // unconditional (the last one reloads): the staging registers stay registers
    s16x8 af[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) af[rt] = lds_afrag(a_lds[buf] + rt * 16 * PF_ALD, PF_ALD, 0, lane);
#pragma unroll
    for (int i = 0; i < PF_TPW; ++i) {
      const int t = t_lo + wave + 8 * i;
      if (t < t_hi) {
        const s16x8 bf = t == t_inj ? inject_bfrag(inj_lds[buf], a.C, lane) : lds_bfrag(b_lds[buf] + (t - t_lo) * 512, 0, lane);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) sl[i][rt] = mfma<D>(af[rt], bf, sl[i][rt]);
      }
    }
    if ((ch + 1) % KSC == 0) {  // slice done: add it to the branch sum
#pragma unroll
      for (int i = 0; i < PF_TPW; ++i)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          br[i][rt] = br[i][rt] + sl[i][rt];
          sl[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
  }

  // Branch partials: bpart[c][m][n].
#pragma unroll
  for (int i = 0; i < PF_TPW; ++i) {
    const int t = t_lo + wave + 8 * i;
    const int n = 16 * t + (lane & 15);
    if (t < t_hi && n < a.R + a.C) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * (lane >> 4) + r;
          if (row < M) bpart[((int64_t)c * a.M + m0 + row) * g.NP + n] = br[i][rt][r];
        }
    }
  }
}

// --------------------------------------------------------------- pf_uppre

// LDS: hidden tile [64][R + 8], then the up_weight chunks [2][C * 4 tiles]
// [32][16], later reused for up rounded to T [64][C][64].
static size_t pf_uppre_lds_bytes(int C, int R) {
  const size_t wu = (size_t)2 * C * 4 * 512 * 2, up = (size_t)PF_BM * C * PF_BF * 2;
  return (size_t)PF_BM * (R + 8) * 2 + (wu > up ? wu : up);
}

constexpr int PF_HV = 8;  // hidden chunks per thread (64 rows x R/8 <= 64 chunks over 512 threads)

// Eight waves: wave w takes features 16 (w % 4) .. +16 of the block and row
// tiles 2 (w / 4), 2 (w / 4) + 1, for every branch. CB: branches the
// registers are sized for (4 or 8).
template <DT D, int CB, bool FROM_SO>
__global__ __launch_bounds__(512) void k_pf_uppre(Args a, const float* __restrict__ rinv,
                                                  const void* __restrict__ hidden) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int R = a.R, HLD = R + 8, R8 = R >> 3, C = a.C;
  uint16_t* hid_lds = (uint16_t*)smem;       // [64][R + 8]
  uint16_t* wu_lds = hid_lds + PF_BM * HLD;  // [2][C*4][32][16]
  uint16_t* up_lds = wu_lds;                 // [64][C][64] after the chain
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ft = wave & 3, rg = wave >> 2;  // feature tile, row-tile pair
  const int64_t m0 = (int64_t)blockIdx.x * PF_BM;
  const int M = (int)min((int64_t)PF_BM, a.M - m0);
  const int f0 = blockIdx.y * PF_BF;
  const bool pro = a.prev_out != nullptr;

  // Epilogue inputs of this thread's item: row er, features eh .. eh+7.
  const int er = tid >> 3, eh = f0 + 8 * (tid & 7);
  const bool e_ok = er < M && eh < a.H;
  const int64_t em = m0 + min(er, M - 1);
  const int ehc = min(eh, a.H - 8);
  uint4 es[CB], ens[CB], ep;
  uint32_t eg[CB];
  float erv[CB];
  auto load_epilogue = [&]() {
#pragma unroll
    for (int cc = 0; cc < CB; ++cc) {
      const int c = min(cc, C - 1);
      es[cc] = *(const uint4*)((const uint16_t*)(FROM_SO ? a.streams_out : a.streams) + em * a.K +
                               (int64_t)c * a.H + ehc);
      ens[cc] = *(const uint4*)((const uint16_t*)a.ns + (int64_t)c * a.H + ehc);
      eg[cc] = (!FROM_SO && pro) ? ((const uint16_t*)a.prev_gate)[em * C + c] : 0u;
      erv[cc] = rinv[em * C + c];
    }
    if (!FROM_SO && pro) ep = *(const uint4*)((const uint16_t*)a.prev_out + em * a.H + ehc);
  };
  // With up to four branches the epilogue inputs are issued first and used
  // last; with more, their registers go to the accumulators until then.
  constexpr bool EPI_EARLY = CB <= 4;
  if (EPI_EARLY) load_epilogue();

  // The hidden tile [64][R]: every chunk of this thread loaded before any is
  // stored (rows past the batch zero).
  const int hchunks = PF_BM * R8;
  uint4 hv[PF_HV];
#pragma unroll
  for (int i = 0; i < PF_HV; ++i) {
    const int ch = min(tid + 512 * i, hchunks - 1), r = ch / R8;
    hv[i] = *(const uint4*)((const uint16_t*)hidden + (m0 + min(r, M - 1)) * R + 8 * (ch - r * R8));
  }

  // Up chain. Chunk: up_weight rows k0 .. k0+31, for each branch the 64
  // features (four 16-column tiles) in whole 128-byte rows; item idx = tid +
  // 512 i -> row idx / (8C), branch and 8-feature chunk idx % (8C).
  const uint16_t* wu = (const uint16_t*)a.wu;
  const int nwi = 32 * 8 * C;  // 16-byte chunks per k-chunk
  int w_goff[CB / 2], w_loff[CB / 2];
#pragma unroll
  for (int i = 0; i < CB / 2; ++i) {
    const int idx = tid + 512 * i, ic = min(idx, nwi - 1);
    const int rr = ic / (8 * C), cj = ic - rr * 8 * C, c = cj >> 3, j = cj & 7;
    w_goff[i] = rr * a.K + c * a.H + min(f0 + 8 * j, a.H - 8);
    w_loff[i] = idx < nwi ? (c * 4 + (j >> 1)) * 512 + rr * 16 + 8 * (j & 1) : -1;
  }
  u32x4 wr[CB / 2];
#pragma unroll
  for (int i = 0; i < CB / 2; ++i) wr[i] = *(const u32x4*)(wu + w_goff[i]);
  f32x4 acc[CB][2];
#pragma unroll
  for (int cc = 0; cc < CB; ++cc)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) acc[cc][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const bool tile_ok = f0 + 16 * ft < a.H;  // this wave's 16 features exist
#pragma unroll
  for (int i = 0; i < PF_HV; ++i) {
    const int ch = tid + 512 * i, r = ch / R8;
    if (ch < hchunks) *(uint4*)(hid_lds + r * HLD + 8 * (ch - r * R8)) = r < M ? hv[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int k0 = 0; k0 < R; k0 += 32) {
    uint16_t* wb = wu_lds + ((k0 >> 5) & 1) * (C * 4 * 512);
#pragma unroll
    for (int i = 0; i < CB / 2; ++i)
      if (w_loff[i] >= 0) *(u32x4*)(wb + w_loff[i]) = wr[i];
    __syncthreads();
    {  // next chunk (unconditional, the last one reloads: the staging registers stay registers)
      const int64_t kn = (int64_t)min(k0 + 32, R - 32) * a.K;
#pragma unroll
      for (int i = 0; i < CB / 2; ++i) wr[i] = *(const u32x4*)(wu + kn + w_goff[i]);
    }
    if (tile_ok) {
      s16x8 af[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) af[rt] = lds_afrag(hid_lds + (2 * rg + rt) * 16 * HLD, HLD, k0, lane);
#pragma unroll
      for (int cc = 0; cc < CB; ++cc)
        if (cc < C) {
          const s16x8 bf = lds_bfrag(wb + (cc * 4 + ft) * 512, 0, lane);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) acc[cc][rt] = mfma<D>(af[rt], bf, acc[cc][rt]);
        }
    }
  }
  if (!EPI_EARLY) load_epilogue();
  __syncthreads();  // every wave is done with the up_weight chunks
  // up rounded to T: up_lds[row][c][feature].
  if (tile_ok) {
#pragma unroll
    for (int cc = 0; cc < CB; ++cc)
      if (cc < C) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * (2 * rg + rt) + 4 * (lane >> 4) + r;
            up_lds[(row * C + cc) * PF_BF + 16 * ft + (lane & 15)] = (uint16_t)to_bits<D>(acc[cc][rt][r]);
          }
      }
  }
  __syncthreads();

  // Epilogue: pre[m][h .. h+7] = rT(rs * sum_c hn_c * g_c), c ascending.
  if (e_ok) {
    float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float p[8];
    if (!FROM_SO && pro) unpack8<D>(ep, p);
#pragma unroll
    for (int cc = 0; cc < CB; ++cc)
      if (cc < C) {
        float x[8], nsv[8], up[8];
        unpack8<D>(es[cc], x);
        unpack8<D>(ens[cc], nsv);
        unpack8<D>(*(const uint4*)(up_lds + (er * C + cc) * PF_BF + (eh - f0)), up);
        const float q = widen<D>(eg[cc]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float S = (!FROM_SO && pro) ? prologue<D>(x[e], q, p[e]) : x[e];
          const float hn = hnorm<D>(S, erv[cc], nsv[e]);
          sum[e] = sum[e] + hn * up_gate<D>(up[e]);
        }
      }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = rT<D>(a.rs * sum[e]);
    *(uint4*)((uint16_t*)a.pre + em * a.H + eh) = pack8<D>(o);
  }
}

// --------------------------------------------------------------- launchers

template <DT D>
static hipError_t run_prefill(const Args& a, char* ws, const Workspace& w, const Geometry& g, hipStream_t s,
                              Marks* mk) {
  float* rinv = (float*)(ws + w.rinv);
  void* hidden = ws + w.hidden;
  float* bpart = (float*)(ws + w.partial);
  const bool from_so = a.streams_out != nullptr;
  const size_t lds = pf_uppre_lds_bytes(a.C, a.R);
  const void* ku = a.C <= 4 ? (from_so ? (const void*)k_pf_uppre<D, 4, true> : (const void*)k_pf_uppre<D, 4, false>)
                            : (from_so ? (const void*)k_pf_uppre<D, 8, true> : (const void*)k_pf_uppre<D, 8, false>);
  const int slot = 4 + (D == DT::BF16 ? 0 : 1) * 4 + (a.C <= 4 ? 0 : 2) + (from_so ? 0 : 1);
  hipError_t e = allow_dynamic_lds(ku, slot, lds);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  const unsigned rows = (unsigned)((a.M + PF_BM - 1) / PF_BM), ncg = (unsigned)((g.NT + PF_TPG - 1) / PF_TPG);
  const dim3 gd(rows, (unsigned)a.C, ncg);
  // pf_down rebuilds hn from streams_out only when the workgroup wrote those
  // rows itself (one column group); other column groups recompute S.
  if (from_so && ncg == 1) hipLaunchKernelGGL((k_pf_down<D, true>), gd, dim3(512), 0, s, a, g, bpart, rinv);
  else hipLaunchKernelGGL((k_pf_down<D, false>), gd, dim3(512), 0, s, a, g, bpart, rinv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  e = launch_branch_reduce(a, (int)D, g.NP, bpart, hidden, s);
  if (e != hipSuccess) return e;
  if ((e = mark(mk, s)) != hipSuccess) return e;
  const dim3 gu(rows, (unsigned)((a.H + PF_BF - 1) / PF_BF));
  if (a.C <= 4) {
    if (from_so) hipLaunchKernelGGL((k_pf_uppre<D, 4, true>), gu, dim3(512), lds, s, a, (const float*)rinv, (const void*)hidden);
    else hipLaunchKernelGGL((k_pf_uppre<D, 4, false>), gu, dim3(512), lds, s, a, (const float*)rinv, (const void*)hidden);
  } else {
    if (from_so) hipLaunchKernelGGL((k_pf_uppre<D, 8, true>), gu, dim3(512), lds, s, a, (const float*)rinv, (const void*)hidden);
    else hipLaunchKernelGGL((k_pf_uppre<D, 8, false>), gu, dim3(512), lds, s, a, (const float*)rinv, (const void*)hidden);
  }
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
