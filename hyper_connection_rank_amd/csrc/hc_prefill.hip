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

#include <algorithm>

namespace hc {

constexpr int PF_BM = 64;      // rows per workgroup (four 16-row matrix-core tiles)
constexpr int PF_ALD = 40;     // padded LDS row of an hn chunk (32 + 8 elements)
constexpr int PF_TPW = 3;      // [down | inject] output tiles per wave
constexpr int PF_TPG = 24;     // output tiles per column group (8 waves x PF_TPW)
constexpr int PF_RQ = 8;       // 16-byte chunks per lane of a row that pass 1 loads at once
constexpr int PF_BF = 64;      // features per pf_uppre workgroup
constexpr int PF_S = 4;        // stages of pf_down's load ring (chunks in flight: PF_S - 1); four arrays below
constexpr int PF_LPC = 6;      // loads each pf_down wave issues per chunk (a fixed count: see below)

typedef __attribute__((address_space(3))) void pf_lds_void;
typedef __attribute__((address_space(1))) void pf_glb_void;

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// lds_base + 16 l (lds_base the same in every lane).
__device__ __forceinline__ void pf_load_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((pf_glb_void*)src, (pf_lds_void*)lds_base, 16, 0, 0);
}

// Wait until at most N of this wave's vector memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));  // expcnt, lgkmcnt: no wait
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt(0)), not for its global loads: __syncthreads() also drains the
// load counter, which would empty the ring at every chunk. Loads that write
// LDS directly are covered by the explicit vmcnt waits around it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reads of a ring stage, written as assembly so that the compiler does not
// see LDS reads to order after the direct-to-LDS loads still filling the
// other stages (it would wait for every one of them before each read). The
// stage has been filled before these run: each wave has waited for its own
// loads of the chunk and the workgroup has met at a barrier. Each block waits
// for its own results (lgkmcnt(0)) before returning them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
__device__ __forceinline__ void ring_read3(const void* p0, const void* p1, const void* p2, u32x2& v0, u32x2& v1,
                                           u32x2& v2) {
  asm volatile(
      "ds_read_b64 %0, %3\n"
      "ds_read_b64 %1, %4\n"
      "ds_read_b64 %2, %5\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2))
      : "memory");
}
// B fragments of three 16-column tiles of 32 pitched rows (see
// lds_bfrag_pitched()).
__device__ __forceinline__ void ring_bfrag3(const void* rows, int pitch_bytes, int c0, int c1, int c2, int lane,
                                            s16x8& f0, s16x8& f1, s16x8& f2) {
  const int g = lane >> 4, j = lane & 15, r = j >> 2, cb = j & 3;
  const uint32_t base = lds_addr(rows) + (8 * g + r) * pitch_bytes + 8 * cb, hi = 4 * pitch_bytes;
  const uint32_t a0 = base + 2 * c0, a1 = base + 2 * c1, a2 = base + 2 * c2;
  u32x2 l0, h0, l1, h1, l2, h2;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %6\n"
      "ds_read_b64_tr_b16 %1, %7\n"
      "ds_read_b64_tr_b16 %2, %8\n"
      "ds_read_b64_tr_b16 %3, %9\n"
      "ds_read_b64_tr_b16 %4, %10\n"
      "ds_read_b64_tr_b16 %5, %11\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1), "=&v"(l2), "=&v"(h2)
      : "v"(a0), "v"(a0 + hi), "v"(a1), "v"(a1 + hi), "v"(a2), "v"(a2 + hi)
      : "memory");
  f0 = __builtin_bit_cast(s16x8, u32x4{l0.x, l0.y, h0.x, h0.y});
  f1 = __builtin_bit_cast(s16x8, u32x4{l1.x, l1.y, h1.x, h1.y});
  f2 = __builtin_bit_cast(s16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
}
// The inject tile's B fragment from the flat values [32][C] (see
// inject_bfrag()).
__device__ __forceinline__ s16x8 ring_inject_bfrag(const void* flat, int C, int lane) {
  const int col = min(lane & 15, C - 1), row0 = 8 * (lane >> 4);
  const uint32_t b = lds_addr(flat) + 2 * (row0 * C + col), st = 2 * C;
  uint32_t v0, v1, v2, v3, v4, v5, v6, v7;
  asm volatile(
      "ds_read_u16 %0, %8\n"
      "ds_read_u16 %1, %9\n"
      "ds_read_u16 %2, %10\n"
      "ds_read_u16 %3, %11\n"
      "ds_read_u16 %4, %12\n"
      "ds_read_u16 %5, %13\n"
      "ds_read_u16 %6, %14\n"
      "ds_read_u16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
      : "v"(b), "v"(b + st), "v"(b + 2 * st), "v"(b + 3 * st), "v"(b + 4 * st), "v"(b + 5 * st), "v"(b + 6 * st),
        "v"(b + 7 * st)
      : "memory");
  const uint32_t m = (lane & 15) < C ? 0xFFFFFFFFu : 0u;
  return __builtin_bit_cast(s16x8, u32x4{(v0 | (v1 << 16)) & m, (v2 | (v3 << 16)) & m, (v4 | (v5 << 16)) & m,
                                         (v6 | (v7 << 16)) & m});
}

// pf_down's LDS ring stage: the raw S chunk [64 rows][32] (and prev_out's
// [64][32] when S is rebuilt), the chunk's 32 norm_scale values, its inject
// values [32][C], and the weight rows [32][bp bytes] of this column group.
// The stages are separate static arrays, each step of the chunk loop bound to
// its stage at compile time, so the compiler can tell that a stage being read
// is not one that loads are still filling (with one array indexed at run time
// it waits for every load before every LDS read).
constexpr int PF_RING_RAW = 0, PF_RING_PRAW = 4096, PF_RING_NS = 8192, PF_RING_INJ = 8192 + 256,
              PF_RING_B = 8192 + 256 + 512;
constexpr int PF_BP_MAX = 832;  // pitch for PF_TPG tiles (768 bytes) rounded to an odd multiple of 64
constexpr int PF_STAGE = PF_RING_B + 32 * PF_BP_MAX;

// Weight row pitch for a column group: the group's down columns (bytes)
// rounded up to an odd multiple of 64, so that the four rows of a transposing
// read fall on different banks.
__host__ __device__ inline int pf_pitch(int R, int t_lo, int t_hi) {
  const int wbytes = (min(16 * t_hi, R) - 16 * t_lo) * 2;
  int bp = ((wbytes > 0 ? wbytes : 16) + 63) / 64 * 64;
  if ((bp / 64) % 2 == 0) bp += 64;
  return bp;
}

// --------------------------------------------------------------- pf_down

// FROM_SO: hn is rebuilt from streams_out (written in pass 1) instead of from
// streams, prev_block_output and prev_post_gate.
template <DT D, bool FROM_SO>
__global__ __launch_bounds__(512) void k_pf_down(Args a, Geometry g, float* __restrict__ bpart,
                                                 float* __restrict__ rinv_out) {
  __shared__ float rinv_s[PF_BM];
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][PF_BM * PF_ALD];
  __shared__ __attribute__((aligned(16))) unsigned char sink[64];  // target of the padding loads
  __shared__ __attribute__((aligned(16))) unsigned char ring0[PF_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[PF_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[PF_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[PF_STAGE];
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
  wait_vm_le<0>();  // streams_out of these rows is written before any wave reads it back
  __syncthreads();

  // ---- Pass 2. The branch's K range in chunks of 32, through a ring of
  //      PF_S LDS stages filled by direct global->LDS loads issued PF_S - 1
  //      chunks ahead. Every wave issues exactly PF_LPC loads per chunk (four
  //      weight rows, then one or two of: a quarter of the raw S chunk, a
  //      quarter of prev_out's, norm_scale, inject, or a one-lane padding
  //      load), so "this wave's loads of chunk ch are done" is "at most
  //      PF_LPC * (PF_S - 2) of its loads are pending".
  const int bp = pf_pitch(a.R, t_lo, t_hi);
  const int KSC = g.KS >> 5;  // chunks per slice
  const int nch = a.H >> 5;   // chunks of the branch
  const bool rebuild = !FROM_SO && pro;  // S = prologue(streams, gate, prev_out) again
  const int nbl = max((min(16 * t_hi, a.R) - 16 * t_lo) >> 3, 1);  // 16-byte pieces of a weight row
  const int t_inj = a.R >> 4;  // tile holding the inject columns
  const bool inj_here = t_inj >= t_lo && t_inj < t_hi;
  const int64_t kc0 = (int64_t)c * a.H;  // first row of the branch in K
  const uint16_t* wrow = (const uint16_t*)a.wd + kc0 * a.R + 16 * t_lo + 8 * min(lane, nbl - 1);
  const uint16_t* ssrc = (const uint16_t*)(FROM_SO ? a.streams_out : a.streams);
  const int arow = 16 * (wave & 3) + (lane >> 2);  // row of this lane's raw-S piece
  const uint16_t* araw = ssrc + (m0 + min(arow, M - 1)) * a.K + kc0 + 8 * (lane & 3);
  const uint16_t* praw = pro ? (const uint16_t*)a.prev_out + (m0 + min(arow, M - 1)) * a.H + 8 * (lane & 3) : araw;
  const uint16_t* nsrc = (const uint16_t*)a.ns + kc0 + 8 * min(lane, 3);
  const uint16_t* isrc = (const uint16_t*)a.wi + kc0 * a.C + 8 * min(lane, 4 * a.C - 1);
  auto stage = [&](auto J) -> unsigned char* {
    constexpr int j = decltype(J)::value % PF_S;
    return j == 0 ? ring0 : j == 1 ? ring1 : j == 2 ? ring2 : ring3;
  };
  auto issue = [&](unsigned char* st, int ch) {
    const int chv = min(ch, nch - 1);  // past the end: reload the last chunk (kept count, unused stage)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave + 8 * i;
      if (lane < nbl) pf_load_lds16(wrow + (int64_t)(32 * chv + row) * a.R, st + PF_RING_B + row * bp);
    }
    if (wave < 4) {
      pf_load_lds16(araw + 32 * chv, st + PF_RING_RAW + 1024 * wave);
    } else if (rebuild) {
      pf_load_lds16(praw + 32 * chv, st + PF_RING_PRAW + 1024 * (wave - 4));
    } else if (lane == 0) {
      pf_load_lds16(nsrc, sink);
    }
    if (wave == 0) {
      if (lane < 4) pf_load_lds16(nsrc + 32 * chv, st + PF_RING_NS);
    } else if (wave == 1 && inj_here) {
      if (lane < 4 * a.C) pf_load_lds16(isrc + (int64_t)32 * chv * a.C, st + PF_RING_INJ);
    } else if (lane == 0) {
      pf_load_lds16(nsrc, sink);
    }
  };

  // hn staging role: row hr of the tile, four k at 4 hq.
  const int hr = tid >> 3, hq = tid & 7;
  const float hgate = rebuild ? ld<D>(a.prev_gate, (m0 + min(hr, M - 1)) * a.C + c) : 0.0f;

  f32x4 sl[PF_TPW][4], br[PF_TPW][4];
#pragma unroll
  for (int i = 0; i < PF_TPW; ++i)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      sl[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      br[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  issue(stage(std::integral_constant<int, 0>{}), 0);
  issue(stage(std::integral_constant<int, 1>{}), 1);
  issue(stage(std::integral_constant<int, 2>{}), 2);
  // One chunk: J = ch % PF_S, known at compile time.
  auto step = [&](auto J, int ch) {
    unsigned char* st = stage(J);
    wait_vm_le<PF_LPC * (PF_S - 2)>();  // this wave's loads of chunk ch are in
    lds_barrier();                       // everyone's are; the stage of chunk ch - 1 is free
    issue(stage(std::integral_constant<int, decltype(J)::value + PF_S - 1>{}), ch + PF_S - 1);
    uint16_t* at = a_lds[decltype(J)::value & 1];
    {  // hn chunk [64][32] into a_lds, four values per thread
      float x[4], nsv[4], hv[4];
      u32x2 rs, rp, rn;
      ring_read3(st + PF_RING_RAW + hr * 64 + 8 * hq, st + PF_RING_PRAW + hr * 64 + 8 * hq,
                 st + PF_RING_NS + 8 * hq, rs, rp, rn);
      unpack4<D>(rs, x);
      if (rebuild) {
        float p[4];
        unpack4<D>(rp, p);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = prologue<D>(x[e], hgate, p[e]);
      }
      unpack4<D>(rn, nsv);
      const float rv = rinv_s[hr];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = hr < M ? hnorm_raw(x[e], rv, nsv[e]) : 0.0f;
      *(uint2*)(at + hr * PF_ALD + 4 * hq) = make_uint2(pack2<D>(hv[0], hv[1]), pack2<D>(hv[2], hv[3]));
    }
    lds_barrier();
    s16x8 af[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) af[rt] = lds_afrag(at + rt * 16 * PF_ALD, PF_ALD, 0, lane);
    s16x8 bf[PF_TPW];
    {  // this wave's tiles t_lo + wave + 8i (past the group or the inject tile: read tile 0, unused)
      int col[PF_TPW];
#pragma unroll
      for (int i = 0; i < PF_TPW; ++i) {
        const int t = t_lo + wave + 8 * i;
        col[i] = t < t_hi && t != t_inj ? 16 * (t - t_lo) : 0;
      }
      static_assert(PF_TPW == 3, "three fragments per read block");
      ring_bfrag3(st + PF_RING_B, bp, col[0], col[1], col[2], lane, bf[0], bf[1], bf[2]);
    }
#pragma unroll
    for (int i = 0; i < PF_TPW; ++i) {
      const int t = t_lo + wave + 8 * i;
      if (t == t_inj) bf[i] = ring_inject_bfrag(st + PF_RING_INJ, a.C, lane);
      if (t < t_hi) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) sl[i][rt] = mfma<D>(af[rt], bf[i], sl[i][rt]);
      }
    }
    if ((ch + 1) % KSC == 0) {  // slice done: add it to the branch sum
      asm volatile("");  // a real branch, not selects executed at every chunk
#pragma unroll
      for (int i = 0; i < PF_TPW; ++i)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          br[i][rt] = br[i][rt] + sl[i][rt];
          sl[i][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
  };
  for (int ch = 0; ch < nch; ch += PF_S) {  // nch is a multiple of PF_S or the tail steps are skipped
    step(std::integral_constant<int, 0>{}, ch);
    if (ch + 1 < nch) step(std::integral_constant<int, 1>{}, ch + 1);
    if (ch + 2 < nch) step(std::integral_constant<int, 2>{}, ch + 2);
    if (ch + 3 < nch) step(std::integral_constant<int, 3>{}, ch + 3);
  }
  wait_vm_le<0>();  // the reloads past the end have landed before the LDS goes away

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
        for (int e = 0; e < 8; e += 2) {  // pairs: one conversion rounds two values
          const float S0 = (!FROM_SO && pro) ? prologue<D>(x[e], q, p[e]) : x[e];
          const float S1 = (!FROM_SO && pro) ? prologue<D>(x[e + 1], q, p[e + 1]) : x[e + 1];
          float h0 = hnorm_raw(S0, erv[cc], nsv[e]), h1 = hnorm_raw(S1, erv[cc], nsv[e + 1]);
          rT2<D>(h0, h1);
          float g0 = up_gate_raw<D>(up[e]), g1 = up_gate_raw<D>(up[e + 1]);  // up is already T
          rT2<D>(g0, g1);
          sum[e] = sum[e] + h0 * g0;
          sum[e + 1] = sum[e + 1] + h1 * g1;
        }
      }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = a.rs * sum[e];
    *(uint4*)((uint16_t*)a.pre + em * a.H + eh) = pack8<D>(o);  // rounds pre_output to T
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
  const unsigned rows = (unsigned)((a.M + PF_BM - 1) / PF_BM), ncg = (unsigned)((g.NT + PF_TPG - 1) / PF_TPG);
  const dim3 gd(rows, (unsigned)a.C, ncg);
  // pf_down rebuilds hn from streams_out only when the workgroup wrote those
  // rows itself (one column group); other column groups recompute S.
  const bool so_down = from_so && ncg == 1;
  e = so_down ? launch(mk, k_pf_down<D, true>, gd, dim3(512), 0, s, a, g, bpart, rinv)
              : launch(mk, k_pf_down<D, false>, gd, dim3(512), 0, s, a, g, bpart, rinv);
  if (e != hipSuccess) return e;
  e = launch_branch_reduce(a, (int)D, g.NP, bpart, hidden, s, mk);
  if (e != hipSuccess) return e;
  const dim3 gu(rows, (unsigned)((a.H + PF_BF - 1) / PF_BF));
  const float* rv = rinv;
  const void* hd = hidden;
  if (a.C <= 4)
    return from_so ? launch(mk, k_pf_uppre<D, 4, true>, gu, dim3(512), lds, s, a, rv, hd)
                   : launch(mk, k_pf_uppre<D, 4, false>, gu, dim3(512), lds, s, a, rv, hd);
  return from_so ? launch(mk, k_pf_uppre<D, 8, true>, gu, dim3(512), lds, s, a, rv, hd)
                 : launch(mk, k_pf_uppre<D, 8, false>, gu, dim3(512), lds, s, a, rv, hd);
}

hipError_t launch_prefill(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                          hipStream_t s, Marks* mk) {
  if (dtype == 16) return run_prefill<DT::BF16>(a, ws, w, g, s, mk);
  if (dtype == 10) return run_prefill<DT::F16>(a, ws, w, g, s, mk);
  return hipErrorInvalidValue;
}

}  // namespace hc
