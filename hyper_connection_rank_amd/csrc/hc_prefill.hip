// Prefill path (many rows) of the HyperConnectionLowRankMix block on gfx950:
// down/inject and up become dense GEMMs on the matrix cores (the general path
// of onnxruntime PR #33384, "CUDA implementation", done with our own kernels
// and always with fp32 accumulation).
//
//   pf_rms    one wave per (row, branch): S (prologue), streams_out, the
//             canonical sum of squares and rinv.
//   pf_down   grid (128-row tile, branch c, column group), eight waves.
//             hn @ [down | inject] over the branch's K range in chunks of 32
//             through a ring of LDS stages; one 16x16x32 matrix-core chain
//             per slice, slices added in order; one fp32 partial per branch.
//             With few rows (prefill_slices) a workgroup takes one slice
//             and writes that slice's chain instead.
//   pf_dfew   slice mode with few rows: one workgroup per (64 rows, slice,
//             64 columns), the decode kernel's chains, the same partials.
//   branch_reduce  adds the branch partials in ascending c and applies
//             ScaledSiLU / the inject gate (the decode path's order: slices
//             within a branch, then branches); slice_reduce does the same
//             from per-slice partials.
//   pf_prep + pf_up2  (bf16, more than 512 rows, C in {1,2,4,8})
//             up_weight transposed and the sigmoid table, then a persistent
//             kernel: up = hidden @ up_weight on the matrix cores, sigmoid
//             and the pre-mix over branches. After a branch-partial down
//             pass, the branch reduction and pf_prep share one launch
//             (reduce_prep, their workgroups interleaved).
//   pf_upb + pf_premix  (at most 128 rows) up per (64 features, branch)
//             workgroup with fp32 products hn * g in the workspace, then the
//             pre-mix adds them in ascending c.
//   pf_uppre  the same for other shapes and row counts: grid (64-row tile,
//             64 features).
//
// Every arithmetic step is the same function, in the same order, as in the
// decode kernels, so a row's bits match the decode path's.
#include "hc_mfma_common.h"

#include <algorithm>
#include <type_traits>

namespace hc {

constexpr int PF_BM = 64;      // rows per pf_uppre workgroup (four 16-row matrix-core tiles)
constexpr int PF_BF = 64;      // features per pf_uppre workgroup

typedef __attribute__((address_space(3))) void pf_lds_void;
typedef __attribute__((address_space(1))) void pf_glb_void;

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// lds_base + 16 l (lds_base the same in every lane).
__device__ __forceinline__ void pf_load_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((pf_glb_void*)src, (pf_lds_void*)lds_base, 16, 0, 0);
}

// A buffer descriptor of `bytes` bytes from `base` (raw, no stride), and 16
// bytes per lane from it straight into LDS: lane l writes lds_base + 16 l
// (lds_base the same in every lane), from base + voff (per lane) + soff (the
// same in every lane: read from the first active lane, so that the compiler
// never wraps the load in a loop over distinct values when soff went through
// a vector register on a divergent path).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pf_desc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void pf_bload(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (pf_lds_void*)lds_base, 16, voff, __builtin_amdgcn_readfirstlane(soff), 0,
                                           0);
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// ---- LDS access by assembly. The ring below is filled by direct
// global->LDS loads that the compiler cannot tell apart from the stage being
// read, so it would wait for every one of them before each LDS access. These
// helpers only issue the access; a later lgkm_tie*() waits for it and hands
// the registers on, so nothing reads them before the data is in.
__device__ __forceinline__ u32x4 lds_rd128(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ u32x2 lds_rdtr(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_rdu16(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
template <int OFF> __device__ __forceinline__ u32x4 lds_rd128o(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
  return v;
}
template <int OFF> __device__ __forceinline__ u32x2 lds_rdtro(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
  return v;
}
template <int OFF> __device__ __forceinline__ void lds_wr128o(uint32_t base, u32x4 v) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(base), "v"(v), "n"(OFF) : "memory");
}
// Calls f(integral_constant<int, I>) for I = B .. E-1 (compile-time loop).
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
__device__ __forceinline__ void lds_wr128(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// s_waitcnt lgkmcnt(N) that also redefines the given registers.
template <int N> __device__ __forceinline__ void lgkm_tie(u32x4& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N) : "memory");
}
template <int N> __device__ __forceinline__ void lgkm_tie(u32x4& x, u32x4& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "n"(N) : "memory");
}
template <int N> __device__ __forceinline__ void lgkm_tie(u32x4& x, u32x4& y, u32x4& z, u32x4& w) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(x), "+v"(y), "+v"(z), "+v"(w) : "n"(N) : "memory");
}
template <int N> __device__ __forceinline__ void lgkm_tie(u32x2* b) {  // ten B-fragment halves
  asm volatile("s_waitcnt lgkmcnt(%10)"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7]),
                 "+v"(b[8]), "+v"(b[9])
               : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_tie(uint32_t& w0, uint32_t& w1, uint32_t& w2, uint32_t& w3, u32x4& x, u32x4& y) {
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3), "+v"(x), "+v"(y)
               : "n"(N)
               : "memory");
}
template <int N> __device__ __forceinline__ void lgkm_tie8(uint32_t* v) {  // eight inject halfwords
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
               : "n"(N)
               : "memory");
}

// Weight row pitch for a column group: the group's down columns (bytes)
// rounded up to an odd multiple of 64, so that the four rows of a transposing
// read fall on different banks.
__host__ __device__ inline int pf_pitch(int R, int t_lo, int t_hi) {
  const int wbytes = (min(16 * t_hi, R) - 16 * t_lo) * 2;
  int bp = ((wbytes > 0 ? wbytes : 16) + 63) / 64 * 64;
  if ((bp / 64) % 2 == 0) bp += 64;
  return bp;
}

// --------------------------------------------------------------- pf_rms

// One wave per (row, branch): S (prologue), streams_out, the canonical sum of
// squares and rinv. Lane L holds chunks L + 64 t (t ascending), which belong
// to quarter t mod 4 of the 256 virtual lanes; a batch's loads are all issued
// before any is used.
constexpr int PR_T = 8;  // chunks per lane per batch
template <DT D>
__global__ __launch_bounds__(256) void k_pf_rms(Args a, float* __restrict__ rinv) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.M * a.C) return;  // wave-uniform
  const int64_t m = pair / a.C;
  const int c = (int)(pair - m * a.C);
  const bool pro = a.prev_out != nullptr;
  const uint16_t* sr = (const uint16_t*)a.streams + m * a.K + (int64_t)c * a.H;
  const uint16_t* pr = pro ? (const uint16_t*)a.prev_out + m * a.H : sr;
  const float q = pro ? ld<D>(a.prev_gate, m * a.C + c) : 0.0f;
  uint16_t* so = a.streams_out ? (uint16_t*)a.streams_out + m * a.K + (int64_t)c * a.H : nullptr;
  const int NQ = a.H >> 3;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0 = 0; 64 * t0 < NQ; t0 += PR_T) {
    u32x4 sv[PR_T], pv[PR_T];
#pragma unroll
    for (int i = 0; i < PR_T; ++i) {
      const int ch = min(lane + 64 * (t0 + i), NQ - 1);
      sv[i] = *(const u32x4*)(sr + 8 * ch);
      if (pro) pv[i] = *(const u32x4*)(pr + 8 * ch);
    }
#pragma unroll
    for (int i = 0; i < PR_T; ++i) {
      const int ch = lane + 64 * (t0 + i);
      if (ch < NQ) {
        float x[8];
        unpack8<D>(to_uint4(sv[i]), x);
        if (pro) {
          float p[8];
          unpack8<D>(to_uint4(pv[i]), p);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], q, p[e]);
        }
        if (so) *(uint4*)(so + 8 * ch) = pack8<D>(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i & 3] = acc[i & 3] + x[e] * x[e];
      }
    }
  }
  const float ss = ss_combine(wave_allsum(acc[0]), wave_allsum(acc[1]), wave_allsum(acc[2]), wave_allsum(acc[3]));
  if (lane == 0) rinv[m * a.C + c] = rinv_from_ss(ss, a.Hn, a.eps);
}

// --------------------------------------------------------------- pf_down

constexpr int PD_BM = 128;             // rows per workgroup
constexpr int PD_NCW = 5;              // down tiles per wave
constexpr int PD_TPG = 4 * PD_NCW;     // down tiles per column group
constexpr int PD_HLD = 80;             // bytes per hn row in the double buffer (32 values + 8 pad)
constexpr int PD_BP = 704;             // largest weight row pitch (20 tiles: 640 bytes -> odd multiple of 64)
constexpr int PD_RAW = 0;              // raw S chunk [128][64 bytes]

// hn @ [down | inject] for a tile of 128 rows and one branch c, over the
// branch's K range in chunks of 32. Per chunk, through a ring of LDS stages
// filled by direct global->LDS loads: the raw S chunk [128][32], the weight
// rows [32][group columns], the inject rows [32][C] and the chunk's 32
// norm_scale values (one copy per wave). Each wave loads exactly the raw rows
// its own threads turn into hn, and its own norm_scale copy, so it builds hn
// of the next chunk (into the other half of a double buffer) as soon as its
// own loads are in, after issuing this chunk's matrix-core work: one barrier
// per chunk. One chain per slice and 16x16 tile, slices added in order into
// the branch total: the decode path's order.
//
// Eight waves, two per SIMD, so that one wave's waits are partly covered by
// the other's matrix work. Wave w takes row tiles 4 (w >> 2) .. +3 and down
// tiles t_lo + (w & 3) + 4j (j < 5), and the inject tile of row tile w. It
// loads raw rows 16 w .. 16 w + 15, four of the chunk's 32 weight rows and its
// own norm_scale copy, and turns exactly those raw rows into hn. No register
// is pinned to a file, so the compiler keeps every accumulator in the vector
// file, which at 512 threads gives each wave 256 registers.
template <bool REB> struct PdStage {
  static constexpr int PRAW = 8192;                   // raw prev_out chunk (REB only)
  static constexpr int NS = REB ? 16384 : 8192;       // norm_scale [8 waves][32]
  static constexpr int INJ = NS + 512;                // inject rows [32][C], C <= 8
  static constexpr int B = INJ + 512;                 // weight rows [32][bp]
  static constexpr int BYTES = B + 32 * PD_BP;
  static constexpr int STAGES = REB ? 3 : 4;
  static constexpr int LOADS = 4 + 1 + (REB ? 1 : 0) + 1 + 1;  // direct loads per wave per chunk
};

// nsl: slices of a branch the grid's y dimension spreads (1: a workgroup
// takes the branch's whole K range and writes one partial per branch; the
// slice count: a workgroup takes one slice and writes that slice's chain).
template <DT D, bool REB>
__global__ __launch_bounds__(512) void k_pf_down(Args a, Geometry g, const float* __restrict__ rinv,
                                                  float* __restrict__ bpart, int nsl) {
  using SG = PdStage<REB>;
  constexpr int S = SG::STAGES, L = SG::LOADS;
  constexpr int CR = REB ? 3 : 2;  // conversion reads per chunk
  __shared__ __attribute__((aligned(16))) unsigned char ring[S * SG::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char hbuf[2 * PD_BM * PD_HLD];
  __shared__ __attribute__((aligned(16))) unsigned char zero16[16];  // inject columns >= C read this
  __shared__ __attribute__((aligned(16))) unsigned char sink[64];    // target of the padding loads
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int sy = blockIdx.y, c = sy / nsl, cg = blockIdx.z;  // partial index sy = c nsl + slice
  const int rh = wave >> 2, cq = wave & 3;
  const int64_t m0 = (int64_t)blockIdx.x * PD_BM;
  const int M = (int)min((int64_t)PD_BM, a.M - m0);
  const int NDT = a.R >> 4;  // down tiles
  const int t_lo = PD_TPG * cg, t_hi = min(NDT, t_lo + PD_TPG);
  const bool inj_here = cg == 0;
  const int bp = pf_pitch(a.R, t_lo, t_hi);
  const int nbl = 2 * (t_hi - t_lo);  // 16-byte pieces of a weight row
  const int KSC = g.KS >> 5, nch = nsl == 1 ? a.H >> 5 : KSC;
  const int64_t kc0 = (int64_t)c * a.H + (int64_t)(sy - c * nsl) * g.KS;  // first K of this workgroup
  const uint16_t* ssrc = (const uint16_t*)(REB || !a.streams_out ? a.streams : a.streams_out);
  if (tid < 4) ((uint32_t*)zero16)[tid] = 0u;

  const uint32_t ring0 = lds_addr(ring), hb0 = lds_addr(hbuf);
  constexpr int HB = PD_BM * PD_HLD;  // bytes of one hn buffer half

  // ---- direct loads of one chunk (exactly L per wave; every one has at
  //      least one active lane), through buffer descriptors of the
  //      workgroup's sources: per-lane offsets are fixed for the kernel and a
  //      chunk moves only the scalar offset, so a chunk's loads cost no vector
  //      address arithmetic. (The launcher takes this kernel only where every
  //      extent below fits 31 bits.)
  const uint32_t lw = 16u * (uint32_t)min(lane, nbl - 1);
  const uint32_t lr = (uint32_t)min(16 * wave + (lane >> 2), M - 1);  // this lane's raw row in the tile
  const uint32_t ls = lr * (uint32_t)a.K * 2u + 16u * (uint32_t)(lane & 3);
  const uint32_t lp = REB ? lr * (uint32_t)a.H * 2u + 16u * (uint32_t)(lane & 3) : 0u;
  const uint32_t ln = 16u * (uint32_t)min(lane, 3);
  const uint32_t li = 16u * (uint32_t)min(lane, 4 * a.C - 1);
  const int64_t k_end = kc0 + (int64_t)32 * nch;  // one past the workgroup's last K
  const auto rw = pf_desc((const char*)a.wd + (kc0 * a.R + 16 * t_lo) * 2, (k_end - kc0) * a.R * 2);
  const auto rs = pf_desc((const char*)ssrc + (m0 * a.K + kc0) * 2, (int64_t)M * a.K * 2);
  const auto rp = pf_desc((const char*)a.prev_out + (REB ? (m0 * a.H + (kc0 - (int64_t)c * a.H)) * 2 : 0),
                       REB ? (int64_t)M * a.H * 2 : 16);  // branch-relative
  const auto rn = pf_desc((const char*)a.ns + kc0 * 2, (k_end - kc0) * 2);
  const auto ri = pf_desc((const char*)a.wi + kc0 * a.C * 2, (k_end - kc0) * a.C * 2);
  auto issue = [&](int j, int ch) {
    unsigned char* st = ring + j * SG::BYTES;
    const uint32_t chv = (uint32_t)min(ch, nch - 1);  // past the end: reload the last chunk (same count, unused stage)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave + 8 * i;
      if (lane < nbl) pf_bload(rw, st + SG::B + row * bp, lw, (32u * chv + (uint32_t)row) * (uint32_t)a.R * 2u);
    }
    pf_bload(rs, st + PD_RAW + 1024 * wave, ls, 64u * chv);
    if (REB) pf_bload(rp, st + SG::PRAW + 1024 * wave, lp, 64u * chv);
    if (lane < 4) pf_bload(rn, st + SG::NS + 64 * wave, ln, 64u * chv);
    if (wave == 0) {
      if (lane < 4 * a.C) pf_bload(ri, st + SG::INJ, li, 64u * chv * (uint32_t)a.C);
    } else if (lane == 0) {
      pf_bload(rn, sink, 0u, 0u);
    }
  };

  // ---- LDS addresses of this lane
  struct LdsOffs {
    uint32_t a, b, c, n, w, i, i_stage, i_step;
  };
  auto lds_offs = [&]() {
    const int t = tid, fg = lane >> 4, fj = lane & 15, hr = t >> 2, hq = t & 3;
    LdsOffs o;
    o.a = hb0 + (uint32_t)((64 * rh + fj) * PD_HLD + 16 * fg);                             // A frag, first row tile
    o.b = ring0 + SG::B + (uint32_t)((8 * fg + (fj >> 2)) * bp + 8 * (fj & 3) + 32 * cq);  // B frag, tile t_lo + cq
    o.c = ring0 + PD_RAW + (uint32_t)(hr * 64 + 16 * hq);                                  // raw S (+PRAW: prev_out)
    o.n = ring0 + SG::NS + (uint32_t)(64 * wave + 16 * hq);                                // norm_scale copy
    o.w = hb0 + (uint32_t)(hr * PD_HLD + 16 * hq);                                         // hn write
    o.i = fj < a.C ? ring0 + SG::INJ + (uint32_t)(2 * (8 * fg * a.C + fj)) : lds_addr(zero16);
    o.i_stage = fj < a.C ? (uint32_t)SG::BYTES : 0u;
    o.i_step = fj < a.C ? (uint32_t)(2 * a.C) : 0u;
    return o;
  };
  const uint32_t b_hi = 4u * (uint32_t)bp;  // second half of a B frag (wave-uniform)
  const LdsOffs lo = lds_offs();

  // hn builder: thread tid takes row tid / 4 (one of this wave's raw rows), values 8 (tid & 3) .. +7
  const int64_t hm = m0 + min(tid >> 2, M - 1);
  const float rv = rinv[hm * a.C + c];
  const float hgate = REB ? ld<D>(a.prev_gate, hm * a.C + c) : 0.0f;
  struct ConvIn {
    u32x4 s, n, p;
  };
  auto conv_issue = [&](const LdsOffs& o, int j, ConvIn& r) {  // CR reads
    const uint32_t cs = o.c + j * SG::BYTES;
    r.s = lds_rd128o<0>(cs);
    r.n = lds_rd128o<0>(o.n + j * SG::BYTES);
    if (REB) r.p = lds_rd128o<SG::PRAW - PD_RAW>(cs);
  };
  auto conv_finish = [&](const LdsOffs& o, ConvIn& r, int b) {  // reads complete (caller waits); 1 write
    float x[8], nsv[8], hv[8];
    unpack8<D>(to_uint4(r.s), x);
    unpack8<D>(to_uint4(r.n), nsv);
    if (REB) {
      float p[8];
      unpack8<D>(to_uint4(r.p), p);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], hgate, p[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = hnorm_raw(x[e], rv, nsv[e]);
    lds_wr128o<0>(o.w + b * HB, to_u32x4(pack8<D>(hv)));
  };

  f32x4 sl[4][PD_NCW], br[4][PD_NCW], sli, bri;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < PD_NCW; ++j) br[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bri = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Prologue: chunks 0 .. S-2 in flight; hn of chunk 0 into half 0.
#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(j, j);
  wait_vm_le<L * (S - 2)>();  // this wave's loads of chunk 0
  {
    const LdsOffs& o = lo;
    ConvIn r;
    conv_issue(o, 0, r);
    lgkm_tie<0>(r.s, r.n);
    if (REB) lgkm_tie<0>(r.p);
    conv_finish(o, r, 0);
  }

  // One chunk, in stage J = ch % S. At the barrier every wave has its loads of
  // chunk ch in and has written its rows of hn(ch); the stage of chunk ch - 1
  // is free for chunk ch + S - 1. FIRST: the chunk starts a slice.
  const f32x4 z4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto step = [&](auto FC, int ch) {
    constexpr bool FIRST = decltype(FC)::value;
    const int J = ch % S, J1 = J + 1 == S ? 0 : J + 1;
    lds_barrier();
    issue(J == 0 ? S - 1 : J - 1, ch + S - 1);
    const LdsOffs& o = lo;
    const uint32_t ab = o.a + (ch & 1) * HB;
    const uint32_t bb = o.b + J * SG::BYTES, bbh = bb + b_hi;
    // Reads, oldest first: B x10, A0 .. A3. LDS operations complete in order,
    // so "at most n outstanding" names exactly which are in.
    u32x2 bh[2 * PD_NCW];
    static_for<0, PD_NCW>([&](auto JC) {
      constexpr int j = decltype(JC)::value;
      bh[2 * j] = lds_rdtro<128 * j>(bb);
      bh[2 * j + 1] = lds_rdtro<128 * j>(bbh);
    });
    u32x4 af[4];
    af[0] = lds_rd128o<0>(ab);
    af[1] = lds_rd128o<16 * PD_HLD>(ab);
    af[2] = lds_rd128o<2 * 16 * PD_HLD>(ab);
    af[3] = lds_rd128o<3 * 16 * PD_HLD>(ab);
    s16x8 bf[PD_NCW];
    ConvIn cv;
    static_for<0, 4>([&](auto IC) {
      constexpr int i = decltype(IC)::value;
      if constexpr (i == 0) {
        lgkm_tie<3>(bh);  // A1 .. A3 may remain
        lgkm_tie<3>(af[0]);
#pragma unroll
        for (int j = 0; j < PD_NCW; ++j)
          bf[j] = __builtin_bit_cast(s16x8, u32x4{bh[2 * j].x, bh[2 * j].y, bh[2 * j + 1].x, bh[2 * j + 1].y});
      } else {
        lgkm_tie<3 - i + CR>(af[i]);  // A(i+1) .. A3, then the conversion reads
      }
      const s16x8 av = __builtin_bit_cast(s16x8, af[i]);
#pragma unroll
      for (int j = 0; j < PD_NCW; ++j)  // a tile past the group computes unused values
        sl[i][j] = mfma<D>(av, bf[j], FIRST ? z4 : sl[i][j]);
      if constexpr (i == 0) {
        wait_vm_le<L * (S - 2)>();  // this wave's loads of chunk ch + 1
        conv_issue(o, J1, cv);
      }
    });
    // Inject tile of row tile `wave` (unused outside column group 0): its A
    // fragment is this wave's own A fragment cq (row tile 4 rh + cq = wave);
    // the B fragment is eight zero-extending halfword loads, packed in pairs
    // once they are in.
    uint32_t iw[8];
    const u32x4 ai = cq == 0 ? af[0] : cq == 1 ? af[1] : cq == 2 ? af[2] : af[3];
    {
      const uint32_t ad = o.i + J * o.i_stage;
#pragma unroll
      for (int e = 0; e < 8; ++e) iw[e] = lds_rdu16(ad + e * o.i_step);
    }
    // The conversion reads are older than these 8: at most 8 outstanding
    // means they are in.
    lgkm_tie<8>(cv.s, cv.n);
    if (REB) lgkm_tie<8>(cv.p);
    conv_finish(o, cv, (ch + 1) & 1);  // 1 write
    lgkm_tie8<0>(iw);
    {
      const s16x8 bi = __builtin_bit_cast(
          s16x8, u32x4{iw[0] | (iw[1] << 16), iw[2] | (iw[3] << 16), iw[4] | (iw[5] << 16), iw[6] | (iw[7] << 16)});
      sli = mfma<D>(__builtin_bit_cast(s16x8, ai), bi, FIRST ? z4 : sli);
    }
  };
  // Slices of KSC chunks (KS divides H, so nch is a multiple of KSC).
  for (int ch = 0; ch < nch; ch += KSC) {
    step(std::true_type{}, ch);
    for (int k = 1; k < KSC; ++k) step(std::false_type{}, ch + k);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < PD_NCW; ++j) br[i][j] = br[i][j] + sl[i][j];  // slice done: add it to the branch total
    bri = bri + sli;
  }
  wait_vm_le<0>();  // the reloads past the end have landed before the LDS goes away

  // Branch partials: bpart[c][m][n].
  const int fg = lane >> 4, fj = lane & 15;
#pragma unroll
  for (int j = 0; j < PD_NCW; ++j) {
    const int t = t_lo + cq + 4 * j;
    if (t < t_hi) {
      const int n = 16 * t + fj;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * (4 * rh + i) + 4 * fg + r;
          if (row < M) bpart[((int64_t)sy * a.M + m0 + row) * g.NP + n] = br[i][j][r];
        }
    }
  }
  if (inj_here && fj < a.C) {
    const int n = a.R + fj;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * wave + 4 * fg + r;
      if (row < M) bpart[((int64_t)sy * a.M + m0 + row) * g.NP + n] = bri[r];
    }
  }
}

// --------------------------------------------------------------- pf_dfew (slice mode, few rows)
//
// hn @ [down | inject] for few rows, one unit of work per (64-row block,
// slice s of branch c, 64-column group b): the unit's hn tile [rows][KS] is built in LDS
// from S (streams_out, or the prologue inputs), rinv and norm_scale; its
// weight tile [KS][64] (with the inject columns in the group that holds
// column R) goes to LDS as four [KS][16] tiles; wave w runs the chain of
// column tile 4b + w for each 16-row tile. These are the decode kernel's
// chains, in the same order, and they write the same per-slice partials as
// k_pf_down in slice mode. Every load of a unit is issued before it waits on
// any. Units are ordered row block, slice, column group, and an XCD's
// workgroups take consecutive units, so the column groups of a slice share
// that XCD's L2 copy of its S; the grid has at most two workgroups per
// compute unit (66 KB of LDS each), which walk the units.
constexpr int PF_FEW_ROWS = 64;
constexpr int PF_FKS = 256;         // largest slice length
constexpr int PF_FHN = PF_FKS + 8;  // hn row pitch (elements)

template <DT D, bool REB>
__global__ __launch_bounds__(256) void k_pf_dfew(Args a, Geometry g, const float* __restrict__ rinv,
                                                 float* __restrict__ bpart, int units) {
  __shared__ __attribute__((aligned(16))) uint16_t hn_lds[PF_FEW_ROWS * PF_FHN];
  __shared__ __attribute__((aligned(16))) uint16_t w_lds[4 * PF_FKS * 16];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int KS = g.KS, NQS = KS >> 3, NG = (g.NT + 3) >> 2;
  const int G = gridDim.x;
  const int v = (G & 7) == 0 ? (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const uint16_t* ssrc = (const uint16_t*)(REB || !a.streams_out ? a.streams : a.streams_out);
  const int q = tid & 31, hr = tid >> 5;  // this thread's chunk of a slice row; rows hr + 8 j
  const int qc = min(q, NQS - 1);
  for (int u = v; u < units; u += G) {
    const int rb = u / (g.NS * NG), us = u - rb * (g.NS * NG), s = us / NG, b = us - s * NG, c = s / g.SPB;
    const int64_t m0 = (int64_t)rb * PF_FEW_ROWS;
    const int M = (int)min((int64_t)PF_FEW_ROWS, a.M - m0), MT = (M + 15) >> 4;
    const int64_t hbase = (int64_t)(s - c * g.SPB) * KS, kbase = (int64_t)c * a.H + hbase;
    // 1. Every load of the unit (rows past the batch and chunks past the
    //    slice read a valid address; those values are not used).
    u32x4 sv[8], pv[8];
    float rv[8], gv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t m = m0 + min(hr + 8 * j, M - 1);
      sv[j] = *(const u32x4*)(ssrc + m * a.K + kbase + 8 * qc);
      if constexpr (REB) {
        pv[j] = *(const u32x4*)((const uint16_t*)a.prev_out + m * a.H + hbase + 8 * qc);
        gv[j] = ld<D>(a.prev_gate, m * a.C + c);
      }
      rv[j] = rinv[m * a.C + c];
    }
    const uint4 nsr = *(const uint4*)((const uint16_t*)a.ns + kbase + 8 * qc);
    u32x4 wreg[PF_FKS / 32];
    const int col8 = 64 * b + 8 * (tid & 7);
    const bool col_ok = col8 + 8 <= a.R, inj_wg = b == (a.R >> 6);
    if (64 * b < a.R) {
      const uint16_t* wd = (const uint16_t*)a.wd + (kbase + (tid >> 3)) * a.R + min(col8, a.R - 8);
#pragma unroll
      for (int p = 0; p < PF_FKS / 32; ++p)
        if (32 * p < KS) wreg[p] = *(const u32x4*)(wd + (size_t)(32 * p) * a.R);
    }
    uint4 injw = make_uint4(0u, 0u, 0u, 0u);
    if (inj_wg) injw = inject_word((const uint16_t*)a.wi, a.C, kbase, KS, tid);

    // 2. hn of the unit's rows into LDS, rounded to T (rows past the batch,
    //    up to the end of the last 16-row tile, zero).
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = hr + 8 * j;
      if (q < NQS && m < 16 * MT) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (m < M) {
          float x[8], nsv[8], hv[8];
          unpack8<D>(to_uint4(sv[j]), x);
          if constexpr (REB) {
            float p[8];
            unpack8<D>(to_uint4(pv[j]), p);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], gv[j], p[e]);
          }
          unpack8<D>(nsr, nsv);
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = hnorm_raw(x[e], rv[j], nsv[e]);
          w = pack8<D>(hv);
        }
        *(uint4*)(hn_lds + m * PF_FHN + 8 * q) = w;
      }
    }

    // 3. The weight tile to LDS as four [KS][16] tiles (columns past R zero),
    //    then the inject columns into their tile.
    if (64 * b < a.R) {
#pragma unroll
      for (int p = 0; p < PF_FKS / 32; ++p)
        if (32 * p < KS) {
          const int rr = 32 * p + (tid >> 3), j = tid & 7;
          *(u32x4*)(w_lds + (j >> 1) * (PF_FKS * 16) + rr * 16 + 8 * (j & 1)) = col_ok ? wreg[p] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (inj_wg) {
      __syncthreads();  // the zero chunks of the inject tile are in place
      inject_scatter(w_lds + ((a.R - 64 * b) >> 4) * (PF_FKS * 16), a.C, KS, tid, injw);
    }
    __syncthreads();

    // 4. Chains: wave w takes column tile t = 4b + w, one chain over the
    //    slice per 16-row tile, and writes the slice partials of its rows.
    const int t = 4 * b + wave;
    if (t < g.NT) {
      const int n = 16 * t + (lane & 15);
      for (int i = 0; i < MT; ++i) {
        const f32x4 acc =
            mfma_chain<D, PF_FKS / 32>(hn_lds + 16 * i * PF_FHN, PF_FHN, w_lds + wave * (PF_FKS * 16), KS, lane);
        if (n < a.R + a.C)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * (lane >> 4) + r;
            if (m < M) bpart[((int64_t)s * a.M + m0 + m) * g.NP + n] = acc[r];
          }
      }
    }
    __syncthreads();  // the tiles are rewritten by the next unit
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

// --------------------------------------------------------------- pf_upb + pf_premix (few rows)
//
// For at most 128 rows the other up kernels keep most compute units idle or
// read up_weight in column tiles that use 32 of every 128 bytes they fetch;
// a compute unit has only so many line requests in flight, so what bounds
// them is lines per compute unit, not bytes. Here a unit of work is 64
// features of ONE branch (whole 128-byte pieces of each up_weight row, each
// read by exactly one unit): H/64 x C units. A unit runs the up chains of its
// 64 rows x 64 features, g, and writes the fp32 product hn * g of each (row,
// branch, feature), which is exact for 16-bit T; k_pf_premix then adds the C
// products of each output in ascending c, scales by rs and rounds once: the
// same operations in the same order as the other up kernels.
//
// Rows come in blocks of 64, each with its own GL workgroups (GL x blocks <=
// compute units); workgroup v of a block takes units v, v + GL, ... Every unit
// of a block reads the same hidden tile (its rows, all of R), which a
// workgroup loads into LDS once, and a workgroup with more units loads the
// next unit's up_weight piece into registers (and its epilogue inputs) while
// it runs the current unit's chains and epilogue.
constexpr int PB_BM = 64;   // rows per workgroup (four row tiles)
// The upb path's row limit: two row blocks. It beats k_pf_uppre by 1.5-2.4 us
// on the 4x2560 block and 5.6-7.4 us on the 8x4096 fp16 one from 65 to 128
// rows. Past that its rounds per workgroup grow faster than k_pf_uppre's
// time does: at 192 rows it loses 3.6 us on the fp16 block, and from 256 rows
// 3.5-29 us on both.
constexpr int PB_MAXROWS = 128;
constexpr int PB_BF = 64;   // features per unit (four column tiles of one branch)
constexpr int PB_HV = 8;    // hidden chunks per thread: 64 rows x R / 8 chunks over 512 threads, R <= 512
constexpr int PB_WV = 8;    // up_weight pieces per thread: R rows x 8 pieces over 512 threads, R <= 512

// LDS: hidden tile [64][R + 8], up_weight piece [R][64], up rounded to T [64][64].
static size_t pf_upb_lds_bytes(int R) {
  return (size_t)PB_BM * (R + 8) * 2 + (size_t)R * PB_BF * 2 + (size_t)PB_BM * PB_BF * 2;
}
bool prefill_up_few(int64_t M, int C, int H, int R) {
  return M <= PB_MAXROWS && H % PB_BF == 0 && R <= 512 && pf_upb_lds_bytes(R) <= 150 * 1024;
}

// MULTI: some workgroup has more than one unit (else the loop and the
// prefetch are compiled out).
template <DT D, bool FROM_SO, bool MULTI>
__global__ __launch_bounds__(512) void k_pf_upb(Args a, const float* __restrict__ rinv,
                                                const void* __restrict__ hidden, float* __restrict__ prod, int units,
                                                int gl) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int R = a.R, HLD = R + 8, R8 = R >> 3;
  uint16_t* hid_lds = (uint16_t*)smem;       // [64][R + 8]
  uint16_t* wu_lds = hid_lds + PB_BM * HLD;  // [R][64]: 128 bytes of each up_weight row
  uint16_t* up_lds = wu_lds + R * PB_BF;     // [64][64]
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nfb = a.H / PB_BF;  // feature blocks per branch; unit u = (block u mod nfb, branch u / nfb)
  const int rb = (int)blockIdx.x / gl;  // row block (uniform)
  const int64_t m0 = (int64_t)rb * PB_BM;
  const int M = (int)min((int64_t)PB_BM, a.M - m0);
  const bool pro = a.prev_out != nullptr;
  int u = (int)blockIdx.x - rb * gl;
  if (u >= units) return;  // (whole workgroup: before any barrier)

  // up_weight piece of unit v: rows 0..R-1, columns c H + f0 .. +63; piece
  // e = tid + 512 i is row e / 8, 16-byte column piece e % 8.
  auto wsrc = [&](int v) {
    return (const uint16_t*)a.wu + (size_t)(v / nfb) * a.H + (size_t)(v % nfb) * PB_BF;
  };
  // Epilogue inputs of unit v for this thread: row er = tid / 8, features f0 + 8 (tid % 8) .. +7.
  const int er = tid >> 3;
  const int64_t em = m0 + min(er, M - 1);
  struct EpIn {
    uint4 s, n, p;
    float rv, q;
  };
  auto ep_load = [&](int v, EpIn& e) {
    const int c = v / nfb, eh = (v % nfb) * PB_BF + 8 * (tid & 7);
    e.s = *(const uint4*)((const uint16_t*)(FROM_SO ? a.streams_out : a.streams) + em * a.K + (int64_t)c * a.H + eh);
    e.n = *(const uint4*)((const uint16_t*)a.ns + (int64_t)c * a.H + eh);
    e.p = (!FROM_SO && pro) ? *(const uint4*)((const uint16_t*)a.prev_out + em * a.H + eh) : make_uint4(0u, 0u, 0u, 0u);
    e.rv = rinv[em * a.C + c];
    e.q = (!FROM_SO && pro) ? ld<D>(a.prev_gate, em * a.C + c) : 0.0f;
  };

  // First unit. Every global load is issued before the workgroup waits on
  // any, and it waits once: an LDS write after direct global->LDS loads waits
  // for all of them, so the hidden tile goes to LDS only after the last issue.
  // 1. The hidden tile [64][R] into registers: chunk tid + 512 i (rows past
  //    the batch zero; PB_HV chunks per thread cover 64 rows of R <= 512).
  EpIn cur;
  {
    uint4 hv[PB_HV];
#pragma unroll
    for (int i = 0; i < PB_HV; ++i) {
      const int ch = tid + 512 * i, r = ch / R8, k = ch - r * R8;
      hv[i] = (ch < PB_BM * R8 && r < M) ? *(const uint4*)((const uint16_t*)hidden + (m0 + r) * R + 8 * k)
                                         : make_uint4(0u, 0u, 0u, 0u);
    }
    // 2. The first unit's up_weight piece straight into LDS: a load of 64
    //    lanes covers 8 rows (lane l: row l / 8, piece l % 8).
    const uint16_t* wu = wsrc(u) + 8 * (lane & 7) + (size_t)(lane >> 3) * a.K;
    for (int p = wave; 8 * p < R; p += 8) pf_load_lds16(wu + (size_t)(8 * p) * a.K, wu_lds + 8 * p * PB_BF);
    // 3. The first unit's epilogue inputs (before the LDS writes below,
    //    which wait for every load issued so far).
    ep_load(u, cur);
#pragma unroll
    for (int i = 0; i < PB_HV; ++i) {
      const int ch = tid + 512 * i, r = ch / R8, k = ch - r * R8;
      if (ch < PB_BM * R8) *(uint4*)(hid_lds + r * HLD + 8 * k) = hv[i];
    }
  }
  wait_vm_le<0>();
  __syncthreads();

  const int ct = wave & 3, rt0 = 2 * (wave >> 2);
  u32x4 wn[PB_WV];
  EpIn nxt;
  for (;;) {
    const int un = u + gl;
    const bool more = MULTI && un < units;
    // 4. The next unit's piece into registers and its epilogue inputs, in
    //    flight during this unit's chains and epilogue.
    if (more) {
      const uint16_t* ws = wsrc(un);
#pragma unroll
      for (int i = 0; i < PB_WV; ++i) {
        const int e = tid + 512 * i, r = min(e >> 3, R - 1);
        wn[i] = *(const u32x4*)(ws + (size_t)r * a.K + 8 * (e & 7));
      }
      ep_load(un, nxt);
    }

    // 5. Chains: wave w takes column tile w & 3 (16 features) and row tiles
    //    2 (w >> 2), 2 (w >> 2) + 1; one chain over R per 16x16 tile, k ascending.
    f32x4 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < R; k0 += 32) {
      const s16x8 bf = lds_bfrag_pitched(wu_lds + k0 * PB_BF, PB_BF * 2, 16 * ct, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i] = mfma<D>(lds_afrag(hid_lds + (rt0 + i) * 16 * HLD, HLD, k0, lane), bf, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        up_lds[(16 * (rt0 + i) + 4 * (lane >> 4) + r) * PB_BF + 16 * ct + (lane & 15)] = (uint16_t)to_bits<D>(acc[i][r]);
    __syncthreads();  // up of every tile is in LDS; every wave is done with the up_weight piece

    // 6. prod[m][c][h] = rT(hn) * rT(g), exact in fp32.
    if (er < M) {
      float x[8], nsv[8], up[8], pv[8], t[8];
      unpack8<D>(cur.s, x);
      unpack8<D>(cur.n, nsv);
      unpack8<D>(*(const uint4*)(up_lds + er * PB_BF + 8 * (tid & 7)), up);
      if (!FROM_SO && pro) unpack8<D>(cur.p, pv);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float S0 = (!FROM_SO && pro) ? prologue<D>(x[e], cur.q, pv[e]) : x[e];
        const float S1 = (!FROM_SO && pro) ? prologue<D>(x[e + 1], cur.q, pv[e + 1]) : x[e + 1];
        float h0 = hnorm_raw(S0, cur.rv, nsv[e]), h1 = hnorm_raw(S1, cur.rv, nsv[e + 1]);
        rT2<D>(h0, h1);
        float g0 = up_gate_raw<D>(up[e]), g1 = up_gate_raw<D>(up[e + 1]);  // up is already T
        rT2<D>(g0, g1);
        t[e] = h0 * g0;
        t[e + 1] = h1 * g1;
      }
      const int c = u / nfb, eh = (u % nfb) * PB_BF + 8 * (tid & 7);
      float* dst = prod + ((em * a.C + c) * (int64_t)a.H + eh);
#pragma unroll
      for (int e = 0; e < 8; e += 4) *(f32x4*)(dst + e) = f32x4{t[e], t[e + 1], t[e + 2], t[e + 3]};
    }
    if (!more) break;
    // 7. The next unit's piece into LDS (every wave passed the barrier above,
    //    so the old piece is no longer read; up_lds is read again only after
    //    the next unit's chains and barrier).
#pragma unroll
    for (int i = 0; i < PB_WV; ++i) {
      const int e = tid + 512 * i;
      if (e < 8 * R) *(u32x4*)(wu_lds + (e >> 3) * PB_BF + 8 * (e & 7)) = wn[i];
    }
    cur = nxt;
    u = un;
    __syncthreads();
  }
}

// pre[m][h] = rT(rs * (((0 + prod[m][0][h]) + prod[m][1][h]) + ...)): four
// features of one row per thread.
template <DT D>
__global__ __launch_bounds__(256) void k_pf_premix(Args a, const float* __restrict__ prod) {
  const int64_t total = a.M * (a.H >> 2);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / (a.H >> 2);
    const int h = 4 * (int)(i - m * (a.H >> 2));
    f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < a.C; ++c) sum = sum + *(const f32x4*)(prod + (m * a.C + c) * a.H + h);
    const float o0 = a.rs * sum[0], o1 = a.rs * sum[1], o2 = a.rs * sum[2], o3 = a.rs * sum[3];
    *(uint2*)((uint16_t*)a.pre + m * a.H + h) = make_uint2(pack2<D>(o0, o1), pack2<D>(o2, o3));
  }
}

// --------------------------------------------------------------- pf_up2 (bf16)
//
// up = hidden @ up_weight, g = sigmoid(up), and the pre-mix, for a workgroup
// of 512 rows and a block of 128 columns: features f0 .. f0 + UF - 1 of every
// branch (UF = 128 / C). The products are taken transposed: with the
// up_weight block as the A operand and hidden rows as the B operand, each
// 16x16x32 step yields the transpose of the usual tile, bit for bit (checked
// on gfx950 over 2^24 random chains in bf16 and fp16), so a lane ends with
// four consecutive features of one row and S, norm_scale and pre_output move
// eight bytes at a time. The block sits in LDS transposed ([column][k]) for
// the whole workgroup, and each wave runs its 32-row chunks on its own (two
// waves per SIMD: one's sigmoids overlap the other's matrix work). The
// sigmoid of a bf16 up value comes from an LDS table built with the same
// function, sigmoid_t, for |up| in [2^-16, 256); other inputs compute it.
constexpr int PU_RPW = 512;              // rows per workgroup
constexpr int PU_CH = 32;                // rows per chunk (two row tiles)
constexpr int PU_COLS = 128;             // columns per workgroup (eight 16-column tiles)
constexpr int PU_RMAX = 320;             // largest rank (a chunk's hidden fragments stay in registers)
constexpr int PU_KMAX = PU_RMAX / 32;    // k-steps
constexpr int PU_AD = 3;                 // block LDS reads in flight ahead of the matrix ops
constexpr int PU_WP = PU_RMAX + 8;       // LDS pitch of a block column (every rank laid out as PU_RMAX)
constexpr int PU_TE0 = 111, PU_TNE = 24; // table: bf16 exponents [111, 135)
constexpr int PU_TAB = 2 * PU_TNE * 128; // entries (positive half, then negative)
// In LDS the table is indexed by the bf16 bits of up themselves, less
// PU_TLO: entries [0, PU_TNE 128) hold the positive half and entries
// [0x8000, 0x8000 + PU_TNE 128) the negative half; the gap between is never
// read (no bf16 value in range falls in it).
constexpr uint32_t PU_TLO = (uint32_t)PU_TE0 << 7;  // bits of the smallest |up| in range
constexpr uint32_t PU_THI = PU_TLO + (PU_TNE << 7); // one past the largest
constexpr int PU_TDIR = 0x8000 + PU_TNE * 128;      // LDS entries

__device__ __forceinline__ uint32_t pu_gate_bits(const uint16_t* tab, uint32_t ub) {
  const uint32_t t = (ub & 0x7FFFu) - PU_TLO;
  const bool in = t < (uint32_t)(PU_TNE << 7);
  uint32_t g = tab[in ? ub - PU_TLO : 0u];
  if (!in) g = f32_to_bf16_bits(sigmoid_t(bf16_bits_to_f32(ub)));
  return g;
}

// The shapes this kernel takes (others use k_pf_uppre).
// Offsets inside a row block are 32-bit element counts: PU_RPW rows of
// streams must stay below 2^32 elements.
static bool pf_up2_ok(int dtype, int C, int H, int R) {
  return dtype == 16 && (C == 1 || C == 2 || C == 4 || C == 8) && H % (PU_COLS / C) == 0 && R <= PU_RMAX &&
         R % 32 == 0 && (int64_t)C * H * PU_RPW <= 0xFFFFFFFFLL;
}
// Rows above which k_pf_up2 (with k_pf_prep's transposed copy of up_weight)
// beats k_pf_uppre (measured at C=4, H=2560, R=320: 17.2 against 14.6 us at
// 64 rows, 31.6 against 37.5 us at 1024).
constexpr int64_t PU_MIN_ROWS = 512;
bool prefill_up_fast(int dtype, int64_t M, int C, int H, int R) {
  return M > PU_MIN_ROWS && pf_up2_ok(dtype, C, H, R);
}

// Few rows: k_pf_down's grid (128-row tiles x branches x column groups) would
// leave most compute units idle, each workgroup walking a whole branch, so it
// takes one slice per workgroup and writes per-slice partials instead (the
// same chains, added in the same order by k_slice_reduce).
bool prefill_slices(int64_t M, int C, int H, int R) {
  const int64_t tiles = (M + PD_BM - 1) / PD_BM, ncg = ((R >> 4) + PD_TPG - 1) / PD_TPG;
  return tiles * C * ncg <= 64 && slice_length(H) > 0;
}
static_assert(PREFILL_GTAB_BYTES == PU_TAB * 2, "sigmoid table size");

// Per-call preparation for k_pf_up2: wut[j][n] = up_weight[n][j] (so that a
// column's R values are contiguous), by 64x32 tiles through LDS, and (the
// extra column of tiles) the bf16 sigmoid table. Tile (bx, by) of an nx x ny
// grid.
__device__ __forceinline__ void prep_tile(const Args& a, uint16_t* __restrict__ wut, uint16_t* __restrict__ gtab,
                                          int bx, int by, int nx, int ny, uint16_t (*t)[64 + 2]) {
  const int tid = threadIdx.x;
  if (bx == nx - 1) {  // the table
    for (int e = by * 256 + tid; e < PU_TAB; e += ny * 256) {
      const uint32_t b = (e >= PU_TNE * 128 ? 0x8000u : 0u) | (uint32_t)((PU_TE0 << 7) + e % (PU_TNE * 128));
      gtab[e] = (uint16_t)f32_to_bf16_bits(sigmoid_t(bf16_bits_to_f32(b)));
    }
    return;
  }
  const int64_t j0 = (int64_t)bx * 64;
  const int n0 = by * 32;
  {  // rows n0 .. n0+31 of up_weight, columns j0 .. j0+63: 8 values per thread
    const int n = tid >> 3, jq = 8 * (tid & 7);
    const uint4 v = *(const uint4*)((const uint16_t*)a.wu + (int64_t)(n0 + n) * a.K + j0 + jq);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[n][jq + 2 * i] = (uint16_t)(w[i] & 0xFFFFu);
      t[n][jq + 2 * i + 1] = (uint16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
  {  // wut rows j0 .. j0+63, values n0 .. n0+31: 8 per thread
    const int j = tid >> 2, nq = 8 * (tid & 3);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)t[nq + 2 * i][j] | ((uint32_t)t[nq + 2 * i + 1][j] << 16);
    *(uint4*)(wut + (j0 + j) * a.R + n0 + nq) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ __launch_bounds__(256) void k_pf_prep(Args a, uint16_t* __restrict__ wut, uint16_t* __restrict__ gtab) {
  __shared__ uint16_t t[32][64 + 2];
  prep_tile(a, wut, gtab, blockIdx.x, blockIdx.y, gridDim.x, gridDim.y, t);
}

// The branch reduction and k_pf_prep's work in one launch: neither needs the
// other's results, and each alone leaves memory bandwidth unused. Workgroups
// alternate between the two kinds while both have work left; the reduction's
// nred workgroups stride over its items as k_branch_reduce does.
template <DT D>
__global__ __launch_bounds__(256) void k_pf_reduce_prep(Args a, int NP, const float* __restrict__ partial,
                                                        void* __restrict__ hidden, int nred, uint16_t* __restrict__ wut,
                                                        uint16_t* __restrict__ gtab, int px, int py) {
  __shared__ uint16_t t[32][64 + 2];
  const int b = blockIdx.x, npre = px * py, both = 2 * min(nred, npre);
  int r, q;  // index of a reduction workgroup, or of a prep tile (the other -1)
  if (b < both) {
    r = b & 1 ? -1 : b >> 1;
    q = b & 1 ? b >> 1 : -1;
  } else {
    r = nred > npre ? b - both + npre : -1;
    q = nred > npre ? -1 : b - both + nred;
  }
  if (r >= 0) {
    branch_reduce_items<D>(a, NP, partial, hidden, (int64_t)r * 256 + threadIdx.x, (int64_t)nred * 256);
    return;
  }
  prep_tile(a, wut, gtab, q % px, q / px, px, py, t);
}

// Feature order inside the LDS block. The output tile of a lane holds four
// consecutive columns of one row; pairing the column tiles of a branch so
// that tile 2p takes features 32p + 8 s + (0..3) and tile 2p + 1 takes
// 32p + 8 s + (4..7) in column slots 4 s .. 4 s + 3 gives a lane eight
// consecutive features (16-byte loads and stores). With one tile per branch
// the slots are the features. Returns the branch-relative feature of column
// slot `slot` of the branch's tile t.
template <int FT> __device__ __forceinline__ int pu_feature(int t, int slot) {
  if constexpr (FT == 1) return slot;
  else return 32 * (t >> 1) + 8 * (slot >> 2) + 4 * (t & 1) + (slot & 3);
}

template <int C, bool FROM_SO, bool FULL>
__global__ __launch_bounds__(512) void k_pf_up2(Args a, const float* __restrict__ rinv,
                                                const void* __restrict__ hidden, const uint16_t* __restrict__ wutg,
                                                const uint16_t* __restrict__ gtab) {
  constexpr DT D = DT::BF16;
  constexpr int UF = PU_COLS / C, FT = UF / 16;   // features per workgroup, feature tiles per branch
  constexpr int GW = FT == 1 ? 4 : 8;             // consecutive features a lane holds per group
  constexpr int NG = FT == 1 ? 1 : FT / 2;        // feature groups per branch
  __shared__ __attribute__((aligned(16))) uint16_t wut[PU_COLS * PU_WP];  // [column][k], zero for k >= R
  __shared__ __attribute__((aligned(16))) uint16_t tab[PU_TDIR];
  __shared__ __attribute__((aligned(16))) uint16_t nsl[2][PU_COLS];  // norm_scale of the block's features, [c][f], by unit parity
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int R = a.R, NKS = R >> 5;
  constexpr int WP = PU_WP;
  // Work units are (row block of PU_RPW rows, column group) pairs in
  // row-block-major order; the grid has one workgroup per compute unit (it
  // loads the sigmoid table once) and workgroup v takes units v, v + G,
  // v + 2G, ... At any time the grid works on G consecutive units, a few
  // row blocks, so their hidden rows stay in L2; the column block is loaded
  // for each unit. Workgroups go to the eight XCDs round-robin by id; v
  // numbers them XCD by XCD, so an XCD's workgroups take consecutive units.
  const int nrb = (int)((a.M + PU_RPW - 1) / PU_RPW), ncg = a.H / UF, nun = nrb * ncg;
  const int G = gridDim.x;
  const int v = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  if (v >= nun) return;  // (whole workgroup: before any barrier)
  const int nst = (nun - v + G - 1) / G;  // units of this workgroup

  // The column block of column group cg (pitch WP) and its norm_scale, by
  // direct global->LDS loads: lane l of a wave fills the 16-byte LDS slot
  // base + l, slot s holding piece s mod (WP/8) of column s / (WP/8) (pieces
  // from R/8 on are padding and zero; a load there fetches a real piece into
  // the pitch's last slot, which is never read, and leaves the zeros alone).
  auto load_block = [&](int cg, int nb) {
    constexpr int PC = WP / 8, total = PU_COLS * PC;
    const int f0 = cg * UF, RP = R >> 3;
    for (int base = wave * 64; base < total; base += 512) {
      const int sl = base + lane, col = sl / PC, kp = sl - col * PC;
      const int j = col >> 4, c = j / FT, f = pu_feature<FT>(j - c * FT, col & 15);
      if (sl < total && (kp < RP || kp == PC - 1))
        pf_load_lds16(wutg + ((int64_t)c * a.H + f0 + f) * R + 8 * min(kp, RP - 1), wut + 8 * base);
    }
    if (wave == 7 && lane < PU_COLS / 8) {  // nsl slot l: branch l / (UF/8), features 8 (l mod (UF/8)) ..
      const int c = lane / (UF / 8), f8 = 8 * (lane - c * (UF / 8));
      pf_load_lds16((const uint16_t*)a.ns + (int64_t)c * a.H + f0 + f8, nsl[nb]);
    }
  };
  // Ranks below PU_RMAX: the block's k >= R stays zero (the loads never touch it).
  if (R < PU_RMAX)
    for (int e = tid; e < PU_COLS * ((PU_RMAX - R) >> 3); e += 512) {
      const int col = e / ((PU_RMAX - R) >> 3), k8 = R + 8 * (e - col * ((PU_RMAX - R) >> 3));
      *(uint4*)(wut + col * WP + k8) = make_uint4(0u, 0u, 0u, 0u);
    }
  // The sigmoid table: twelve 64-piece runs, six per sign.
  for (int k = wave; k < PU_TAB / 512; k += 8)
    pf_load_lds16(gtab + 8 * (64 * k + lane), tab + (k < PU_TNE / 4 ? 512 * k : 0x8000 + 512 * (k - PU_TNE / 4)));
  int cg_cur = v % ncg, nb_cur = 0;
  load_block(cg_cur, nb_cur);
  wait_vm_le<0>();
  __syncthreads();

  // Lane (fg, fj): row fj of each row tile; for branch c and group g, the GW
  // features h(c, g) .. + GW - 1 (tiles c FT + 2g and c FT + 2g + 1, or tile c).
  const int fg = lane >> 4, fj = lane & 15;
  auto hrel = [&](int g) { return (uint32_t)(FT == 1 ? 4 * fg : 32 * g + 8 * fg); };  // feature offset from f0
  typedef typename std::conditional<GW == 8, u32x4, u32x2>::type vec;
  const bool pro = !FROM_SO && a.prev_out != nullptr;
  const uint32_t K = (uint32_t)a.K, H = (uint32_t)a.H;
  // Chunk z of this workgroup: rows 32 (z mod 16) .. of the row block of unit
  // v + G (z / 16). Its bases are uniform (scalar registers); everything
  // inside the row block is a 32-bit unsigned offset from them.
  struct Geo {
    int64_t m0;
    int rlast, cg, q;  // last row of the row block (relative), column group, chunk in the block
  };
  auto geo = [&](int z) {
    Geo g;
    const int u = v + G * (z >> 4);
    const int rb = __builtin_amdgcn_readfirstlane(u / ncg);  // (uniform: keep it and what follows scalar)
    g.cg = u - rb * ncg;
    g.m0 = (int64_t)rb * PU_RPW;
    g.rlast = __builtin_amdgcn_readfirstlane((int)min((int64_t)PU_RPW - 1, a.M - 1 - g.m0));
    g.q = z & 15;
    return g;
  };
  const int nz = nst * 16;
  static_assert(PU_RPW / PU_CH == 16, "16 chunks per row block");

  // A chunk's hidden fragments run through a ring of PU_HR k-steps, refilled
  // PU_HR steps ahead inside the chain; the next chunk's first PU_HR are
  // issued before this chunk's epilogue, so their latency hides behind it.
  constexpr int PU_HR = 3;  // hidden ring slots
  struct ChunkIn {
    u32x4 hf[PU_HR][2];
  };
  auto rows_of = [&](const Geo& g, uint32_t* mr) {  // block-relative rows, clamped into the batch
#pragma unroll
    for (int i = 0; i < 2; ++i) mr[i] = (uint32_t)min(g.q * PU_CH + 16 * i + fj, g.rlast);
  };
  // Hidden fragment of k-step ks; zero past the rank (FULL: R = PU_RMAX, no
  // such steps), by a uniform mask rather than a branch.
  auto hid = [&](const uint16_t* hb, const uint32_t* mr, int i, int ks) {
    if constexpr (FULL) return *(const u32x4*)(hb + (mr[i] * (uint32_t)R + (uint32_t)(8 * fg + 32 * ks)));
    const uint32_t keep = ks < NKS ? 0xFFFFFFFFu : 0u;
    const u32x4 h = *(const u32x4*)(hb + (mr[i] * (uint32_t)R + (uint32_t)(8 * fg + 32 * min(ks, NKS - 1))));
    return u32x4{h.x & keep, h.y & keep, h.z & keep, h.w & keep};
  };
  ChunkIn cur;
  auto prefetch = [&](int z) {  // the first hidden k-steps of chunk z, if it has rows
    if (z >= nz) return;
    const Geo g = geo(z);
    if (g.q * PU_CH > g.rlast) return;
    const uint16_t* hb = (const uint16_t*)hidden + g.m0 * R;
    uint32_t mr[2];
    rows_of(g, mr);
#pragma unroll
    for (int u = 0; u < PU_HR; ++u)
#pragma unroll
      for (int i = 0; i < 2; ++i) cur.hf[u][i] = hid(hb, mr, i, u);
  };
  // Epilogue state of the wave's latest chunk: its inputs (issued during its
  // chain), up rounded to T, where its output goes and which norm_scale
  // buffer it reads.
  vec sv[2][C][NG], pv[2][NG];
  float rv[2][C], qg[2][C];
  uint32_t upk[8][2][2];
  uint16_t* pre_b = nullptr;
  int q = 0, rlast = 0, nb_e = 0;
  bool table_only = false;
  // Epilogue: pre[m][h ..] = rT(rs * sum_c hn_c * g_c), c ascending; a
  // separate instance for chunks whose every up value is in the table, so
  // that its lookups are plain loads the compiler can batch.
  auto epilogue = [&](auto TABLE_ONLY) {
    auto gate = [&](uint32_t ub) -> float {
      if constexpr (decltype(TABLE_ONLY)::value) return widen<D>(tab[ub - PU_TLO]);
      else return widen<D>(pu_gate_bits(tab, ub));
    };
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = q * PU_CH + 16 * i + fj;  // block-relative row
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float sum[GW];
#pragma unroll
        for (int e = 0; e < GW; ++e) sum[e] = 0.0f;
        float pp[GW];
        if (pro) {
          const uint32_t* pw = (const uint32_t*)&pv[i][g];
#pragma unroll
          for (int e = 0; e < GW; e += 2) {
            pp[e] = widen<D>(pw[e / 2] & 0xFFFFu);
            pp[e + 1] = widen<D>(pw[e / 2] >> 16);
          }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const uint32_t* sw = (const uint32_t*)&sv[i][c][g];
          const vec nv = *(const vec*)(nsl[nb_e] + c * UF + hrel(g));
          const uint32_t* nw = (const uint32_t*)&nv;
          // tiles of this group: j0 (values 0..3), j0 + 1 (values 4..7)
          const int j0 = FT == 1 ? c : c * FT + 2 * g;
#pragma unroll
          for (int e = 0; e < GW; e += 2) {
            float x0 = widen<D>(sw[e / 2] & 0xFFFFu), x1 = widen<D>(sw[e / 2] >> 16);
            if (pro) {
              x0 = prologue<D>(x0, qg[i][c], pp[e]);
              x1 = prologue<D>(x1, qg[i][c], pp[e + 1]);
            }
            float h0 = hnorm_raw(x0, rv[i][c], widen<D>(nw[e / 2] & 0xFFFFu));
            float h1 = hnorm_raw(x1, rv[i][c], widen<D>(nw[e / 2] >> 16));
            rT2<D>(h0, h1);
            const uint32_t uw = upk[j0 + (e >> 2)][i][(e >> 1) & 1];
            sum[e] = sum[e] + h0 * gate(uw & 0xFFFFu);
            sum[e + 1] = sum[e + 1] + h1 * gate(uw >> 16);
          }
        }
        if (r <= rlast) {
          uint32_t o[GW / 2];
#pragma unroll
          for (int e = 0; e < GW; e += 2) o[e / 2] = pack2<D>(a.rs * sum[e], a.rs * sum[e + 1]);
          vec ov;
          __builtin_memcpy(&ov, o, sizeof(ov));
          *(vec*)(pre_b + ((uint32_t)r * H + hrel(g))) = ov;
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one row tile at a time (bounds the live registers)
    }
  };
  auto finish = [&]() {
    if (table_only) epilogue(std::true_type{});
    else epilogue(std::false_type{});
  };
  // A chunk's epilogue runs at the top of the wave's next iteration (one
  // call site). The two waves of a SIMD (waves w and w + 4 when waves go to
  // SIMDs in turn, w and w + 1 when they go two at a time: the test below
  // picks one of each pair either way) would start every unit together,
  // after the block load; one of them runs its last epilogue of a unit after
  // the next unit's block load instead of before it, so from then on one
  // wave of the pair runs its epilogue (vector and LDS work) while the other
  // runs its chain (matrix work). Every wave passes the same barriers, the
  // two kinds at different points of their code.
  const bool late_wave = (((wave >> 2) ^ wave) & 1) != 0;
  auto next_block = [&](int cg) {
    __syncthreads();  // all waves are done with the old block
    cg_cur = cg;
    nb_cur ^= 1;      // (a pending epilogue still reads the other norm_scale buffer)
    load_block(cg_cur, nb_cur);
    wait_vm_le<0>();
    __syncthreads();
  };
  bool pend = false;
  prefetch(wave);
  for (int z = wave;; z += 8) {
    const bool more = z < nz;
    const Geo gz = geo(more ? z : wave);
    const bool change = more && gz.cg != cg_cur;  // every wave meets this at its first chunk of the unit
    if (change && late_wave) next_block(gz.cg);
    if (pend) {
      finish();
      pend = false;
    }
    if (change && !late_wave) next_block(gz.cg);
    if (!more) break;
    if (gz.q * PU_CH > gz.rlast) {  // rows past the batch (last row block only)
      prefetch(z + 8);
      continue;
    }
    q = gz.q;
    rlast = gz.rlast;
    nb_e = nb_cur;
    const int f0 = gz.cg * UF;
    const int64_t m0 = gz.m0;
    const uint16_t* src = (const uint16_t*)(FROM_SO ? a.streams_out : a.streams) + m0 * a.K + f0;
    const uint16_t* hid_b = (const uint16_t*)hidden + m0 * R;
    const float* rinv_b = rinv + m0 * C;
    const uint16_t* pg_b = (const uint16_t*)a.prev_gate + (pro ? m0 * C : 0);
    const uint16_t* po_b = (const uint16_t*)a.prev_out + (pro ? m0 * a.H + f0 : 0);
    pre_b = (uint16_t*)a.pre + m0 * a.H + f0;
    uint32_t mr[2];
    rows_of(gz, mr);
    // Epilogue inputs. They come from HBM, and loads complete in order: issued
    // before the chain, they held it up at its first wait for a hidden refill
    // issued after them, so they are issued inside the chain right after its
    // last refill (one branch with S rebuilt from the prologue inputs keeps
    // them before the chain: inside it they would not fit the registers).
    constexpr bool EPI_IN_CHAIN = FROM_SO || C > 1;
    auto load_epi = [&]() {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int g = 0; g < NG; ++g) sv[i][c][g] = *(const vec*)(src + (mr[i] * K + (uint32_t)c * H + hrel(g)));
#pragma unroll
        for (int c = 0; c < C; ++c) {
          rv[i][c] = rinv_b[mr[i] * (uint32_t)C + (uint32_t)c];
          qg[i][c] = pro ? widen<D>(pg_b[mr[i] * (uint32_t)C + (uint32_t)c]) : 0.0f;
        }
        if (pro)
#pragma unroll
          for (int g = 0; g < NG; ++g) pv[i][g] = *(const vec*)(po_b + (mr[i] * H + hrel(g)));
      }
    };
    if constexpr (!EPI_IN_CHAIN) load_epi();
    // Up chain over R: k-steps ascending, from zero; hidden ring refilled PU_HR steps ahead.
    f32x4 acc[8][2];
    {
      // The block's LDS reads are issued PU_AD ahead of their matrix ops
      // through a ring of PU_AD + 1 registers (the reads are asm, each waited
      // for by a tied lgkmcnt); the hidden ring has compile-time slots. Every
      // rank runs PU_KMAX k-steps: past R both operands are zero, which adds
      // exact zeros.
      constexpr int NK = PU_KMAX, NT = NK * 8, AD = PU_AD;
      const uint32_t wl0 = lds_addr(wut) + (uint32_t)(2 * (fj * WP + 8 * fg));  // tiles 0..3
      const uint32_t wl1 = wl0 + (uint32_t)(2 * 64 * WP);                      // tiles 4..7
      u32x4 aw[AD + 1];
      u32x4 h0, h1;
      auto rd = [&](auto TT) {
        constexpr int t = decltype(TT)::value, ks = t / 8, j = t % 8;
        constexpr int off = 2 * (16 * (j & 3) * WP + 32 * ks);
        aw[t % (AD + 1)] = lds_rd128o<off>(j < 4 ? wl0 : wl1);
      };
      static_for<0, AD>(rd);
      static_for<0, NT>([&](auto TT) {
        constexpr int t = decltype(TT)::value, ks = t / 8, j = t % 8, slot = ks % PU_HR;
        if constexpr (j == 0) {
          h0 = cur.hf[slot][0];
          h1 = cur.hf[slot][1];
          if constexpr (ks + PU_HR < NK) {
            cur.hf[slot][0] = hid(hid_b, mr, 0, ks + PU_HR);
            cur.hf[slot][1] = hid(hid_b, mr, 1, ks + PU_HR);
          }
          if constexpr (EPI_IN_CHAIN && ks == NK - PU_HR - 1) load_epi();  // right after the last refill
        }
        if constexpr (t + AD < NT) rd(std::integral_constant<int, t + AD>{});
        constexpr int pend = t + AD < NT ? AD : NT - 1 - t;
        lgkm_tie<pend>(aw[t % (AD + 1)]);
        const s16x8 a8 = __builtin_bit_cast(s16x8, aw[t % (AD + 1)]);
        acc[j][0] = mfma<D>(a8, __builtin_bit_cast(s16x8, h0), ks == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[j][0]);
        acc[j][1] = mfma<D>(a8, __builtin_bit_cast(s16x8, h1), ks == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[j][1]);
      });
    }

    // up rounded to T, two values per word; whether every value of the chunk
    // is inside the table (then no lane needs the computed sigmoid).
    u16x2 amax = {0, 0}, amin = {0xFFFF, 0xFFFF};  // of |up| bits, two halves at a time
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          upk[j][i][h] = pack2<D>(acc[j][i][2 * h], acc[j][i][2 * h + 1]);
          const u16x2 mag = __builtin_bit_cast(u16x2, upk[j][i][h] & 0x7FFF7FFFu);
          amax = __builtin_elementwise_max(amax, mag);
          amin = __builtin_elementwise_min(amin, mag);
        }
    const bool inside = min(amin.x, amin.y) >= PU_TLO && max(amax.x, amax.y) < PU_THI;
    table_only = __all(inside);
    // The next chunk's first hidden k-steps, in flight during this epilogue.
    prefetch(z + 8);
    pend = true;
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
  const int64_t pairs = a.M * a.C;
  if ((pairs + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;  // grid x limit
  e = launch(mk, k_pf_rms<D>, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, a, rinv);
  if (e != hipSuccess) return e;
  const unsigned ncg = (unsigned)(((a.R >> 4) + PD_TPG - 1) / PD_TPG);
  const int nsl = prefill_slices(a.M, a.C, a.H, a.R) ? g.SPB : 1;
  const dim3 gd((unsigned)((a.M + PD_BM - 1) / PD_BM), (unsigned)(a.C * nsl), ncg);
  // k_pf_down's buffer descriptors: a workgroup's weight rows and its 128 rows of S in 31 bits.
  if ((int64_t)a.K * a.R * 2 > 0x7FFFFFFF || (int64_t)PD_BM * a.K * 2 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool reb = !from_so && a.prev_out != nullptr;  // S must be rebuilt from the prologue inputs
  const float* rv = rinv;
  const int64_t few_units = ((a.M + PF_FEW_ROWS - 1) / PF_FEW_ROWS) * g.NS * ((g.NT + 3) / 4);
  if (nsl > 1 && g.KS <= PF_FKS && few_units <= 2 * device_compute_units()) {
    // Few rows, and one unit of (64 rows, slice, 64 columns) per workgroup,
    // two workgroups per compute unit (with more units k_pf_down's pipeline
    // over the slice's chunks wins: wide fp16 block 18.1 against 23.7 us).
    const int fu = (int)few_units;
    e = reb ? launch(mk, k_pf_dfew<D, true>, dim3((unsigned)fu), dim3(256), 0, s, a, g, rv, bpart, fu)
            : launch(mk, k_pf_dfew<D, false>, dim3((unsigned)fu), dim3(256), 0, s, a, g, rv, bpart, fu);
  } else {
    e = reb ? launch(mk, k_pf_down<D, true>, gd, dim3(512), 0, s, a, g, rv, bpart, nsl)
            : launch(mk, k_pf_down<D, false>, gd, dim3(512), 0, s, a, g, rv, bpart, nsl);
  }
  if (e != hipSuccess) return e;
  const void* hd = hidden;
  const bool up_fast = prefill_up_fast((int)D, a.M, a.C, a.H, a.R);
  uint16_t* wt = (uint16_t*)(ws + w.wut);
  uint16_t* gt = (uint16_t*)(ws + w.gtab);
  const int px = a.K / 64 + 1, py = a.R / 32;  // k_pf_prep's tiles (the last column: the table)
  if (nsl == 1 && up_fast) {
    // The branch reduction and the up kernel's preparation in one launch.
    const int64_t wr = (a.M * (g.NP >> 2) + 255) / 256;
    const int nred = (int)(wr < 65536 ? wr : 65536);
    if (g.NP % 16 != 0 || a.R % 4 != 0) return hipErrorInvalidValue;
    e = launch(mk, k_pf_reduce_prep<D>, dim3((unsigned)(nred + px * py)), dim3(256), 0, s, a, g.NP,
               (const float*)bpart, hidden, nred, wt, gt, px, py);
  } else {
    e = nsl == 1 ? launch_branch_reduce(a, (int)D, g.NP, bpart, hidden, s, mk)
                 : launch_slice_reduce(a, (int)D, g.NP, g.SPB, bpart, hidden, s, mk);
    if (e != hipSuccess) return e;
    if (up_fast) e = launch(mk, k_pf_prep, dim3((unsigned)px, (unsigned)py), dim3(256), 0, s, a, wt, gt);
  }
  if (e != hipSuccess) return e;
  if (up_fast) {
    const uint16_t* wtc = wt;
    const uint16_t* gtc = gt;
    // One workgroup per compute unit (each holds 152 KB of LDS), at most one per unit of work.
    const int64_t units = ((a.M + PU_RPW - 1) / PU_RPW) * (a.H / (PU_COLS / a.C));
    const dim3 g2((unsigned)std::min<int64_t>(units, device_compute_units()));
    switch (a.C) {
      case 1: return from_so ? launch(mk, a.R == PU_RMAX ? k_pf_up2<1, true, true> : k_pf_up2<1, true, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc)
                             : launch(mk, k_pf_up2<1, false, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc);
      case 2: return from_so ? launch(mk, a.R == PU_RMAX ? k_pf_up2<2, true, true> : k_pf_up2<2, true, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc)
                             : launch(mk, k_pf_up2<2, false, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc);
      case 4: return from_so ? launch(mk, a.R == PU_RMAX ? k_pf_up2<4, true, true> : k_pf_up2<4, true, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc)
                             : launch(mk, k_pf_up2<4, false, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc);
      default: return from_so ? launch(mk, a.R == PU_RMAX ? k_pf_up2<8, true, true> : k_pf_up2<8, true, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc)
                              : launch(mk, k_pf_up2<8, false, false>, g2, dim3(512), 0, s, a, rv, hd, wtc, gtc);
    }
  }
  if (prefill_up_few(a.M, a.C, a.H, a.R)) {
    float* prod = (float*)(ws + w.prod);
    const size_t lb = pf_upb_lds_bytes(a.R);
    // Each row block's GL workgroups take units in balanced rounds; GL is
    // rounded to a multiple of 8 where it can be, so the workgroups of all
    // row blocks that read one up_weight piece run on one XCD.
    const int units = (a.H / PB_BF) * a.C;
    const int nrb = (int)((a.M + PB_BM - 1) / PB_BM);
    const int cap = std::max(1, device_compute_units() / nrb);
    const int rounds = (units + cap - 1) / cap;
    int gl = (units + rounds - 1) / rounds;
    if (nrb > 1 && gl > 8 && (gl + 7) / 8 * 8 <= cap) gl = (gl + 7) / 8 * 8;
    const int nwg = gl * nrb;
    const bool multi = units > gl;
    const void* kb = multi ? (from_so ? (const void*)k_pf_upb<D, true, true> : (const void*)k_pf_upb<D, false, true>)
                           : (from_so ? (const void*)k_pf_upb<D, true, false> : (const void*)k_pf_upb<D, false, false>);
    e = allow_dynamic_lds(kb, 12 + (multi ? 4 : 0) + (D == DT::BF16 ? 0 : 2) + (from_so ? 0 : 1), lb);
    if (e != hipSuccess) return e;
    const dim3 gb((unsigned)nwg);
    if (multi)
      e = from_so ? launch(mk, k_pf_upb<D, true, true>, gb, dim3(512), lb, s, a, rv, hd, prod, units, gl)
                  : launch(mk, k_pf_upb<D, false, true>, gb, dim3(512), lb, s, a, rv, hd, prod, units, gl);
    else
      e = from_so ? launch(mk, k_pf_upb<D, true, false>, gb, dim3(512), lb, s, a, rv, hd, prod, units, gl)
                  : launch(mk, k_pf_upb<D, false, false>, gb, dim3(512), lb, s, a, rv, hd, prod, units, gl);
    if (e != hipSuccess) return e;
    const int64_t np = (a.M * (a.H >> 2) + 255) / 256;
    const float* pc = prod;
    return launch(mk, k_pf_premix<D>, dim3((unsigned)(np < 4096 ? np : 4096)), dim3(256), 0, s, a, pc);
  }
  const dim3 gu((unsigned)((a.M + PF_BM - 1) / PF_BM), (unsigned)((a.H + PF_BF - 1) / PF_BF));
  if (a.C <= 4)
    return from_so ? launch(mk, k_pf_uppre<D, 4, true>, gu, dim3(512), lds, s, a, rv, hd)
                   : launch(mk, k_pf_uppre<D, 4, false>, gu, dim3(512), lds, s, a, rv, hd);
  return from_so ? launch(mk, k_pf_uppre<D, 8, true>, gu, dim3(512), lds, s, a, rv, hd)
                 : launch(mk, k_pf_uppre<D, 8, false>, gu, dim3(512), lds, s, a, rv, hd);
}

hipError_t launch_rows_rms(const Args& a, int dtype, float* rinv, hipStream_t s, Marks* mk) {
  const int64_t pairs = a.M * a.C;
  if ((pairs + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;  // grid x limit
  const dim3 grid((unsigned)((pairs + 3) / 4));
  if (dtype == 16) return launch(mk, k_pf_rms<DT::BF16>, grid, dim3(256), 0, s, a, rinv);
  if (dtype == 10) return launch(mk, k_pf_rms<DT::F16>, grid, dim3(256), 0, s, a, rinv);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                          hipStream_t s, Marks* mk) {
  if (dtype == 16) return run_prefill<DT::BF16>(a, ws, w, g, s, mk);
  if (dtype == 10) return run_prefill<DT::F16>(a, ws, w, g, s, mk);
  return hipErrorInvalidValue;
}

}  // namespace hc
