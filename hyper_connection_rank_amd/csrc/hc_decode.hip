// Decode path (at most 16 rows: one matrix-core row tile) of the
// HyperConnectionLowRankMix block on gfx950.
//
// The block streams 13.2 MB of weights (4 x 2560, rank 320, bf16) once from
// HBM, and everything else is latency: a graph-launched kernel costs about
// 1.5 us before it does anything, a trip to memory under load 1-2 us, and a
// wave64 instruction about 3 ns when one wave runs per SIMD. So the block is
// two kernels; every workgroup issues its global loads before it waits on any
// of them (small, early-needed loads first: the load counters complete in
// order); per-row work is spread over all waves; nothing divides by a runtime
// value. Weights stay row-major [K, N] and are used in place (onnxruntime PR
// #33384, "Motivation and Context"); they are read with coalesced 16-byte
// loads, staged in LDS and turned into matrix-core fragments by transposing
// LDS reads.
//
//   hc_down   grid (64-column tile group, slice, branch). Prologue and the
//             branch sum of squares of every row (each wave one quarter of the
//             canonical virtual lanes), hn of its slice (also written out for
//             hc_uppre), one 16x16x32 matrix-core chain per 16 output columns
//             of [down | inject], fp32 partials per slice. The last workgroup
//             of each tile group to finish (an agent-scope arrival counter)
//             adds the slices in their fixed order and writes hidden and
//             post_gate. The workgroups also prefetch the up_weight lines
//             hc_uppre will read into L2, in whole 128-byte lines.
//   hc_uppre  grid: 16 features, one wave per branch. Up chain over R,
//             sigmoid and the pre-mix over branches in ascending c.
//
// The split mirrors the PR's "CUDA implementation" (split-K partials, then a
// fixed-order consumer); where the consumer runs never changes the bits.
#include "hc_mfma_common.h"

#include <type_traits>

namespace hc {

constexpr int KSMAX = 256;        // largest slice length
constexpr int HN_LD = KSMAX + 8;  // padded LDS row of hn (elements)
constexpr int DEC_ROWS = 16;      // rows of the matrix-core tile
constexpr int SLOTS = 8;          // 16-byte chunks of a row group a lane holds (streams, and prev_out)
constexpr int RW_SLOTS = 5;       // the same, with one row per wave (at most 320 chunks per branch row)
constexpr int RED_BATCH = 16;     // slice partials one thread loads before adding them
constexpr int RED_ITEMS = 3;      // outputs whose partials one thread loads together
// The tail's partials in LDS: up to RED_ROWS rows of one tile group's 64
// columns (slices * rows of them per branch), whole branches at a time; a
// branch with more goes through registers. The variant whose registers allow
// several workgroups per compute unit (PRE) takes these rows as dynamic LDS,
// sized at launch: none when its workgroups outnumber the compute units, so
// that they can share them; the others hold them in static LDS.
constexpr int RED_ROWS = 384;
// hc_down runs four compute waves and one prefetch wave. A wave's load counter
// counts its own loads only, so the compute waves' waits never cover the
// prefetch stream; and a wave that has issued loads into LDS is made to wait
// for all of them before it touches LDS again, which keeps such loads out of
// the compute waves altogether.
constexpr int DOWN_THREADS = 320;
// Rows from which the decode path runs the row kernel (S, streams_out, rinv)
// before hc_down instead of having every hc_down workgroup add the squares
// (96-block chain at H = 2560, us per block: 12 rows 21.2 without it against
// 22.2 with it, 13 rows 23.5 against 22.8, 14 rows 23.0 against 22.9).
constexpr int DEC_ROWS_KERNEL_MIN = 13;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Agent-coherent (sc1) store and load: visible to workgroups on every XCD
// without writing back or invalidating a whole L2, which is what a
// device-scope fence costs on this chip (microseconds per workgroup).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this thread's memory operations have completed (vmcnt(0)):
// its stores, and its loads including those that write LDS directly.
__device__ __forceinline__ void wait_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// lds_base + 16 l (lds_base must be the same in every lane).
__device__ __forceinline__ void load_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)lds_base, 16, 0, 0);
}

// ((0 + p[0]) + p[step]) + ... + p[(n-1) step]: the slice partials of one
// output in their fixed order, for N outputs at once, loaded B at a time
// (loads past n clamped and not added). The loads of all N are issued before
// any addition, so a batch costs one memory latency.
template <int B, int N, typename L>
__device__ __forceinline__ void slice_sum_n(const float* const* p, int step, int n, L load, float* sum) {
#pragma unroll
  for (int j = 0; j < N; ++j) sum[j] = 0.0f;
  for (int s0 = 0; s0 < n; s0 += B) {
    float v[N][B];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int i = 0; i < B; ++i) v[j][i] = load(p[j] + min(s0 + i, n - 1) * step);
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int i = 0; i < B; ++i)
        if (s0 + i < n) sum[j] = sum[j] + v[j][i];
  }
}

// --------------------------------------------------------------- hc_down

// NJ: chunk slots per virtual lane, ceil(H / 2048). A row group is SLOTS / NJ
// rows whose streams (and prev_out) chunks are in registers at once, wave w
// playing quarter w of the 256 virtual lanes of each.
// RW (at most 64 RW_SLOTS chunks per branch row, H <= 2560): a row group is
// four rows instead, wave w taking row w of the group and playing all four
// quarters: lane l holds chunks 64 i + l of the row (i < ceil(NQ / 64)),
// chunk i belonging to virtual lane 64 (i mod 4) + l, so each virtual lane
// still adds its chunks in ascending order. The waves then carry equal work
// where NQ is not a multiple of 256 (H = 2560: 5 chunks per wave and group,
// against 8 for wave 0 otherwise).
// PRE: rinv of every (row, branch) is already in the workspace (from the row
// kernel that runs first with more rows, which also writes streams_out), so
// the workgroup only builds hn of its own slice.
template <DT D, int NJ, bool PRE, bool RW = false>
__global__ __launch_bounds__(DOWN_THREADS) void k_hc_down(Args a, Geometry g, float* __restrict__ partial,
                                                 void* __restrict__ hn_out, void* __restrict__ hidden,
                                                 unsigned* __restrict__ tickets, int up_prefetch,
                                                 const float* __restrict__ rinv_in, int red_rows) {
  static_assert(!RW || (NJ == 1 && !PRE), "row-per-wave groups: NJ unused, not with PRE");
  constexpr int RG = RW ? 4 : SLOTS / NJ;
  constexpr int NSL = RW ? RW_SLOTS : SLOTS;  // register slots per row group
  __shared__ __attribute__((aligned(16))) uint16_t hn_lds[DEC_ROWS * HN_LD];
  __shared__ __attribute__((aligned(16))) float w_f[4 * KSMAX * 16 / 2];
  __shared__ float ss_lds[DEC_ROWS * 4];
  __shared__ __attribute__((aligned(16))) uint16_t pf_lds[4 * 512];  // sink of the up_weight prefetch
  __shared__ int is_last;
  __shared__ __attribute__((aligned(16))) float red_st[PRE ? 1 : RED_ROWS * 64];  // the tail's slice partials
  extern __shared__ __attribute__((aligned(16))) float red_dyn[];                 // the same for PRE: [red_rows][64]
  float* const red_lds = PRE ? red_dyn : red_st;
  uint16_t* w_lds = (uint16_t*)w_f;  // [4 tiles][KS][16]
  float* br_lds = w_f;               // [C][M][64], reused by the reduction

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int b = blockIdx.x, s_in = blockIdx.y, c = blockIdx.z, NG = gridDim.x;
  const int s = c * g.SPB + s_in;      // slice index over all branches
  const int KS = g.KS, NQS = KS >> 3;  // slice length and its chunks
  const int q_lo = NQS * s_in;         // first chunk of the slice in the branch row
  const int NQ = a.H >> 3;             // chunks per branch row
  const int M = (int)a.M;
  const int kbase = c * a.H + s_in * KS;
  const bool pro = a.prev_out != nullptr;
  const uint16_t* srow0 = (const uint16_t*)a.streams + c * a.H;
  const uint16_t* prow0 = pro ? (const uint16_t*)a.prev_out : srow0;
  const uint16_t* gate0 = pro ? (const uint16_t*)a.prev_gate + c : srow0;
  uint16_t* so = !PRE && b == 0 && a.streams_out ? (uint16_t*)a.streams_out + c * a.H : nullptr;
  const int vl = 64 * wave + lane;  // this lane's virtual lane in the canonical sum of squares

  // 1. Streams (and prev_out) chunks of the first row group: chunk q_j =
  //    vl + 256 j of each row, clamped into the row (invalid slots are masked
  //    when used), rows of the group past the batch not loaded. Two register
  //    sets: the next group's loads go out while a group is processed.
  uint4 sv[2][NSL], pv[2][NSL];
  uint32_t gv[2][RG];
  auto issue = [&](int rg, auto BUF) {
    constexpr int u = decltype(BUF)::value;
    if constexpr (RW) {
      const int m = rg * RG + wave;
      if (m < M) {
#pragma unroll
        for (int i = 0; i < NSL; ++i)
          if (64 * i < NQ) {
            const int q = min(64 * i + lane, NQ - 1);
            sv[u][i] = *(const uint4*)(srow0 + (size_t)m * a.K + 8 * q);
            if (pro) pv[u][i] = *(const uint4*)(prow0 + (size_t)m * a.H + 8 * q);
          }
        gv[u][0] = pro ? gate0[m * a.C] : 0u;
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int m = rg * RG + r;
      if (m < M) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int q = min(vl + 256 * j, NQ - 1);
          sv[u][r * NJ + j] = *(const uint4*)(srow0 + (size_t)m * a.K + 8 * q);
          if (pro) pv[u][r * NJ + j] = *(const uint4*)(prow0 + (size_t)m * a.H + 8 * q);
        }
        gv[u][r] = pro ? gate0[m * a.C] : 0u;
      }
    }
  };
  const std::integral_constant<int, 0> B0{};
  const std::integral_constant<int, 1> B1{};
  const bool inj_wg = a.R >= 64 * b && a.R < 64 * b + 64;

  // Wave 4: prefetch of hc_uppre's up_weight tiles into this XCD's L2 and the
  // memory-side cache. hc_uppre's workgroups on XCD x (workgroup id mod 8, the
  // dispatch order) take features [x H/8, (x+1) H/8) of every branch, so the
  // workgroups here whose linear id is x mod 8 fetch exactly those rows, in
  // whole 128-byte lines, into an LDS area that nothing reads. The wave then
  // passes the compute waves' barriers up to the arrival counter (one per row
  // group, one for the inject tile, one for the weight tiles, two around the
  // counter) without waiting for its loads, waits for them, and ends; a
  // barrier waits only for the waves that have not ended.
  if (wave == 4) {
    if (up_prefetch) {
      const int id = b + NG * (s_in + g.SPB * c);
      const int nk = (NG * g.SPB * a.C) >> 3, k = id >> 3, x = id & 7;
      const int seg_words = a.H >> 6;  // 16-byte words of one (row, branch) segment of those features
      for (int w = lane; w < a.C * seg_words; w += 64) {
        const int pc = w / seg_words;
        const uint16_t* wu = (const uint16_t*)a.wu + pc * a.H + x * (a.H >> 3) + 8 * (w - pc * seg_words);
        for (int n = k; n < a.R; n += nk) load_lds16(wu + (size_t)n * a.K, pf_lds);
      }
    }
    const int nbar = (PRE ? 0 : (M + RG - 1) / RG) + (inj_wg ? 1 : 0) + 3;
    for (int i = 0; i < nbar; ++i) __builtin_amdgcn_s_barrier();
    wait_vm();
    return;
  }
  // PRE: this thread's chunks of the slice (rows hr and hr + 8, chunk kq):
  // S from the inputs (the prologue redone on 16 values), rinv from the
  // workspace. All loads go out before any is used.
  const int hr = tid >> 5, kq = tid & 31;  // hn role: row hr of a group, slice chunk kq (NQS <= 32)
  uint4 ps[2], pp[2];
  uint32_t pg[2];
  float prv[2];
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = min(hr + 8 * i, M - 1), q = q_lo + min(kq, NQS - 1);
      ps[i] = *(const uint4*)(srow0 + (size_t)m * a.K + 8 * q);
      pp[i] = pro ? *(const uint4*)(prow0 + (size_t)m * a.H + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
      pg[i] = pro ? gate0[m * a.C] : 0u;
      prv[i] = rinv_in[m * a.C + c];
    }
  } else {
    issue(0, B0);
  }

  // 2. norm_scale of this thread's hn chunk, then the weight tile: rows
  //    kbase .. kbase+KS of columns [64b, 64b+64) of [down | inject | 0], eight
  //    threads per row, 16 bytes each (columns past R read a valid column and
  //    are zeroed in LDS). The C inject columns are KS*C contiguous values of
  //    inject_weight, loaded as flat words by the group that holds column R.
  const uint4 nsr = *(const uint4*)((const uint16_t*)a.ns + kbase + 8 * min(kq, NQS - 1));
  uint4 wreg[KSMAX / 32];
  const int col8 = 64 * b + 8 * (tid & 7);
  const bool col_ok = col8 + 8 <= a.R;
  if (64 * b < a.R) {
    const uint16_t* wd = (const uint16_t*)a.wd + (size_t)(kbase + (tid >> 3)) * a.R + min(col8, a.R - 8);
#pragma unroll
    for (int p = 0; p < KSMAX / 32; ++p)
      if (32 * p < KS) wreg[p] = *(const uint4*)(wd + (size_t)(32 * p) * a.R);
  }
  uint4 injw = make_uint4(0u, 0u, 0u, 0u);
  if (inj_wg) injw = inject_word((const uint16_t*)a.wi, a.C, kbase, KS, tid);

  // Rows of the tile past the batch are zero.
  for (int i = tid; i < (DEC_ROWS - M) * 32; i += 256) {
    const int r = M + (i >> 5), q = i & 31;
    if (q < NQS) *(uint4*)(hn_lds + r * HN_LD + 8 * q) = make_uint4(0u, 0u, 0u, 0u);
  }

  // 3. Per row group: each wave adds the squares of its quarter of the virtual
  //    lanes; the lanes holding chunks of this slice put S there (and into
  //    streams_out, once per slice); then hn of the slice, in place, and into
  //    the workspace for hc_uppre.
  // S of one chunk of row m (prologue applied), its squares added to acc in
  // ascending order; written to the slice's hn tile (and streams_out) when
  // the chunk is in the slice.
  auto chunk = [&](int m, int q, uint4 sw, uint4 pw, float gate, float& acc) {
    float x[8];
    unpack8<D>(sw, x);
    if (pro) {
      float p[8];
      unpack8<D>(pw, p);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], gate, p[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = acc + x[e] * x[e];
    if (q >= q_lo && q < q_lo + NQS) {
      const uint4 w = pack8<D>(x);
      *(uint4*)(hn_lds + m * HN_LD + 8 * (q - q_lo)) = w;
      if (so) *(uint4*)(so + (size_t)m * a.K + 8 * q) = w;
    }
  };
  auto group = [&](int rg, auto BUF) {
    constexpr int u = decltype(BUF)::value;
    float acc[4];
    if constexpr (RW) {
      // acc[k]: this lane's virtual lane of quarter k of row rg RG + wave.
      const int m = rg * RG + wave;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = 0.0f;
      if (m < M) {
        const float gate = widen<D>(gv[u][0]);
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
          const int q = 64 * i + lane;
          if (q < NQ) chunk(m, q, sv[u][i], pv[u][i], gate, acc[i & 3]);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + xor_partner<32>(acc[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + xor_partner<16>(acc[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + xor_partner<8>(acc[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + xor_partner<4>(acc[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + xor_partner<2>(acc[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + xor_partner<1>(acc[k]);
      if (lane == 0 && m < M)
#pragma unroll
        for (int k = 0; k < 4; ++k) ss_lds[m * 4 + k] = acc[k];
    } else {
    static_assert(RG <= 8, "row group");
    float accr[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int m = rg * RG + r;
      accr[r] = 0.0f;
      if (m >= M) continue;
      const float gate = widen<D>(gv[u][r]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = vl + 256 * j;
        if (q < NQ) chunk(m, q, sv[u][r * NJ + j], pv[u][r * NJ + j], gate, accr[r]);
      }
    }
    // Each row's butterfly (the additions of wave_allsum), the rows' steps
    // interleaved so that their cross-lane latencies overlap.
#pragma unroll
    for (int r = 0; r < RG; ++r) accr[r] = accr[r] + xor_partner<32>(accr[r]);
#pragma unroll
    for (int r = 0; r < RG; ++r) accr[r] = accr[r] + xor_partner<16>(accr[r]);
#pragma unroll
    for (int r = 0; r < RG; ++r) accr[r] = accr[r] + xor_partner<8>(accr[r]);
#pragma unroll
    for (int r = 0; r < RG; ++r) accr[r] = accr[r] + xor_partner<4>(accr[r]);
#pragma unroll
    for (int r = 0; r < RG; ++r) accr[r] = accr[r] + xor_partner<2>(accr[r]);
#pragma unroll
    for (int r = 0; r < RG; ++r) accr[r] = accr[r] + xor_partner<1>(accr[r]);
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < RG; ++r)
        if (rg * RG + r < M) ss_lds[(rg * RG + r) * 4 + wave] = accr[r];
    (void)acc;
    }
    __syncthreads();
    const int m = rg * RG + hr;
    if (hr < RG && m < M && kq < NQS) {
      const float rv = rinv_from_ss(
          ss_combine(ss_lds[m * 4], ss_lds[m * 4 + 1], ss_lds[m * 4 + 2], ss_lds[m * 4 + 3]), a.Hn, a.eps);
      uint4* hp = (uint4*)(hn_lds + m * HN_LD + 8 * kq);
      float x[8], nsv[8], hv[8];
      unpack8<D>(*hp, x);
      unpack8<D>(nsr, nsv);
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = hnorm_raw(x[e], rv, nsv[e]);
      const uint4 w = pack8<D>(hv);  // rounds each hn to T
      *hp = w;
      if (b == 0) *(uint4*)((uint16_t*)hn_out + (size_t)m * a.K + kbase + 8 * kq) = w;
    }
  };
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = hr + 8 * i;
      if (m < M && kq < NQS) {
        float x[8], nsv[8], hv[8];
        unpack8<D>(ps[i], x);
        if (pro) {
          float p[8];
          unpack8<D>(pp[i], p);
          const float gate = widen<D>(pg[i]);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], gate, p[e]);
        }
        unpack8<D>(nsr, nsv);
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = hnorm_raw(x[e], prv[i], nsv[e]);
        const uint4 w = pack8<D>(hv);  // rounds each hn to T
        *(uint4*)(hn_lds + m * HN_LD + 8 * kq) = w;
        if (b == 0) *(uint4*)((uint16_t*)hn_out + (size_t)m * a.K + kbase + 8 * kq) = w;
      }
    }
  } else {
    for (int rg = 0; rg * RG < M; rg += 2) {  // groups in pairs: the register sets alternate
      if ((rg + 1) * RG < M) issue(rg + 1, B1);
      group(rg, B0);
      if ((rg + 1) * RG >= M) break;
      if ((rg + 2) * RG < M) issue(rg + 2, B0);
      group(rg + 1, B1);
    }
  }

  // 4. Weights to LDS, one [KS][16] tile per compute wave.
  if (64 * b < a.R) {
#pragma unroll
    for (int p = 0; p < KSMAX / 32; ++p)
      if (32 * p < KS) {
        const int rr = 32 * p + (tid >> 3), j = tid & 7;
        *(uint4*)(w_lds + (j >> 1) * (KSMAX * 16) + rr * 16 + 8 * (j & 1)) =
            col_ok ? wreg[p] : make_uint4(0u, 0u, 0u, 0u);
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
    const f32x4 acc = mfma_chain<D, KSMAX / 32>(hn_lds, HN_LD, w_lds + wave * (KSMAX * 16), KS, lane);  // a slice: one batch
    const int n = 16 * t + (lane & 15);
    if (n < a.R + a.C) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;
        if (m < M) st_agent(partial + (s * M + m) * g.NP + n, acc[r]);
      }
    }
  }

  // 6. Arrival counter: the last of the NS slice workgroups of tile group b
  //    adds the partials. They went out as agent-coherent stores; once those
  //    have completed, one relaxed device-scope increment publishes them.
  wait_vm();
  __syncthreads();
  unsigned* ticket = tickets + b * TICKET_STRIDE;
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(g.NS - 1);
  __syncthreads();
  if (!is_last) {
    // Next block of a chain: this workgroup's own tile of the next block's
    // down_weight (and inject_weight) rows, which the next call's workgroup
    // with this id (so on this XCD) will read, into this XCD's L2 and the
    // memory-side cache; one 16-byte load per 128-byte line. The tile groups'
    // last workgroups, still adding partials, hold this kernel open for about
    // as long as these loads take.
    if (a.next_wd && 64 * b < a.R) {
      const int cbytes = 2 * min(64, a.R - 64 * b);
      for (int i = tid; i < KS; i += 256) {
        const char* row = (const char*)a.next_wd + ((size_t)(kbase + i) * a.R + 64 * b) * 2;
        load_lds16(row, pf_lds + 512 * wave);
        if ((((uintptr_t)row & 127) + cbytes) > 128) load_lds16(row + cbytes - 16, pf_lds + 512 * wave);
      }
      if (a.next_wi && inj_wg) {
        const int bytes = KS * a.C * 2, nl = (bytes + 127) / 128;
        const char* base = (const char*)a.next_wi + (size_t)kbase * a.C * 2;
        for (int l = tid; l < nl; l += 256) load_lds16(base + min(128 * l, bytes - 16), pf_lds + 512 * wave);
      }
    }
    wait_vm();  // the prefetches have landed before the workgroup's LDS goes away
    return;
  }

  // Branch sums (slices ascending) of item = (branch, row, column of the
  // group).
  const int sstep = M * g.NP, nitems = a.C * M * 64;
  const int bra = g.SPB * M;         // partial rows of one branch: r = (c SPB + sl) M + m
  const int cpf = (PRE ? red_rows : RED_ROWS) / bra;  // branches whose partial rows one LDS fill holds
  if (cpf >= 1 && nitems > 256) {
    // The partial rows of cpf branches at a time, straight into LDS (16 bytes
    // a lane, agent-coherent like ld_agent: one memory round trip per fill),
    // then each thread adds the slices of four adjacent columns in order from
    // LDS. Columns past NP are not loaded and not read. (With one output a
    // thread, the loads into registers below are one round trip as well.)
    const int nval = min(64, g.NP - 64 * b), np = nval >> 2;  // valid columns (a multiple of 16), their 16-byte pieces
    const int pc = lane & 15;
    for (int c0 = 0; c0 < a.C; c0 += cpf) {
      const int nb = min(cpf, a.C - c0), nrow = nb * bra;
      const float* prow = partial + (size_t)c0 * bra * g.NP + 64 * b + 4 * pc;
      if (c0 > 0) __syncthreads();  // the previous fill has been read
      for (int r0 = 4 * wave; r0 < nrow; r0 += 16) {
        const int r = r0 + (lane >> 4);
        if (r < nrow && pc < np)
          __builtin_amdgcn_global_load_lds((glb_void*)(prow + (size_t)r * g.NP), (lds_void*)(red_lds + r0 * 64), 16,
                                           0, 16 /* sc1 */);
      }
      wait_vm();
      __syncthreads();
      for (int it = tid; it < nb * M * 16; it += 256) {
        const int q = it & 15, cm = it >> 4, cl = cm / M, m = cm - cl * M;
        if (q < np) {
          const float* src = red_lds + (cl * g.SPB * M + m) * 64 + 4 * q;
          f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
          for (int sl = 0; sl < g.SPB; ++sl) sum = sum + *(const f32x4*)(src + sl * M * 64);
          *(f32x4*)(br_lds + ((c0 + cl) * M + m) * 64 + 4 * q) = sum;
        }
      }
    }
  } else {
  // A thread takes N items at a time (items it, it + 256, ...), N = 1 when it
  // has one item in all, else RED_ITEMS, and issues every slice load of a
  // batch before its additions.
  auto reduce = [&](auto NC) {
    constexpr int N = decltype(NC)::value;
    for (int it0 = tid; it0 < nitems; it0 += 256 * N) {
      const float* p[N];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const int it = min(it0 + 256 * j, nitems - 1);  // past the end: a valid item, not stored
        const int nl = it & 63, cm = it >> 6, cc = cm / M, m = cm - cc * M;
        p[j] = partial + (cc * g.SPB * M + m) * g.NP + min(64 * b + nl, g.NP - 1);
      }
      float sum[N];
      slice_sum_n<RED_BATCH, N>(p, sstep, g.SPB, ld_agent, sum);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const int it = it0 + 256 * j;
        if (it < nitems) {
          const int nl = it & 63, cm = it >> 6, cc = cm / M, m = cm - cc * M;
          br_lds[(cc * M + m) * 64 + nl] = sum[j];
        }
      }
    }
  };
  if (nitems <= 256) reduce(std::integral_constant<int, 1>{});
  else reduce(std::integral_constant<int, RED_ITEMS>{});
  }
  __syncthreads();
  // Totals over branches (ascending), then ScaledSiLU -> hidden or the gate.
  for (int it = tid; it < M * 64; it += 256) {
    const int m = it >> 6, nl = it & 63, n = 64 * b + nl;
    if (n < a.R + a.C) {
      float tot = 0.0f;
      for (int cc = 0; cc < a.C; ++cc) tot = tot + br_lds[(cc * M + m) * 64 + nl];
      finish_down_inject<D>(a, m, n, tot, hidden);
    }
  }
  if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // zero for the next call
  wait_vm();
}

// --------------------------------------------------------------- hc_uppre

constexpr int HIDREG = 4;  // hidden chunks a thread holds in registers (more rows go through a loop)

// LDS of hc_uppre: hidden tile [16][R + 8] (T), up_weight tile [C][R][16]
// (T) and products [C][16][16] (fp32).
size_t uppre_lds_bytes(int C, int R) {
  return (size_t)DEC_ROWS * (R + 8) * 2 + (size_t)C * R * 16 * 2 + (size_t)C * 256 * 4;
}

template <DT D>
__global__ __launch_bounds__(1024) void k_hc_uppre(Args a, const void* __restrict__ hn_in,
                                                  const void* __restrict__ hidden) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int R = a.R, HLD = R + 8, R8 = R >> 3;
  uint16_t* hid_lds = (uint16_t*)smem;             // [16][R + 8]
  uint16_t* wu_lds = hid_lds + DEC_ROWS * HLD;     // [C][R][16]
  float* e_lds = (float*)(wu_lds + a.C * R * 16);  // [C][16][16]
  // Waves 0..C-1 run the chain of branch c = wave; waves C..2C-1 only help
  // load the up_weight tiles (odd 32-row pieces), so each wave issues half.
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool cw = wave < a.C;
  const int c = cw ? wave : wave - a.C;
  const int nthreads = blockDim.x;
  const int M = (int)a.M;
  // Workgroups on one XCD (blockIdx.x mod 8) take adjacent feature blocks;
  // hc_down prefetched exactly those up_weight lines into that XCD's L2.
  const int nhb = a.H >> 4;
  const int hb = (nhb & 7) == 0 ? (int)(blockIdx.x & 7) * (nhb >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int h0 = hb * 16, h = h0 + (lane & 15);
  const int kc = c * a.H + h;

  // 1. The up_weight tile of branch c, rows 0..R-1, columns c*H + h0 .. +16,
  //    straight from memory into LDS as [R][16] (lane l of the wave carries
  //    row 32p + l/2, half l%2): even pieces p from wave c, odd ones from
  //    wave C + c. The tiles are the long pole, so they go out first.
  const uint16_t* wu = (const uint16_t*)a.wu + kc - (lane & 15) + 8 * (lane & 1) + (size_t)(lane >> 1) * a.K;
  for (int p = cw ? 0 : 1; 32 * p < R; p += 2) load_lds16(wu + (size_t)(32 * p) * a.K, wu_lds + (c * R + 32 * p) * 16);

  // 2. hn of this lane's four outputs (rows 4*(lane/16) + r, clamped into the
  //    batch: every load is unconditional; rows past the batch are not used).
  uint32_t hraw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hraw[r] = ((const uint16_t*)hn_in)[(size_t)min(4 * (lane >> 4) + r, M - 1) * a.K + kc];

  // 3. This thread's first chunks of the hidden rows of the batch.
  const int hchunks = M * R8;
  const uint16_t* hid = (const uint16_t*)hidden;
  uint4 hreg[HIDREG];
#pragma unroll
  for (int i = 0; i < HIDREG; ++i) hreg[i] = *(const uint4*)(hid + 8 * min(tid + i * nthreads, hchunks - 1));

  // 4. The hidden tile [16][R] in LDS (rows beyond the batch zero).
  for (int ch = hchunks + tid; ch < DEC_ROWS * R8; ch += nthreads) {
    const int r = ch / R8;
    *(uint4*)(hid_lds + r * HLD + 8 * (ch - r * R8)) = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < HIDREG; ++i) {
    const int ch = tid + i * nthreads, r = ch / R8;
    if (ch < hchunks) *(uint4*)(hid_lds + r * HLD + 8 * (ch - r * R8)) = hreg[i];
  }
  for (int ch = tid + HIDREG * nthreads; ch < hchunks; ch += nthreads) {
    const int r = ch / R8;
    *(uint4*)(hid_lds + r * HLD + 8 * (ch - r * R8)) = *(const uint4*)(hid + 8 * ch);
  }

  // 5. Once the up_weight tile has landed: the up chain; g; the pre-mix over
  //    branches.
  wait_vm();
  __syncthreads();
  if (cw) {
    const f32x4 acc = mfma_chain<D>(hid_lds, HLD, wu_lds + c * R * 16, R, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 4 * (lane >> 4) + r;
      if (rr < M) e_lds[c * 256 + rr * 16 + (lane & 15)] = widen<D>(hraw[r]) * up_gate<D>(acc[r]);
    }
  }
  __syncthreads();
  for (int i = tid; i < M * 16; i += nthreads) {
    float sum = 0.0f;
    for (int cc = 0; cc < a.C; ++cc) sum = sum + e_lds[cc * 256 + i];
    st<D>(a.pre, (size_t)(i >> 4) * a.H + h0 + (i & 15), rT<D>(a.rs * sum));
  }
}

// --------------------------------------------------------------- prefill helper

// Fixed-order reduction of per-branch fp32 partials [C][M][NP] (one partial
// per branch, each already summed over its slices in order) + the down/inject
// epilogue (branch_reduce_items). Used by the prefill path.
template <DT D>
__global__ __launch_bounds__(256) void k_branch_reduce(Args a, int NP, const float* __restrict__ partial,
                                                       void* __restrict__ hidden) {
  branch_reduce_items<D>(a, NP, partial, hidden, (int64_t)blockIdx.x * 256 + threadIdx.x, (int64_t)gridDim.x * 256);
}

// Per-slice partials [C * SPB][M][NP] (the prefill path's slice mode): per
// output, the slices of each branch in order, then the branches in order (the
// decode path's order), then the down/inject epilogue. A workgroup takes 64
// consecutive outputs with one wave per branch: wave c sums branch c's slices
// for its lane's output (RED_BATCH loads issued before their additions), and
// wave 0 adds the C branch sums in ascending c.
template <DT D>
__global__ __launch_bounds__(512) void k_slice_reduce(Args a, int NP, int SPB, const float* __restrict__ partial,
                                                      void* __restrict__ hidden) {
  __shared__ float bs[8][64];
  const int NC = a.R + a.C, c = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t total = a.M * NC, pstep = a.M * NP;
  for (int64_t g0 = (int64_t)blockIdx.x * 64; g0 < total; g0 += (int64_t)gridDim.x * 64) {
    const int64_t gi = min(g0 + lane, total - 1);  // past the end: a valid output, not stored
    const int64_t m = gi / NC;
    const int n = (int)(gi - m * NC);
    const float* p = partial + ((int64_t)c * SPB * a.M + m) * NP + n;
    float br = 0.0f;
    for (int s0 = 0; s0 < SPB; s0 += RED_BATCH) {
      float v[RED_BATCH];
#pragma unroll
      for (int i = 0; i < RED_BATCH; ++i) v[i] = p[(int64_t)min(s0 + i, SPB - 1) * pstep];
#pragma unroll
      for (int i = 0; i < RED_BATCH; ++i)
        if (s0 + i < SPB) br = br + v[i];
    }
    bs[c][lane] = br;
    __syncthreads();
    if (c == 0 && g0 + lane < total) {
      float tot = 0.0f;
      for (int j = 0; j < a.C; ++j) tot = tot + bs[j][lane];
      finish_down_inject<D>(a, m, n, tot, hidden);
    }
    __syncthreads();  // bs is reused by the next 64 outputs
  }
}

// --------------------------------------------------------------- launchers

// Chunk slots per virtual lane for a branch of H features (H <= DECODE_MAX_H).
static int chunk_slots(int H) {
  const int nq = H >> 3;
  return nq <= 256 ? 1 : nq <= 512 ? 2 : 4;
}

template <DT D, int NJ, bool PRE, bool RW = false>
static hipError_t launch_down(const Args& a, const Geometry& g, float* partial, void* hn, void* hidden,
                              unsigned* tickets, const float* rinv, hipStream_t s, Marks* mk) {
  const dim3 grid((unsigned)((g.NT + 3) / 4), (unsigned)g.SPB, (unsigned)a.C);
  // The prefetch assumes hc_uppre's XCD-aware feature mapping and an equal
  // share of hc_down workgroups per XCD.
  const int nwg = (int)(grid.x * grid.y * grid.z);
  const int up_prefetch = ((a.H >> 4) & 7) == 0 && (nwg & 7) == 0;
  // The tail's LDS (96 KB) leaves one workgroup per compute unit; only the
  // row-kernel-first variant (PRE, few registers) could otherwise have more,
  // which counts once its workgroups outnumber the compute units.
  const int red_rows = PRE && nwg <= device_compute_units() ? RED_ROWS : 0;
  const size_t lds = (size_t)red_rows * 64 * sizeof(float);
  if (lds > 0) {
    const hipError_t e = allow_dynamic_lds((const void*)k_hc_down<D, NJ, PRE, RW>, D == DT::BF16 ? 20 : 21, lds);
    if (e != hipSuccess) return e;
  }
  return launch(mk, k_hc_down<D, NJ, PRE, RW>, grid, dim3(DOWN_THREADS), lds, s, a, g, partial, hn, hidden, tickets,
                up_prefetch, rinv, red_rows);
}

template <DT D>
static hipError_t run_decode(const Args& a, char* ws, const Workspace& w, const Geometry& g, hipStream_t s,
                             Marks* mk) {
  void* hn = ws + w.hn;
  void* hidden = ws + w.hidden;
  float* partial = (float*)(ws + w.partial);
  unsigned* tickets = (unsigned*)(ws + w.tickets);
  float* rinv = (float*)(ws + w.rinv);
  const size_t lds = uppre_lds_bytes(a.C, a.R);
  hipError_t e = allow_dynamic_lds((const void*)k_hc_uppre<D>, D == DT::BF16 ? 0 : 1, lds);
  if (e != hipSuccess) return e;
  if (a.M >= DEC_ROWS_KERNEL_MIN) {
    // Every workgroup of hc_down would otherwise add the squares of all rows of
    // its branch: from this many rows a row kernel does that once.
    e = launch_rows_rms(a, (int)D, rinv, s, mk);
    if (e != hipSuccess) return e;
    e = launch_down<D, 1, true>(a, g, partial, hn, hidden, tickets, rinv, s, mk);
  } else if (a.M >= 4 && a.H <= 8 * 64 * RW_SLOTS && ((a.H >> 3) & 255) != 0) {
    // Rows of four, one per wave: the waves' shares are unequal otherwise.
    e = launch_down<D, 1, false, true>(a, g, partial, hn, hidden, tickets, nullptr, s, mk);
  } else {
    switch (chunk_slots(a.H)) {
      case 1: e = launch_down<D, 1, false>(a, g, partial, hn, hidden, tickets, nullptr, s, mk); break;
      case 2: e = launch_down<D, 2, false>(a, g, partial, hn, hidden, tickets, nullptr, s, mk); break;
      default: e = launch_down<D, 4, false>(a, g, partial, hn, hidden, tickets, nullptr, s, mk); break;
    }
  }
  if (e != hipSuccess) return e;
  return launch(mk, k_hc_uppre<D>, dim3((unsigned)(a.H / 16)), dim3((unsigned)(128 * a.C)), lds, s, a,
                (const void*)hn, (const void*)hidden);
}

hipError_t launch_decode(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                         hipStream_t s, Marks* mk) {
  if (a.M > DEC_ROWS || a.H > DECODE_MAX_H || g.KS > KSMAX) return hipErrorInvalidValue;
  if (dtype == 16) return run_decode<DT::BF16>(a, ws, w, g, s, mk);
  if (dtype == 10) return run_decode<DT::F16>(a, ws, w, g, s, mk);
  return hipErrorInvalidValue;
}

hipError_t launch_branch_reduce(const Args& a, int dtype, int NP, const float* partial, void* hidden,
                                hipStream_t s, Marks* mk) {
  const int64_t wg = (a.M * (NP >> 2) + 255) / 256;
  const dim3 grid((unsigned)(wg < 65536 ? wg : 65536));  // grid-stride beyond that
  if (NP % 16 != 0 || a.R % 4 != 0) return hipErrorInvalidValue;
  if (dtype == 16) return launch(mk, k_branch_reduce<DT::BF16>, grid, dim3(256), 0, s, a, NP, partial, hidden);
  if (dtype == 10) return launch(mk, k_branch_reduce<DT::F16>, grid, dim3(256), 0, s, a, NP, partial, hidden);
  return hipErrorInvalidValue;
}

hipError_t launch_slice_reduce(const Args& a, int dtype, int NP, int SPB, const float* partial, void* hidden,
                               hipStream_t s, Marks* mk) {
  const int64_t wg = (a.M * (a.R + a.C) + 63) / 64;  // 64 outputs per workgroup
  const dim3 grid((unsigned)(wg < 65536 ? wg : 65536));  // grid-stride beyond that
  if (a.C < 1 || a.C > 8) return hipErrorInvalidValue;
  const dim3 block((unsigned)(64 * a.C));  // one wave per branch
  if (dtype == 16) return launch(mk, k_slice_reduce<DT::BF16>, grid, block, 0, s, a, NP, SPB, partial, hidden);
  if (dtype == 10) return launch(mk, k_slice_reduce<DT::F16>, grid, block, 0, s, a, NP, SPB, partial, hidden);
  return hipErrorInvalidValue;
}

}  // namespace hc
