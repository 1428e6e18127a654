// Pieces shared by the two matrix-core paths (decode and prefill) of the
// HyperConnectionLowRankMix block. Both paths call these functions in the same
// order, so a row's bits do not depend on which path or row count produced it.
//
// Canonical order of the per-branch sum of squares: the comment on ss_combine()
// in hc_device.h. Canonical order of the down/inject dot products (fixed, per the
// "Numerics contract" of onnxruntime PR #33384: fixed accumulation order, fp32):
//   chain(c, s)  = one v_mfma_f32_16x16x32 chain over the KS/32 chunks of slice
//                  s of branch c, k ascending, starting from zero;
//   branch(c)    = ((0 + chain(c,0)) + chain(c,1)) + ... (slices ascending);
//   total        = ((0 + branch(0)) + branch(1)) + ... (branches ascending).
// The up projection is one chain over R in chunks of 32, n ascending.
// The pre-mix is ((0 + hn_0*g_0) + hn_1*g_1) + ... over branches ascending.
#pragma once

#include "hc_device.h"
#include "hc_internal.h"

namespace hc {

// Eight consecutive elements of S for row-start pointers srow (streams of the
// branch) and prow (prev_block_output row, or null), chunk ch (elements 8ch..8ch+7).
template <DT D>
__device__ __forceinline__ void load_S8(const uint16_t* srow, const uint16_t* prow, float q, int ch,
                                        float* x) {
  unpack8<D>(*(const uint4*)(srow + 8 * ch), x);
  if (prow) {
    float p[8];
    unpack8<D>(*(const uint4*)(prow + 8 * ch), p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = prologue<D>(x[e], q, p[e]);
  }
}

// Row pointers for S of (row m, branch c): streams and prologue inputs.
struct SRow {
  const uint16_t* s;
  const uint16_t* p;
  float q;
};

template <DT D>
__device__ __forceinline__ SRow s_row(const Args& a, int64_t m, int c) {
  SRow r;
  r.s = (const uint16_t*)a.streams + m * a.K + (int64_t)c * a.H;
  r.p = a.prev_out ? (const uint16_t*)a.prev_out + m * a.H : nullptr;
  r.q = a.prev_out ? ld<D>(a.prev_gate, m * a.C + c) : 0.0f;
  return r;
}

// Canonical sum of squares of S over branch c of row m (one wave), vectorised:
// lane L plays the virtual lanes L, L+64, L+128 and L+192 of that order.
// When so_row is not null the S values are also stored there (streams_out of
// the branch).
template <DT D>
__device__ __forceinline__ float branch_sumsq_vec(const SRow& r, int H, int lane,
                                                  uint16_t* so_row = nullptr) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int NQ = H >> 3;
  for (int q0 = 0; q0 < NQ; q0 += 256) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = q0 + 64 * i + lane;
      if (ch < NQ) {
        float x[8];
        load_S8<D>(r.s, r.p, r.q, ch, x);
        if (so_row) *(uint4*)(so_row + 8 * ch) = pack8<D>(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i] = acc[i] + x[e] * x[e];
      }
    }
  }
  return ss_combine(wave_allsum(acc[0]), wave_allsum(acc[1]), wave_allsum(acc[2]), wave_allsum(acc[3]));
}

// S value at (m, c, h): from streams_out when it was written earlier in the
// stream, otherwise recomputed (same bits).
template <DT D>
__device__ __forceinline__ float S_at(const Args& a, int64_t m, int c, int h) {
  const int64_t k = m * a.K + (int64_t)c * a.H + h;
  if (a.streams_out) return ld<D>(a.streams_out, k);
  float s = ld<D>(a.streams, k);
  if (a.prev_out) s = prologue<D>(s, ld<D>(a.prev_gate, m * a.C + c), ld<D>(a.prev_out, m * a.H + h));
  return s;
}

// Eight S values at (m, c, 8ch .. 8ch+7), same source rule as S_at.
template <DT D>
__device__ __forceinline__ void S_at8(const Args& a, int64_t m, int c, int ch, float* x) {
  if (a.streams_out) {
    unpack8<D>(*(const uint4*)((const uint16_t*)a.streams_out + m * a.K + (int64_t)c * a.H + 8 * ch), x);
  } else {
    const SRow r = s_row<D>(a, m, c);
    load_S8<D>(r.s, r.p, r.q, ch, x);
  }
}

// One chain of 16x16x32 matrix-core steps over k = 0 .. klen-1 (klen a
// multiple of 32): A from a row-major [16][lda] LDS tile, B from a [klen][16]
// LDS tile. The fragments of up to CB steps are read before the first of
// their matrix ops (reads past klen are clamped and their steps skipped), so
// a chain of up to CB steps pays the LDS latency once. Accumulation order:
// k ascending.
constexpr int CB = 10;  // steps whose fragments are read at once (NB: the same, per call site)
template <DT D, int NB = CB>
__device__ __forceinline__ f32x4 mfma_chain(const uint16_t* a_tile, int lda, const uint16_t* b_tile, int klen,
                                            int lane) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < klen; k0 += 32 * NB) {
    s16x8 af[NB], bf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int kk = min(k0 + 32 * i, klen - 32);
      af[i] = lds_afrag(a_tile, lda, kk, lane);
      bf[i] = lds_bfrag(b_tile, kk, lane);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (k0 + 32 * i < klen) acc = mfma<D>(af[i], bf[i], acc);
  }
  return acc;
}

// The inject weights of rows [k0, k0 + nrows) are nrows*C contiguous 16-bit
// values. They are loaded as flat 16-byte words (word t holds values
// 8t .. 8t+7; k0*C and nrows*C are multiples of 8) and scattered into an LDS
// tile [nrows][16] (columns C..15 zero) once the loads are in. Threads past
// the last word load the last word again (never scattered): the load is
// unconditional, so no branch merges its register and the compiler need not
// wait for it before the rest of the loads are issued.
__device__ __forceinline__ uint4 inject_word(const uint16_t* wi, int C, int64_t k0, int nrows, int t) {
  const int last = ((nrows * C) >> 3) - 1;
  return *(const uint4*)(wi + k0 * C + 8 * (t < last ? t : last));
}

__device__ __forceinline__ void inject_scatter(uint16_t* tile, int C, int nrows, int t, uint4 v) {
  if (t >= (nrows * C) >> 3) return;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int f = 8 * t + e, row = f / C, col = f - row * C;
    tile[row * 16 + col] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

// B fragment of the inject tile (columns 0..C-1 of a 16-column tile, zero
// beyond) straight from the flat inject values of 32 rows, [32][C] in LDS:
// the same eight values per lane that lds_bfrag() returns for the tile.
__device__ __forceinline__ s16x8 inject_bfrag(const uint16_t* flat, int C, int lane) {
  const int col = lane & 15, row0 = 8 * (lane >> 4);
  s16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = col < C ? (short)flat[(row0 + e) * C + col] : (short)0;
  return v;
}

// Epilogue of one down/inject column n of row m from its fp32 total:
// down -> ScaledSiLU -> hidden (workspace), or inject -> post_gate (output).
template <DT D>
__device__ __forceinline__ void finish_down_inject(const Args& a, int64_t m, int n, float total,
                                                   void* hidden) {
  if (n < a.R) {
    st<D>(hidden, m * a.R + n, scaled_silu<D>(rT<D>(total), a.alpha));
  } else if (n < a.R + a.C) {
    st<D>(a.post, m * a.C + (n - a.R), post_gate<D>(rT<D>(total), a.gate_div, a.gate_mul));
  }
}

// Fixed-order reduction of per-branch fp32 partials [C][M][NP] (one partial
// per branch, each already summed over its slices in order) + the down/inject
// epilogue, for items start, start + stride, ... An item is four adjacent
// columns of a row: one 16-byte load per branch (NP is a multiple of 16), the
// branches added in ascending c, the four hidden values stored as one 8-byte
// word.
template <DT D>
__device__ __forceinline__ void branch_reduce_items(const Args& a, int NP, const float* __restrict__ partial,
                                                    void* __restrict__ hidden, int64_t start, int64_t stride) {
  const int nq = NP >> 2;  // column quads per row
  const int64_t total = a.M * nq;
  for (int64_t gi = start; gi < total; gi += stride) {
    const int64_t m = gi / nq;
    const int n0 = 4 * (int)(gi - m * nq);
    if (n0 >= a.R + a.C) continue;
    f32x4 v[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      v[cc] = cc < a.C ? *(const f32x4*)(partial + ((int64_t)cc * a.M + m) * NP + n0)
                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 tot = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      if (cc < a.C) tot = tot + v[cc];
    if (n0 + 4 <= a.R) {  // four hidden values (R is a multiple of 4 on this path)
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = to_bits<D>(scaled_silu<D>(rT<D>(tot[e]), a.alpha));
      *(uint2*)((uint16_t*)hidden + m * a.R + n0) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) finish_down_inject<D>(a, m, n0 + e, tot[e], hidden);
    }
  }
}

// Pre-mix term of (row m, branch c, feature h) from the fp32 up sum.
template <DT D>
__device__ __forceinline__ float premix_term(const Args& a, const float* rinv, int64_t m, int c, int h,
                                             float up_acc) {
  const float g = up_gate<D>(up_acc);
  const float hn = hnorm<D>(S_at<D>(a, m, c, h), rinv[m * a.C + c], ld<D>(a.ns, (int64_t)c * a.H + h));
  return hn * g;
}

}  // namespace hc
