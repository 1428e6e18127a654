// Zero-padded copies for the matrix-core paths. Their kernels tile every
// branch in 32-feature steps and the rank in 32-column steps; a 16-bit
// problem whose H or R is not a multiple of 32 runs them on a copy padded
// with zeros to the next multiples (H32, R32), and its outputs are copied back.
// Zero features and zero rank columns add exact zeros to every sum of the
// block (onnxruntime PR #33384, "Schema summary": S, hn, the three
// projections and the pre-mix are sums over features or rank), so the padded
// problem computes the caller's one; only the RMS mean keeps dividing by the
// caller's H.
//
// One kernel does every copy of a call: a table of jobs, each a 2-level row
// layout (outer index a, inner index b) whose destination rows take the first
// `ncopy` elements of the matching source row, or zeros where that row or
// element does not exist. A lane copies 8-element chunks of destination rows,
// with 16-byte accesses where the address is aligned and the chunk whole,
// element by element otherwise. A unit of work is 64 chunks of one row, or
// several whole rows when a row has at most 64 chunks; a wave takes UNITS
// consecutive units and issues all their loads before its stores.
#include "hc_internal.h"

namespace hc {

namespace {

constexpr int WAVES = 4;  // waves per workgroup
constexpr int UNITS = 1;  // units (64 chunks of a row, or whole short rows) per wave: 1, 4 and 8
                          // copy the decode block's weights in 6.0, 6.5 and 7.6 us

struct CopyTable {
  CopyJob j[COPY_JOBS];
  int n;
};

__device__ __forceinline__ bool aligned_16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Where the lane's chunk of work unit `unit` sits: destination row q and
// element x of it; false when the lane has no chunk there. I is the index
// type: 32-bit when every row and unit index of the job fits.
template <typename I>
__device__ __forceinline__ bool locate(const CopyJob& J, I unit, int lane, I& q, int& x) {
  int ck;
  if (J.rpw > 0) {
    const int sr = lane / J.cpr;
    ck = lane - sr * J.cpr;
    q = unit * (I)J.rpw + (I)sr;
    if (sr >= J.rpw || q >= (I)(J.dst_a * J.dst_b)) return false;
  } else {
    q = unit / (I)J.spr;
    ck = (int)(unit - q * (I)J.spr) * 64 + lane;
    if (ck >= J.cpr) return false;
  }
  x = 8 * ck;
  return true;
}

template <typename I>
__device__ __forceinline__ void copy_units(const CopyJob& J, I first, int lane) {
  // Every load of the wave's units is issued before the first store.
  uint32_t w[UNITS][4];
  I q[UNITS];
  int x[UNITS];
  bool on[UNITS];
#pragma unroll
  for (int u = 0; u < UNITS; ++u) {
    w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0u;
    on[u] = first + (I)u < (I)J.units && locate<I>(J, first + (I)u, lane, q[u], x[u]);
    if (!on[u]) continue;
    const I a = q[u] / (I)J.dst_b;
    const int b = (int)(q[u] - a * (I)J.dst_b);
    if (a < (I)J.src_a && b < J.src_b && x[u] < J.ncopy) {
      const uint16_t* s = J.src + (((int64_t)a * J.src_b + b) * J.src_pitch + x[u]);
      if (x[u] + 8 <= J.ncopy && aligned_16(s)) {
        const uint4 v = *(const uint4*)s;
        w[u][0] = v.x, w[u][1] = v.y, w[u][2] = v.z, w[u][3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (x[u] + i < J.ncopy) w[u][i >> 1] |= (uint32_t)s[i] << (16 * (i & 1));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UNITS; ++u) {
    if (!on[u]) continue;
    uint16_t* d = J.dst + ((int64_t)q[u] * J.dst_pitch + x[u]);
    if (x[u] + 8 <= J.dst_pitch && aligned_16(d)) {
      *(uint4*)d = make_uint4(w[u][0], w[u][1], w[u][2], w[u][3]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (x[u] + i < J.dst_pitch) d[i] = (uint16_t)(w[u][i >> 1] >> (16 * (i & 1)));
    }
  }
}

__global__ __launch_bounds__(256) void k_copy_pad(CopyTable t) {
  int ji = 0;
  while (ji + 1 < t.n && (int64_t)blockIdx.x >= t.j[ji + 1].wg0) ++ji;
  const CopyJob& J = t.j[ji];
  const int lane = (int)(threadIdx.x & 63);
  const int64_t first =
      (((int64_t)blockIdx.x - J.wg0) * WAVES + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))) * UNITS;
  if (J.narrow)
    copy_units<uint32_t>(J, (uint32_t)first, lane);
  else
    copy_units<int64_t>(J, first, lane);
}

}  // namespace

hipError_t launch_copy(const CopyJob* jobs, int n, hipStream_t s, Marks* mk) {
  if (n < 0 || n > COPY_JOBS) return hipErrorInvalidValue;
  CopyTable t{};
  int64_t wg = 0;
  for (int i = 0; i < n; ++i) {
    CopyJob J = jobs[i];
    if (!J.dst || J.dst_a < 0 || J.src_a < 0 || J.src_b < 1 || J.dst_b < 1 || J.dst_pitch < 1 || J.ncopy < 0 ||
        J.ncopy > J.dst_pitch || J.src_pitch < J.ncopy || (J.ncopy > 0 && J.src_a > 0 && !J.src))
      return hipErrorInvalidValue;
    if (J.dst_a == 0) continue;
    const int64_t rows = J.dst_a * J.dst_b;
    J.cpr = (J.dst_pitch + 7) / 8;
    J.rpw = J.cpr <= 64 ? 64 / J.cpr : 0;
    J.spr = J.cpr <= 64 ? 1 : (J.cpr + 63) / 64;
    J.units = J.rpw > 0 ? (rows + J.rpw - 1) / J.rpw : rows * J.spr;
    J.narrow = rows * J.spr + (int64_t)WAVES * UNITS * 64 < (1LL << 31) && J.src_a < (1LL << 31) ? 1 : 0;
    J.wg0 = wg;
    wg += (J.units + WAVES * UNITS - 1) / (WAVES * UNITS);
    t.j[t.n++] = J;
  }
  if (wg == 0) return hipSuccess;
  if (wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch(mk, k_copy_pad, dim3((unsigned)wg), dim3(64 * WAVES), 0, s, t);
}

}  // namespace hc
