// Internal interfaces between the C-ABI layer (hc_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace hc {

// Everything a kernel needs about one call, passed by value.
struct Args {
  const void* streams;
  const void* ns;         // norm_scale [K]
  const void* wd;         // down_weight [K, R]
  const void* wu;         // up_weight [R, K]
  const void* wi;         // inject_weight [K, C]
  const void* prev_out;   // [M, H] or null
  const void* prev_gate;  // [M, C] or null
  void* pre;              // [M, H]
  void* post;             // [M, C]
  void* streams_out;      // [M, K] or null
  const void* next_wd;    // next block's down_weight [K, R], or null: read into cache only (decode)
  const void* next_wi;    // next block's inject_weight [K, C], or null: likewise
  int64_t M;
  int C, H, R, K;
  int Hn;                 // features per branch that the RMS mean divides by: H, or the problem's own H
                          // when H was zero-padded to a multiple of 32 (padded features are 0)
  float eps, rs, alpha, gate_div, gate_mul;
};

enum Path : int { PATH_AUTO = 0, PATH_DECODE = 1, PATH_PREFILL = 2, PATH_GENERIC = 3 };

// Geometry shared by the matrix-core paths. K is cut into slices of KS
// columns inside one branch (KS is a function of H only); each slice's dot
// products are one chain of 16x16x32 matrix-core steps in ascending k, and the
// slice results are added in ascending slice order. NT output tiles of 16
// columns cover down (R/16 tiles) plus one tile holding the C inject columns.
struct Geometry {
  int KS;    // slice length (multiple of 32, divides H, <= 256)
  int SPB;   // slices per branch = H / KS
  int NS;    // slices = C * SPB
  int NT;    // output tiles = R/16 + 1
  int NP;    // padded output columns = 16 * NT
};

Geometry make_geometry(int C, int H, int R);
// Widest branch the decode kernels take (four 8-element chunks per lane of
// each of the 256 virtual lanes of the canonical sum of squares).
constexpr int DECODE_MAX_H = 8192;
// Slice length rule: the largest multiple of 32 that divides H and is <= 256 (0 if none).
int slice_length(int H);

// Workspace carve-up (byte offsets, 256-byte aligned). The decode tickets
// come first: they must be zero before a workspace's first use, and every
// call leaves them zero.
struct Workspace {
  size_t tickets;   // uint32 counters, TICKET_STRIDE apart, one per decode tile group, in [0, TICKETS_BYTES)
  size_t hn;        // T [M, K]: hn of every row (decode only)
  size_t rinv;      // fp32 [M, C]
  size_t hidden;    // T [M, R]
  size_t partial;   // fp32 [NS, M, NP] (decode), [C, M, NP] (prefill) or [P, M, R + C] (generic)
  size_t wut;       // T [K, R]: up_weight transposed (prefill, fast up kernel only)
  size_t gtab;      // T table of the 16-bit sigmoid (prefill, fast up kernel only)
  size_t prod;      // fp32 [M, C, H]: hn * g per branch (prefill with at most 128 rows)
  size_t bytes;
};

Workspace workspace_layout(int path, int dtype, int64_t M, int C, int H, int R);
// Parts of K that the generic down kernel spreads over workgroups: a function
// of K alone, so that a row's summation order does not depend on the row count.
inline int generic_parts(int64_t K) {
  const int64_t p = (K + 639) / 640;
  return (int)(p < 1 ? 1 : p > 32 ? 32 : p);
}
// Arrival counters sit 256 bytes apart: atomics on one cache line serialize
// at the memory side even when they hit different words.
constexpr int TICKET_STRIDE = 64;
// The counters' prefix of every workspace: one counter per decode tile group
// of 64 columns, ceil((R/16 + 1) / 4) <= 9 of them for R <= 512 (the decode
// path's largest rank), TICKET_STRIDE words apart.
constexpr size_t TICKETS_BYTES = 4096;
static_assert(((512 / 16 + 1 + 3) / 4) * TICKET_STRIDE * 4 <= TICKETS_BYTES, "counter prefix");

// Raises a kernel's dynamic-LDS limit once per device (not a stream operation,
// so it is kept out of the per-call path that callers may capture in a graph).
hipError_t allow_dynamic_lds(const void* kernel, int slot, size_t bytes);
// Compute units of the current device, looked up once per device.
int device_compute_units();

// Optional timing: caller-created HIP events, two per kernel. The i-th kernel
// of a call is dispatched with events[2i] and events[2i+1] as its start and
// stop events, which the runtime stamps from the dispatch itself, so the
// interval is the kernel's own execution time with nothing queued between.
struct Marks {
  void* const* ev;
  int n;
  int used;
};

// Launches kernel k (plain launch when mk carries no events).
template <typename... P, typename... A>
inline hipError_t launch(Marks* mk, void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         A... args) {
  std::tuple<P...> params{static_cast<P>(args)...};
  void* argv[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&argv](auto&... x) {
    int i = 0;
    ((argv[i++] = (void*)&x), ...);
  }, params);
  if (!mk || !mk->ev) return hipLaunchKernel((const void*)k, grid, block, argv, lds, s);
  if (mk->used + 2 > mk->n) return hipErrorInvalidValue;
  hipEvent_t e0 = (hipEvent_t)mk->ev[mk->used], e1 = (hipEvent_t)mk->ev[mk->used + 1];
  mk->used += 2;
  return hipExtLaunchKernel((const void*)k, grid, block, argv, lds, s, e0, e1, 0);
}

hipError_t launch_generic(const Args& a, int dtype, char* ws, const Workspace& w, hipStream_t s, Marks* mk);
hipError_t launch_decode(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                         hipStream_t s, Marks* mk);
// Fixed-order reduction of per-branch fp32 partials [C][M][NP] + the down/inject epilogue.
hipError_t launch_branch_reduce(const Args& a, int dtype, int NP, const float* partial, void* hidden,
                                hipStream_t s, Marks* mk);
hipError_t launch_slice_reduce(const Args& a, int dtype, int NP, int SPB, const float* partial, void* hidden,
                               hipStream_t s, Marks* mk);
// Whether the prefill path's down kernel runs one slice per workgroup
// (per-slice partials [C * SPB][M][NP]) rather than one branch.
bool prefill_slices(int64_t M, int C, int H, int R);

// The prefill path's row kernel (S, streams_out, the canonical sum of squares
// and rinv [M, C]), also run by the decode path from a few rows on.
hipError_t launch_rows_rms(const Args& a, int dtype, float* rinv, hipStream_t s, Marks* mk);

// Standalone inv_rms: one fp32 value per row of x [rows, dim] (dtype: ONNX code).
hipError_t launch_inv_rms(const void* x, float* out, int64_t rows, int64_t dim, int dtype, float eps,
                          hipStream_t s);

hipError_t launch_prefill(const Args& a, int dtype, char* ws, const Workspace& w, const Geometry& g,
                          hipStream_t s, Marks* mk);

// One copy of 16-bit elements between row layouts, for problems the
// matrix-core paths run zero-padded. The destination holds dst_a x dst_b rows
// of dst_pitch elements (row index a * dst_b + b); its row (a, b) takes the
// first ncopy elements of source row (a, b) (row index a * src_b + b, src_pitch
// elements apart) when a < src_a and b < src_b, and is zero everywhere else.
// The caller fills the geometry; launch_copy fills the rest.
struct CopyJob {
  const uint16_t* src;
  uint16_t* dst;
  int64_t src_a, dst_a;
  int src_b, dst_b;
  int src_pitch, dst_pitch, ncopy;
  int cpr;        // 8-element chunks per destination row
  int rpw;        // rows one unit copies when a row has at most 64 chunks, else 0
  int spr;        // units per row when it has more (64 chunks each), else 1
  int narrow;     // every row and unit index fits 31 bits: 32-bit index arithmetic
  int64_t units;  // units of work of the job
  int64_t wg0;    // its first workgroup
};
constexpr int COPY_JOBS = 8;
// All n jobs in one launch (none when every job is empty).
hipError_t launch_copy(const CopyJob* jobs, int n, hipStream_t s, Marks* mk);
// Whether the prefill path uses its fast up/pre-mix kernel for this shape
// (which needs the transposed up_weight and the sigmoid table in the workspace).
bool prefill_up_fast(int dtype, int64_t M, int C, int H, int R);
// Whether it uses k_pf_upb + k_pf_premix instead (at most 128 rows), which
// need the per-branch products in the workspace.
bool prefill_up_few(int64_t M, int C, int H, int R);
constexpr size_t PREFILL_GTAB_BYTES = 2 * 24 * 128 * 2;

}  // namespace hc
