// C-ABI of libhclrmix: validation, the shape rule, workspace sizing, path
// selection and launches. Everything is checked on the host before anything
// is enqueued; on error nothing is launched and no output is touched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/hclrmix.h"
#include "hc_internal.h"

// Scratch of hclrmix_run_noalloc: a static device array, one copy per GPU
// (zero-filled when the code object is loaded). Host code never uses this
// name as an address: the per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[HCLRMIX_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

hclrmix_status fail(hclrmix_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hclrmix_status ok() {
  g_last_error.clear();
  return HCLRMIX_OK;
}

size_t elem_size(int dtype) { return dtype == HCLRMIX_F32 ? 4 : 2; }

bool dtype_known(int dtype) {
  return dtype == HCLRMIX_F32 || dtype == HCLRMIX_F16 || dtype == HCLRMIX_BF16;
}

struct Dims {
  int64_t M, C, H, R, K;
};

// Schema checks shared by every entry point (problem and attributes only).
hclrmix_status check_problem(const hclrmix_problem* p, const hclrmix_attrs* at, Dims* d) {
  if (!p || !at) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "problem and attrs must not be NULL");
  if (p->reserved != 0) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "problem.reserved must be 0");
  if (!dtype_known(p->dtype)) return fail(HCLRMIX_ERR_UNSUPPORTED, "unknown dtype %d", (int)p->dtype);
  if (at->num_branches < 1) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "num_branches must be >= 1");
  if (p->rows < 0) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (p->width < 1) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "streams width must be >= 1");
  if (p->width % at->num_branches != 0)
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "streams width %lld is not a multiple of num_branches %lld",
                (long long)p->width, (long long)at->num_branches);
  if (p->rank < 1) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "rank must be >= 1");
  if (p->has_prologue != 0 && p->has_prologue != 1)
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "has_prologue must be 0 or 1");
  if (p->path < HCLRMIX_PATH_AUTO || p->path > HCLRMIX_PATH_GENERIC)
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "unknown path %d", (int)p->path);
  const float fa[5] = {at->epsilon, at->reduction_scale, at->silu_alpha, at->gate_div, at->gate_mul};
  for (float f : fa)
    if (!std::isfinite(f)) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "attributes must be finite");
  if (at->gate_div == 0.0f) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "gate_div must not be 0");
  d->M = p->rows;
  d->C = at->num_branches;
  d->K = p->width;
  d->H = p->width / at->num_branches;
  d->R = p->rank;
  // Index ranges the kernels use 32-bit arithmetic for.
  if (d->K > (1LL << 24) || d->R > (1LL << 24) || d->K * d->R > 0x7FFFFFFFLL || d->C > 4096)
    return fail(HCLRMIX_ERR_UNSUPPORTED, "width %lld x rank %lld is beyond the supported index range",
                (long long)d->K, (long long)d->R);
  if (d->M > (1LL << 40) / (d->K > d->R ? d->K : d->R))
    return fail(HCLRMIX_ERR_UNSUPPORTED, "rows %lld too large", (long long)d->M);
  return HCLRMIX_OK;
}

int64_t up32(int64_t x) { return (x + 31) & ~(int64_t)31; }

// The matrix-core paths take 16-bit T, 1 <= C <= 8 and R <= 512. H and R
// that are not multiples of 32 run zero-padded to the next multiples (the
// padded sizes must stay inside the kernels' 32-bit index ranges).
bool in_mfma_envelope(int dtype, const Dims& d) {
  const int64_t K32 = d.C * up32(d.H);
  return (dtype == HCLRMIX_F16 || dtype == HCLRMIX_BF16) && d.C >= 1 && d.C <= 8 && d.R <= 512 &&
         K32 <= (1LL << 24) && K32 * up32(d.R) <= 0x7FFFFFFFLL;
}

hclrmix_status resolve_path(const hclrmix_problem* p, const Dims& d, int* path) {
  const bool mfma = in_mfma_envelope(p->dtype, d);
  switch (p->path) {
    case HCLRMIX_PATH_AUTO:
      *path = !mfma ? HCLRMIX_PATH_GENERIC
                    : (d.M <= HCLRMIX_DECODE_MAX_ROWS && up32(d.H) <= hc::DECODE_MAX_H ? HCLRMIX_PATH_DECODE
                                                                                      : HCLRMIX_PATH_PREFILL);
      break;
    case HCLRMIX_PATH_DECODE:
    case HCLRMIX_PATH_PREFILL:
      if (!mfma)
        return fail(HCLRMIX_ERR_UNSUPPORTED,
                    "matrix-core paths need T in {f16,bf16}, 1<=C<=8, R<=512");
      if (p->path == HCLRMIX_PATH_DECODE && d.M > HCLRMIX_DECODE_MAX_ROWS)
        return fail(HCLRMIX_ERR_UNSUPPORTED, "the decode path takes at most %d rows", HCLRMIX_DECODE_MAX_ROWS);
      if (p->path == HCLRMIX_PATH_DECODE && up32(d.H) > hc::DECODE_MAX_H)
        return fail(HCLRMIX_ERR_UNSUPPORTED, "the decode path takes branches of at most %d features",
                    hc::DECODE_MAX_H);
      *path = p->path;
      break;
    default:
      *path = HCLRMIX_PATH_GENERIC;
  }
  if (*path == HCLRMIX_PATH_GENERIC && d.R > 8192)
    return fail(HCLRMIX_ERR_UNSUPPORTED, "the generic path supports rank <= 8192");
  return HCLRMIX_OK;
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;
};

bool overlaps(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

}  // namespace

namespace hc {

int slice_length(int H) {
  for (int ks = 256; ks >= 32; ks -= 32)
    if (H % ks == 0) return ks;
  return 0;
}

Geometry make_geometry(int C, int H, int R) {
  Geometry g;
  g.KS = slice_length(H);
  g.SPB = g.KS ? H / g.KS : 0;
  g.NS = C * g.SPB;
  g.NT = R / 16 + 1;
  g.NP = 16 * g.NT;
  return g;
}

hipError_t allow_dynamic_lds(const void* kernel, int slot, size_t bytes) {
  // slot: a small id per kernel instantiation; limits recorded per device.
  static std::mutex mu;
  static size_t done[64][32] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || slot < 0 || slot >= 32) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(mu);
  if (done[dev][slot] >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[dev][slot] = bytes;
  return e;
}

int device_compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace workspace_layout(int path, int dtype, int64_t M, int C, int H, int R) {
  Workspace w{};
  if (M == 0) return w;
  // The decode arrival counters sit in a fixed prefix that every path keeps
  // clear, so one workspace can serve calls of any problem and path (the
  // counters must stay zero between calls).
  w.tickets = 0;
  size_t off = TICKETS_BYTES;
  w.hn = off;
  if (path == PATH_DECODE) off = align256(off + (size_t)M * C * H * (dtype == 1 ? 4 : 2));
  w.rinv = off;
  off = align256(off + (size_t)M * C * 4);
  w.hidden = off;
  off = align256(off + (size_t)M * R * (dtype == 1 ? 4 : 2));
  w.partial = off;
  if (path == PATH_DECODE || path == PATH_PREFILL) {
    const Geometry g = make_geometry(C, H, R);
    const size_t parts = path == PATH_DECODE || prefill_slices(M, C, H, R) ? (size_t)g.NS : (size_t)C;
    off = align256(off + parts * (size_t)M * g.NP * 4);
  } else if (path == PATH_GENERIC) {
    off = align256(off + (size_t)generic_parts((int64_t)C * H) * (size_t)M * (size_t)(R + C) * 4);
  }
  w.wut = w.gtab = off;
  if (path == PATH_PREFILL && prefill_up_fast(dtype, M, C, H, R)) {
    off = align256(off + (size_t)C * H * R * 2);
    w.gtab = off;
    off = align256(off + PREFILL_GTAB_BYTES);
  }
  w.prod = off;
  if (path == PATH_PREFILL && !prefill_up_fast(dtype, M, C, H, R) && prefill_up_few(M, C, H, R))
    off = align256(off + (size_t)M * C * H * 4);
  w.bytes = off;
  return w;
}

}  // namespace hc

namespace {

// Workspace of one call. A problem that a matrix-core path runs zero-padded
// (H or R not a multiple of 32) keeps the padded problem's own workspace
// first, so the decode counters stay in the first bytes, then the padded
// copies of its inputs and outputs, then hidden [M, R] as the caller reads it.
struct Plan {
  bool padded = false;
  int H32 = 0, R32 = 0;
  hc::Workspace inner{};  // the workspace of the problem the kernels run
  size_t streams = 0, prev_out = 0, prev_gate = 0, ns = 0, wd = 0, wu = 0, wi = 0;
  size_t pre = 0, post = 0, streams_out = 0;
  size_t hidden = 0;  // hidden [M, R] of T
  size_t bytes = 0;
};

Plan make_plan(int path, int dtype, const Dims& d, bool prologue) {
  Plan p;
  p.padded = path != HCLRMIX_PATH_GENERIC && (d.H % 32 != 0 || d.R % 32 != 0);
  if (!p.padded) {
    p.inner = hc::workspace_layout(path, dtype, d.M, (int)d.C, (int)d.H, (int)d.R);
    p.hidden = p.inner.hidden;
    p.bytes = p.inner.bytes;
    return p;
  }
  p.H32 = (int)up32(d.H);
  p.R32 = (int)up32(d.R);
  if (d.M == 0) return p;
  p.inner = hc::workspace_layout(path, dtype, d.M, (int)d.C, p.H32, p.R32);
  const size_t M = (size_t)d.M, C = (size_t)d.C, K32 = C * p.H32, H32 = p.H32, R32 = p.R32;
  size_t off = p.inner.bytes;
  auto take = [&off](size_t elems) {
    const size_t o = off;
    off = (off + elems * 2 + 255) & ~(size_t)255;
    return o;
  };
  p.streams = take(M * K32);
  if (prologue) {
    p.prev_out = take(M * H32);
    p.prev_gate = take(M * C);
  }
  p.ns = take(K32);
  p.wd = take(K32 * R32);
  p.wu = take(R32 * K32);
  p.wi = take(K32 * C);
  p.pre = take(M * H32);
  p.post = take(M * C);
  p.streams_out = take(M * K32);
  p.hidden = take(M * (size_t)d.R);
  p.bytes = off;
  return p;
}

}  // namespace

extern "C" {

void hclrmix_attrs_init(hclrmix_attrs* attrs) {
  if (!attrs) return;
  attrs->num_branches = 0;
  attrs->epsilon = 1e-5f;
  attrs->reduction_scale = 1.0f;
  attrs->silu_alpha = 1.0f;
  attrs->gate_div = 1.0f;
  attrs->gate_mul = 1.0f;
}

hclrmix_status hclrmix_infer_shapes(const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                    int64_t* hidden, int64_t* pre_cols, int64_t* post_cols,
                                    int64_t* streams_out_cols) {
  Dims d;
  hclrmix_status st = check_problem(problem, attrs, &d);
  if (st != HCLRMIX_OK) return st;
  if (hidden) *hidden = d.H;
  if (pre_cols) *pre_cols = d.H;
  if (post_cols) *post_cols = d.C;
  if (streams_out_cols) *streams_out_cols = d.K;
  return ok();
}

hclrmix_status hclrmix_select_path(const hclrmix_problem* problem, const hclrmix_attrs* attrs, int32_t* path) {
  Dims d;
  hclrmix_status st = check_problem(problem, attrs, &d);
  if (st != HCLRMIX_OK) return st;
  int p = 0;
  st = resolve_path(problem, d, &p);
  if (st != HCLRMIX_OK) return st;
  if (path) *path = p;
  return ok();
}

hclrmix_status hclrmix_workspace_size(const hclrmix_problem* problem, const hclrmix_attrs* attrs, size_t* bytes) {
  Dims d;
  hclrmix_status st = check_problem(problem, attrs, &d);
  if (st != HCLRMIX_OK) return st;
  int p = 0;
  st = resolve_path(problem, d, &p);
  if (st != HCLRMIX_OK) return st;
  if (!bytes) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  *bytes = make_plan(p, problem->dtype, d, problem->has_prologue == 1).bytes;
  return ok();
}

hclrmix_status hclrmix_hidden_offset(const hclrmix_problem* problem, const hclrmix_attrs* attrs, size_t* offset) {
  Dims d;
  hclrmix_status st = check_problem(problem, attrs, &d);
  if (st != HCLRMIX_OK) return st;
  int p = 0;
  st = resolve_path(problem, d, &p);
  if (st != HCLRMIX_OK) return st;
  if (!offset) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "offset must not be NULL");
  if (d.M == 0) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "rows == 0 has no workspace");
  *offset = make_plan(p, problem->dtype, d, problem->has_prologue == 1).hidden;
  return ok();
}

static hclrmix_status run_impl(const void* streams, const void* norm_scale, const void* down_weight,
                               const void* up_weight, const void* inject_weight, const void* prev_block_output,
                               const void* prev_post_gate, void* pre_output, void* post_gate, void* streams_out,
                               void* workspace, size_t workspace_bytes, const hclrmix_problem* problem,
                               const hclrmix_attrs* attrs, void* stream, hc::Marks* mk, int* kernels,
                               const void* next_wd = nullptr, const void* next_wi = nullptr) {
  Dims d;
  hclrmix_status st = check_problem(problem, attrs, &d);
  if (st != HCLRMIX_OK) return st;
  int path = 0;
  st = resolve_path(problem, d, &path);
  if (st != HCLRMIX_OK) return st;
  if (d.M == 0) return ok();

  if (!streams || !norm_scale || !down_weight || !up_weight || !inject_weight || !pre_output || !post_gate)
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT,
                "streams, norm_scale, the three weights, pre_output and post_gate are required");
  const bool pro = prev_block_output != nullptr;
  if (pro != (prev_post_gate != nullptr))
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "prev_block_output and prev_post_gate must be given together");
  if (pro != (problem->has_prologue == 1))
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "prologue pointers do not match problem.has_prologue");

  const size_t es = elem_size(problem->dtype);
  const Plan pl = make_plan(path, problem->dtype, d, pro);
  const uintptr_t z = 0;
  auto rng = [&](const char* n, const void* p, size_t bytes) {
    Range r{n, (uintptr_t)p, (uintptr_t)p + (p ? bytes : 0)};
    if (!p) r.lo = r.hi = z;
    return r;
  };
  const Range in[] = {
      rng("streams", streams, (size_t)d.M * d.K * es),
      rng("norm_scale", norm_scale, (size_t)d.K * es),
      rng("down_weight", down_weight, (size_t)d.K * d.R * es),
      rng("up_weight", up_weight, (size_t)d.R * d.K * es),
      rng("inject_weight", inject_weight, (size_t)d.K * d.C * es),
      rng("prev_block_output", prev_block_output, (size_t)d.M * d.H * es),
      rng("prev_post_gate", prev_post_gate, (size_t)d.M * d.C * es),
  };
  const Range out[] = {
      rng("pre_output", pre_output, (size_t)d.M * d.H * es),
      rng("post_gate", post_gate, (size_t)d.M * d.C * es),
      rng("streams_out", streams_out, (size_t)d.M * d.K * es),
      rng("workspace", workspace, pl.bytes),
  };
  for (const Range& o : out) {
    for (const Range& i : in)
      if (overlaps(o, i)) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, i.name);
    for (const Range& o2 : out)
      if (&o2 != &o && overlaps(o, o2)) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, o2.name);
  }
  if (workspace_bytes < pl.bytes || (pl.bytes > 0 && !workspace))
    return fail(HCLRMIX_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.bytes, workspace_bytes);
  // The matrix-core kernels read and write 16 bytes at a time. A padded
  // problem's kernels see only the workspace; its copy kernel touches the
  // caller's tensors and takes any element-aligned address.
  if (path != HCLRMIX_PATH_GENERIC && !pl.padded) {
    const void* ptrs[] = {streams,   norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                          prev_post_gate, pre_output, post_gate, streams_out, workspace};
    for (const void* q : ptrs)
      if (!aligned16(q)) return fail(HCLRMIX_ERR_UNSUPPORTED, "matrix-core paths need 16-byte aligned tensors");
    if (!aligned16(next_wd) || !aligned16(next_wi))
      return fail(HCLRMIX_ERR_UNSUPPORTED, "next-block weights must be 16-byte aligned");
  } else {
    const void* ptrs[] = {streams,   norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                          prev_post_gate, pre_output, post_gate, streams_out};
    for (const void* q : ptrs)
      if (q && ((uintptr_t)q % es) != 0) return fail(HCLRMIX_ERR_UNSUPPORTED, "tensors must be element-aligned");
    if (workspace && ((uintptr_t)workspace & 15u))
      return fail(HCLRMIX_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  }

  hc::Args a;
  a.streams = streams;
  a.ns = norm_scale;
  a.wd = down_weight;
  a.wu = up_weight;
  a.wi = inject_weight;
  a.prev_out = prev_block_output;
  a.prev_gate = prev_post_gate;
  a.pre = pre_output;
  a.post = post_gate;
  a.streams_out = streams_out;
  a.next_wd = path == HCLRMIX_PATH_DECODE && !pl.padded ? next_wd : nullptr;
  a.next_wi = path == HCLRMIX_PATH_DECODE && !pl.padded ? next_wi : nullptr;
  a.M = d.M;
  a.C = (int)d.C;
  a.H = (int)d.H;
  a.Hn = (int)d.H;
  a.R = (int)d.R;
  a.K = (int)d.K;
  a.eps = attrs->epsilon;
  a.rs = attrs->reduction_scale;
  a.alpha = attrs->silu_alpha;
  a.gate_div = attrs->gate_div;
  a.gate_mul = attrs->gate_mul;

  (void)hipGetLastError();  // do not report an unrelated earlier error as ours
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t e = hipSuccess;
  if (path == HCLRMIX_PATH_GENERIC) {
    e = hc::launch_generic(a, problem->dtype, ws, pl.inner, s, mk);
  } else if (!pl.padded) {
    const hc::Geometry g = hc::make_geometry(a.C, a.H, a.R);
    e = path == HCLRMIX_PATH_DECODE ? hc::launch_decode(a, problem->dtype, ws, pl.inner, g, s, mk)
                                    : hc::launch_prefill(a, problem->dtype, ws, pl.inner, g, s, mk);
  } else {
    // Zero-padded run: copy the inputs into the workspace at H32 features per
    // branch and R32 rank columns, run the kernels there, copy the outputs back.
    const int64_t M = d.M;
    const int C = (int)d.C, H = (int)d.H, R = (int)d.R, H32 = pl.H32, R32 = pl.R32;
    auto at = [ws](size_t off) { return (uint16_t*)(ws + off); };
    auto job = [](const void* src, uint16_t* dst, int64_t src_a, int64_t dst_a, int src_b, int dst_b, int src_pitch,
                  int dst_pitch, int ncopy) {
      hc::CopyJob j{};
      j.src = (const uint16_t*)src;
      j.dst = dst;
      j.src_a = src_a;
      j.dst_a = dst_a;
      j.src_b = src_b;
      j.dst_b = dst_b;
      j.src_pitch = src_pitch;
      j.dst_pitch = dst_pitch;
      j.ncopy = ncopy;
      return j;
    };
    hc::CopyJob in[7];
    int n = 0;
    in[n++] = job(streams, at(pl.streams), M, M, C, C, H, H32, H);             // [M][C][H] -> [M][C][H32]
    if (pro) {
      in[n++] = job(prev_block_output, at(pl.prev_out), M, M, 1, 1, H, H32, H);  // [M][H] -> [M][H32]
      in[n++] = job(prev_post_gate, at(pl.prev_gate), M, M, 1, 1, C, C, C);
    }
    in[n++] = job(norm_scale, at(pl.ns), C, C, 1, 1, H, H32, H);              // [C][H] -> [C][H32]
    in[n++] = job(down_weight, at(pl.wd), C, C, H, H32, R, R32, R);           // [C][H][R] -> [C][H32][R32]
    in[n++] = job(up_weight, at(pl.wu), R, R32, C, C, H, H32, H);             // [R][C][H] -> [R32][C][H32]
    in[n++] = job(inject_weight, at(pl.wi), C, C, 1, 1, H * C, H32 * C, H * C);  // [C][H*C] -> [C][H32*C]
    hc::Args b = a;
    b.streams = at(pl.streams);
    b.ns = at(pl.ns);
    b.wd = at(pl.wd);
    b.wu = at(pl.wu);
    b.wi = at(pl.wi);
    b.prev_out = pro ? at(pl.prev_out) : nullptr;
    b.prev_gate = pro ? at(pl.prev_gate) : nullptr;
    b.pre = at(pl.pre);
    b.post = at(pl.post);
    b.streams_out = streams_out ? at(pl.streams_out) : nullptr;
    b.H = H32;
    b.R = R32;
    b.K = C * H32;
    hc::CopyJob outj[4];
    int m = 0;
    outj[m++] = job(at(pl.pre), (uint16_t*)pre_output, M, M, 1, 1, H32, H, H);  // [M][H32] -> [M][H]
    outj[m++] = job(at(pl.post), (uint16_t*)post_gate, M, M, 1, 1, C, C, C);
    if (streams_out)
      outj[m++] = job(at(pl.streams_out), (uint16_t*)streams_out, M, M, C, C, H32, H, H);  // [M][C][H32] -> [M][C][H]
    outj[m++] = job(ws + pl.inner.hidden, at(pl.hidden), M, M, 1, 1, R32, R, R);         // [M][R32] -> [M][R]
    const hc::Geometry g = hc::make_geometry(C, H32, R32);
    e = hc::launch_copy(in, n, s, mk);
    if (e == hipSuccess)
      e = path == HCLRMIX_PATH_DECODE ? hc::launch_decode(b, problem->dtype, ws, pl.inner, g, s, mk)
                                      : hc::launch_prefill(b, problem->dtype, ws, pl.inner, g, s, mk);
    if (e == hipSuccess) e = hc::launch_copy(outj, m, s, mk);
  }
  if (e != hipSuccess) return fail(HCLRMIX_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  if (kernels) *kernels = mk ? mk->used / 2 : 3;
  return ok();
}

hclrmix_status hclrmix_run(const void* streams, const void* norm_scale, const void* down_weight,
                           const void* up_weight, const void* inject_weight, const void* prev_block_output,
                           const void* prev_post_gate, void* pre_output, void* post_gate, void* streams_out,
                           void* workspace, size_t workspace_bytes, const hclrmix_problem* problem,
                           const hclrmix_attrs* attrs, void* stream) {
  return run_impl(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output, prev_post_gate,
                  pre_output, post_gate, streams_out, workspace, workspace_bytes, problem, attrs, stream,
                  nullptr, nullptr);
}

// Address of the calling thread's current device's copy of `scratch`, looked
// up once per device with that device current, then kept.
static hclrmix_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HCLRMIX_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(HCLRMIX_ERR_UNSUPPORTED, "device %d is beyond the 64 this library tracks", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HCLRMIX_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return HCLRMIX_OK;
}

hclrmix_status hclrmix_run_noalloc(const void* streams, const void* norm_scale, const void* down_weight,
                                   const void* up_weight, const void* inject_weight, const void* prev_block_output,
                                   const void* prev_post_gate, void* pre_output, void* post_gate, void* streams_out,
                                   const hclrmix_problem* problem, const hclrmix_attrs* attrs, void* stream) {
  Dims d;
  hclrmix_status st = check_problem(problem, attrs, &d);
  if (st != HCLRMIX_OK) return st;
  int path = 0;
  st = resolve_path(problem, d, &path);
  if (st != HCLRMIX_OK) return st;
  const size_t need = make_plan(path, problem->dtype, d, problem->has_prologue == 1).bytes;
  if (need > HCLRMIX_NOALLOC_SCRATCH_BYTES)
    return fail(HCLRMIX_ERR_WORKSPACE_TOO_SMALL,
                "hclrmix_run_noalloc: this problem needs %zu bytes of scratch, more than the %u the library holds",
                need, (unsigned)HCLRMIX_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (d.M > 0) {
    st = scratch_address(&ws);
    if (st != HCLRMIX_OK) return st;
  }
  return run_impl(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output, prev_post_gate,
                  pre_output, post_gate, streams_out, ws, ws ? HCLRMIX_NOALLOC_SCRATCH_BYTES : 0, problem, attrs,
                  stream, nullptr, nullptr);
}

hclrmix_status hclrmix_run_timed(const void* streams, const void* norm_scale, const void* down_weight,
                                 const void* up_weight, const void* inject_weight, const void* prev_block_output,
                                 const void* prev_post_gate, void* pre_output, void* post_gate,
                                 void* streams_out, void* workspace, size_t workspace_bytes,
                                 const hclrmix_problem* problem, const hclrmix_attrs* attrs, void* stream,
                                 void* const* events, int n_events, int* kernels) {
  if (!events || n_events < 2 * HCLRMIX_MAX_KERNELS || !kernels)
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "events needs at least %d handles and kernels a pointer",
                2 * HCLRMIX_MAX_KERNELS);
  *kernels = 0;
  hc::Marks mk{events, n_events, 0};
  return run_impl(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output, prev_post_gate,
                  pre_output, post_gate, streams_out, workspace, workspace_bytes, problem, attrs, stream, &mk,
                  kernels);
}

hclrmix_status hclrmix_run_chained(const void* streams, const void* norm_scale, const void* down_weight,
                                   const void* up_weight, const void* inject_weight, const void* prev_block_output,
                                   const void* prev_post_gate, void* pre_output, void* post_gate,
                                   void* streams_out, void* workspace, size_t workspace_bytes,
                                   const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                   const void* next_down_weight, const void* next_inject_weight, void* stream,
                                   void* const* events, int n_events, int* kernels) {
  if (!events)
    return run_impl(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output, prev_post_gate,
                    pre_output, post_gate, streams_out, workspace, workspace_bytes, problem, attrs, stream,
                    nullptr, nullptr, next_down_weight, next_inject_weight);
  if (n_events < 2 * HCLRMIX_MAX_KERNELS || !kernels)
    return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "events needs at least %d handles and kernels a pointer",
                2 * HCLRMIX_MAX_KERNELS);
  *kernels = 0;
  hc::Marks mk{events, n_events, 0};
  return run_impl(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output, prev_post_gate,
                  pre_output, post_gate, streams_out, workspace, workspace_bytes, problem, attrs, stream, &mk,
                  kernels, next_down_weight, next_inject_weight);
}

hclrmix_status hclrmix_inv_rms(const void* x, float* out, int64_t rows, int64_t dim, int32_t dtype, float eps,
                               void* stream) {
  if (rows < 0 || dim < 1) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "rows must be >= 0 and dim >= 1");
  if (dtype != HCLRMIX_F32 && dtype != HCLRMIX_F16 && dtype != HCLRMIX_BF16)
    return fail(HCLRMIX_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!std::isfinite(eps)) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "eps must be finite");
  if (rows == 0) return ok();
  if (!x || !out) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "x and out are required");
  const size_t es = elem_size(dtype);
  if ((uintptr_t)x % es || (uintptr_t)out % 4)
    return fail(HCLRMIX_ERR_UNSUPPORTED, "x and out must be aligned to their elements");
  if (dim > (int64_t(1) << 40) / rows) return fail(HCLRMIX_ERR_UNSUPPORTED, "rows * dim too large");
  const Range rx{"x", (uintptr_t)x, (uintptr_t)x + (size_t)rows * (size_t)dim * es};
  const Range ro{"out", (uintptr_t)out, (uintptr_t)out + (size_t)rows * 4};
  if (overlaps(rx, ro)) return fail(HCLRMIX_ERR_INVALID_ARGUMENT, "out overlaps x");
  (void)hipGetLastError();
  const hipError_t e = hc::launch_inv_rms(x, out, rows, dim, dtype, eps, (hipStream_t)stream);
  if (e != hipSuccess) return fail(HCLRMIX_ERR_DEVICE, "HIP error: %s", hipGetErrorString(e));
  return ok();
}

const char* hclrmix_status_string(hclrmix_status status) {
  switch (status) {
    case HCLRMIX_OK: return "ok";
    case HCLRMIX_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HCLRMIX_ERR_UNSUPPORTED: return "unsupported";
    case HCLRMIX_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HCLRMIX_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* hclrmix_last_error(void) { return g_last_error.c_str(); }

const char* hclrmix_version(void) { return "0.1.0"; }

}  // extern "C"
