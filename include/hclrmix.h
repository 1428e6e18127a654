/*
 * libhclrmix -- the HyperConnectionLowRankMix block on AMD Instinct MI355X
 * (gfx950), as a C ABI.
 *
 * The operation is the one defined in onnxruntime PR #33384
 * ("com.microsoft.HyperConnectionLowRankMix"), section "Schema summary":
 *
 *   HyperConnectionLowRankMix(streams, norm_scale, down_weight, up_weight,
 *                             inject_weight [, prev_block_output, prev_post_gate])
 *       -> (pre_output, post_gate [, streams_out])
 *
 *   S          = streams + prev_post_gate * prev_block_output   (prologue; else S = streams)
 *   hn         = S / sqrt(mean_h(S^2) + epsilon) * norm_scale   (per branch)
 *   d          = ScaledSiLU(hn @ down_weight, silu_alpha)       (..., R)
 *   g          = sigmoid(d @ up_weight)                         (per stream and feature)
 *   pre_output = reduction_scale * sum_c(hn * g)
 *   post_gate  = sigmoid((hn @ inject_weight) / gate_div) * gate_mul
 *
 * Numerics (same page, "Numerics contract"): products and reductions
 * accumulate in fp32; each step is rounded once to T at S, hn, down, Z, SG,
 * hidden, up, g, pre_output, inject and post_gate; the sigmoid is an accurate
 * fp32 exp-based one rounded once. Every sum is taken in one fixed order, so
 * results are reproducible from call to call and each row's outputs are
 * independent of how many rows the call holds, on every path selected for
 * the same (dtype, C, H, R).
 *
 * ScaledSiLU(x, a) is taken as x * sigmoid(a * x) (Z = a*x, SG = sigmoid(Z),
 * hidden = x*SG): the page names the op and its rounding points only.
 *
 * Layout and ownership (all entry points):
 *  - Every tensor is caller-owned device memory, contiguous, row-major, with
 *    the leading dimensions flattened into `rows`, and of element type T.
 *  - streams [rows, C*H] is flattened branch-major (k = c*H + h);
 *    norm_scale [C*H]; down_weight [C*H, R], up_weight [R, C*H] and
 *    inject_weight [C*H, C] are row-major [K, N] and used in place;
 *    prev_block_output [rows, H]; prev_post_gate [rows, C].
 *  - Outputs: pre_output [rows, H], post_gate [rows, C], and optionally
 *    streams_out [rows, C*H] (S after the prologue; a copy of streams without).
 *  - The library never allocates, frees or synchronises. All work is enqueued
 *    on the caller's stream, so a call can be captured into a HIP graph.
 *    Scratch memory is the caller's `workspace`. Zero-fill a workspace once
 *    before its first use: the decode path keeps a few arrival counters in
 *    its first 4 KB, which no path writes otherwise, and every call that
 *    completes leaves them zero again. So the same workspace serves any
 *    number of calls, of any problem and path (sized for the largest), one
 *    at a time (calls that overlap on one workspace race). The rest of it
 *    holds no state.
 *  - Process-wide state, none of it holding results: a thread-local error
 *    string; per-device caches of the compute-unit count and of whether a
 *    kernel's dynamic-LDS limit has been raised (filled on first use, under
 *    a lock or by relaxed atomics); and, for hclrmix_run_noalloc only, a
 *    static device array per GPU with its device address cached per device.
 *    The decode path's arrival counters live in the caller's workspace (its
 *    first 4 KB, above), not in the library.
 */
#ifndef HCLRMIX_H
#define HCLRMIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HCLRMIX_OK = 0,
  HCLRMIX_ERR_INVALID_ARGUMENT = 1,   /* shapes, pointers or attributes violate the schema */
  HCLRMIX_ERR_UNSUPPORTED = 2,        /* valid, but outside what the library handles */
  HCLRMIX_ERR_WORKSPACE_TOO_SMALL = 3,
  HCLRMIX_ERR_DEVICE = 4              /* a HIP launch or runtime call failed */
} hclrmix_status;

/* Element type T, by ONNX TensorProto code ("Schema summary": float, float16, bfloat16). */
typedef enum { HCLRMIX_F32 = 1, HCLRMIX_F16 = 10, HCLRMIX_BF16 = 16 } hclrmix_dtype;

/* Execution path. AUTO picks DECODE for rows <= HCLRMIX_DECODE_MAX_ROWS and
 * PREFILL above, when the shape is inside the matrix-core envelope
 * (T in {f16, bf16}, 1 <= C <= 8, R <= 512, and H rounded up to a multiple
 * of 32 at most 8192 for DECODE); otherwise GENERIC. The matrix-core kernels
 * work in steps of 32 features and 32 rank columns: when H or R is not a
 * multiple of 32, the call copies its inputs into the workspace zero-padded
 * to the next multiples, runs the kernels there and copies the outputs back
 * (two more kernels; the RMS mean still divides by H). DECODE and PREFILL
 * give bit-identical rows; GENERIC (vector-ALU, any shape and T) is
 * batch-invariant on its own but its bits differ from the matrix-core paths.
 * Forcing DECODE or PREFILL outside the envelope, or DECODE with more than
 * HCLRMIX_DECODE_MAX_ROWS rows, returns HCLRMIX_ERR_UNSUPPORTED. */
typedef enum {
  HCLRMIX_PATH_AUTO = 0,
  HCLRMIX_PATH_DECODE = 1,
  HCLRMIX_PATH_PREFILL = 2,
  HCLRMIX_PATH_GENERIC = 3
} hclrmix_path;

#define HCLRMIX_DECODE_MAX_ROWS 16

/* Attributes ("Schema summary"). num_branches is required (C >= 1). */
typedef struct {
  int64_t num_branches;
  float epsilon;          /* default 1e-5 */
  float reduction_scale;  /* default 1 */
  float silu_alpha;       /* default 1 */
  float gate_div;         /* default 1; must be non-zero */
  float gate_mul;         /* default 1 */
} hclrmix_attrs;

typedef struct {
  int64_t rows;           /* product of the leading dimensions; 0 is allowed */
  int64_t width;          /* last dimension of streams: C*H */
  int64_t rank;           /* R: columns of down_weight, rows of up_weight */
  int32_t dtype;          /* hclrmix_dtype */
  int32_t has_prologue;   /* 1 if prev_block_output and prev_post_gate are given */
  int32_t path;           /* hclrmix_path */
  int32_t reserved;       /* must be 0 */
} hclrmix_problem;

/* Fills the schema defaults (epsilon 1e-5, reduction_scale, silu_alpha,
 * gate_div, gate_mul all 1) and num_branches = 0 (must then be set). */
void hclrmix_attrs_init(hclrmix_attrs* attrs);

/* Shape rule (the reviewer's request on the PR for shape inference):
 * H = width / C; pre_output [.., H], post_gate [.., C], streams_out [.., C*H].
 * Returns INVALID_ARGUMENT if C < 1, width % C != 0, width < 1 or rank < 1.
 * Any output pointer may be NULL. */
hclrmix_status hclrmix_infer_shapes(const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                    int64_t* hidden, int64_t* pre_cols, int64_t* post_cols,
                                    int64_t* streams_out_cols);

/* The path AUTO resolves to (or the forced one), after validation. */
hclrmix_status hclrmix_select_path(const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                   int32_t* path);

/* Bytes of device workspace hclrmix_run needs for this problem and path
 * (0 for rows == 0). Sized per path: no path carries another's scratch. A
 * zero-padded problem's workspace also holds the padded copies of its
 * inputs, weights included, and of its outputs.
 * A workspace must be zero-filled before its first use (see above).
 * The onnxruntime page's "CUDA implementation" section takes the operator's
 * temporary buffers (the split-K partials) from the framework's allocator
 * rather than allocating inside the kernel launch; here the caller is that
 * allocator, and this call tells it how much to provide. */
hclrmix_status hclrmix_workspace_size(const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                      size_t* bytes);

/* Byte offset, inside the workspace, of the block's low-rank activation
 * hidden = ScaledSiLU(hn @ down_weight) [rows, R] of element type T (the
 * rounding point "hidden" of the onnxruntime page's "Numerics contract"),
 * which every path leaves there: after a call on this problem has completed,
 * the workspace holds that call's hidden at this offset until the workspace
 * is used again. It lets a caller inspect the bottleneck activation, and a
 * test compare the first step after the down reduction with a reference.
 * Same errors as hclrmix_workspace_size, plus INVALID_ARGUMENT for rows == 0. */
hclrmix_status hclrmix_hidden_offset(const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                     size_t* offset);

/* Runs one block, asynchronously on `stream` (a hipStream_t; NULL = the
 * default stream). Pointers are device pointers as described above;
 * prev_block_output and prev_post_gate are both NULL (no prologue) or both
 * set, matching problem->has_prologue; streams_out may be NULL.
 *
 * Errors (checked on the host before anything is launched; on error nothing
 * is launched and no output is touched):
 *   INVALID_ARGUMENT  bad shape rule, C < 1, rank < 1, rows < 0, NULL required
 *                     pointer, prologue pointers not matching has_prologue,
 *                     gate_div == 0 or a non-finite attribute, reserved != 0,
 *                     an output buffer overlapping any other buffer.
 *   UNSUPPORTED       unknown dtype, a forced path outside its envelope, sizes
 *                     beyond int32 indexing, a pointer not 16-byte aligned
 *                     on DECODE or PREFILL when H and R are multiples of 32
 *                     (otherwise: a tensor not aligned to its element or a
 *                     workspace not 16-byte aligned).
 *   WORKSPACE_TOO_SMALL  workspace_bytes < hclrmix_workspace_size().
 *   DEVICE            a kernel launch failed (hipGetLastError).
 * rows == 0 returns OK without launching. */
hclrmix_status hclrmix_run(const void* streams, const void* norm_scale, const void* down_weight,
                           const void* up_weight, const void* inject_weight,
                           const void* prev_block_output, const void* prev_post_gate,
                           void* pre_output, void* post_gate, void* streams_out,
                           void* workspace, size_t workspace_bytes,
                           const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                           void* stream);

/* Most kernels one call launches (decode 2, or 3 from 13 rows; prefill 4 or 5;
 * generic 4, or 1 for a tiny problem; a zero-padded problem two more: its
 * input and output copies). */
#define HCLRMIX_MAX_KERNELS 7

/* Profiling variant of hclrmix_run, for per-kernel timing: the same call,
 * with the i-th kernel it launches dispatched with events[2i] as its start
 * event and events[2i+1] as its stop event (hipExtLaunchKernel), so that
 * hipEventElapsedTime(events[2i], events[2i+1]) is that kernel's execution
 * time with no extra packet queued between kernels. k = number of kernels
 * is returned in *kernels. events are hipEvent_t handles created by the
 * caller with timing enabled; n_events >= 2 * HCLRMIX_MAX_KERNELS. Same
 * errors as hclrmix_run, plus INVALID_ARGUMENT for missing events or kernels
 * pointer. Kernels of each path, in order: decode = [from 13 rows: the row
 * kernel (S, streams_out, rinv),] down slices (with the fixed-order
 * reduction done by the last workgroup per column group), up/pre-mix;
 * prefill = sums of squares (and streams_out), down per branch, branch
 * reduction, then either [up_weight transposed + sigmoid table,] up/pre-mix,
 * or (at most 128 rows) up per branch and the pre-mix;
 * generic = rms, down per part of K, the parts in order and the down/inject
 * epilogue, up/pre-mix (a tiny problem: all of it in one kernel, the same
 * results bit for bit). A zero-padded problem adds the input copy before its
 * path's kernels and the output copy after them. */
hclrmix_status hclrmix_run_timed(const void* streams, const void* norm_scale, const void* down_weight,
                                 const void* up_weight, const void* inject_weight,
                                 const void* prev_block_output, const void* prev_post_gate,
                                 void* pre_output, void* post_gate, void* streams_out,
                                 void* workspace, size_t workspace_bytes,
                                 const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                 void* stream, void* const* events, int n_events, int* kernels);

/* Chained decode: hclrmix_run (or hclrmix_run_timed when events is not NULL)
 * for one block of a chain, which also brings the NEXT block's weights
 * towards the chip while it runs. The onnxruntime PR
 * "com.microsoft.HyperConnectionLowRankMix", sections "CUDA implementation"
 * (weights are streamed before a kernel waits for its producer) and
 * "Benchmark" (a real model adds per-block overhead over the chain), is the
 * source for this: a block's weights do not depend on the previous block, so
 * their fetch need not wait for it.
 *   next_down_weight    [K, R] T, the next block's down_weight, or NULL.
 *   next_inject_weight  [K, C] T, the next block's inject_weight, or NULL.
 * Both have this problem's shapes and, when given, 16-byte alignment. They
 * are only read into cache (every value read is discarded), never used, so
 * the outputs are bit-identical to hclrmix_run's. Their contents may even be
 * under production by earlier work in the stream: no result depends on what
 * is read. Only the decode path uses them; the prefill and generic paths
 * ignore them. events, n_events and kernels as for hclrmix_run_timed when
 * events is not NULL; with events NULL the call is untimed and kernels may be
 * NULL. A zero-padded problem ignores them too (its kernels read the padded
 * copies). Errors: those of hclrmix_run (or hclrmix_run_timed), plus
 * UNSUPPORTED for a misaligned next pointer on the decode path. */
hclrmix_status hclrmix_run_chained(const void* streams, const void* norm_scale, const void* down_weight,
                                   const void* up_weight, const void* inject_weight,
                                   const void* prev_block_output, const void* prev_post_gate,
                                   void* pre_output, void* post_gate, void* streams_out,
                                   void* workspace, size_t workspace_bytes,
                                   const hclrmix_problem* problem, const hclrmix_attrs* attrs,
                                   const void* next_down_weight, const void* next_inject_weight,
                                   void* stream, void* const* events, int n_events, int* kernels);

/* Scratch hclrmix_run_noalloc holds: 16 MiB of static device memory per GPU,
 * enough for the decode path at every shape it runs unpadded (at most about
 * 11 MB: 8 branches of 8192 features, rank 512, 16 rows), for zero-padded
 * shapes whose padded weights fit beside it, and for the other paths at
 * small row counts. */
#define HCLRMIX_NOALLOC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): hclrmix_run
 * without a workspace argument. Its scratch is a static device array of
 * HCLRMIX_NOALLOC_SCRATCH_BYTES inside the library, one copy on each GPU the
 * library runs on, held until the process ends. It calls no allocating
 * routine. Arguments, outputs, paths and bits are those of hclrmix_run (the
 * same kernels run on the same layout).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents: calls of this entry point that overlap on one GPU (on
 *    two streams, or from two host threads) race and give wrong results; run
 *    them one at a time (calls in order on one stream never overlap).
 *  - The decode path's arrival counters live in the array's first bytes; the
 *    array starts zero-filled and every call that completes leaves them zero.
 *  - The calling thread's current device must be the device of `stream`.
 * Errors: those of hclrmix_run, and WORKSPACE_TOO_SMALL when the problem's
 * workspace (hclrmix_workspace_size) exceeds HCLRMIX_NOALLOC_SCRATCH_BYTES;
 * DEVICE if the array's address cannot be looked up. */
hclrmix_status hclrmix_run_noalloc(const void* streams, const void* norm_scale, const void* down_weight,
                                   const void* up_weight, const void* inject_weight,
                                   const void* prev_block_output, const void* prev_post_gate,
                                   void* pre_output, void* post_gate, void* streams_out,
                                   const hclrmix_problem* problem, const hclrmix_attrs* attrs, void* stream);

/* Standalone inv_rms (FreeToken PR #101, "compute the hyper-connection
 * pre-norm in one kernel", section "The problem"): for each row r of
 * x [rows, dim] (row-major, element type dtype: 1 fp32, 10 fp16, 16 bf16),
 *   out[r] = 1 / sqrt(mean_d(x[r][d]^2) + eps)
 * as one fp32 value (out: rows floats). Callers with leading dimensions
 * flatten them first (the page's x.flatten(2): rows = every leading index,
 * dim = the rest). The value is taken in fp64 and rounded once to fp32, so it
 * is the correctly rounded value except where fp64 rounding lands on an fp32
 * rounding boundary (section "Accuracy" of the page measures forms against
 * exactly this value). One pass over x; no workspace; enqueued on stream.
 * Errors: INVALID_ARGUMENT for rows < 0, dim < 1, NULL x or out with
 * rows > 0, a non-finite eps, or out overlapping x; UNSUPPORTED for an
 * unknown dtype or a pointer not aligned to its element; DEVICE for a failed
 * launch. rows == 0 returns OK without launching. */
hclrmix_status hclrmix_inv_rms(const void* x, float* out, int64_t rows, int64_t dim, int32_t dtype, float eps,
                               void* stream);

/* Static description of a status code. */
const char* hclrmix_status_string(hclrmix_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char* hclrmix_last_error(void);

/* Library version as "major.minor.patch". */
const char* hclrmix_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HCLRMIX_H */
