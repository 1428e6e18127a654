// Measurement kernels (libhcpeaks, not part of libhclrmix): the achievable
// HBM read and copy bandwidth and the achievable dense bf16 matrix-core
// throughput of the GPU they run on. Fractions of these measured peaks are
// reported beside the fractions of the published ones (8 TB/s, 2.5 PFLOP/s).
//
//   read : every 16-byte piece of a buffer read once (non-temporal loads,
//          one 32 KB block per workgroup, eight loads in flight per thread).
//   copy : the same reads, each written to a second buffer (non-temporal).
//   mfma : independent bf16 matrix-core chains on register operands, no
//          memory traffic in the loop: 16x16x32 (the instruction the block's
//          fixed summation order uses) and 32x32x16.
//   floors of one decode block: an empty kernel, one kernel streaming a
//          block's weights once, and a grid barrier inside one kernel.
//   overlap: whether matrix and vector work of the waves of one SIMD run at
//          the same time or take turns.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int PK_T = 8;                   // 16-byte loads in flight per thread
constexpr size_t PK_BLOCK = 256 * PK_T;  // 16-byte pieces per workgroup (32 KB)

// Workgroup b reads pieces [b PK_BLOCK, (b+1) PK_BLOCK), all loads issued
// before any is used; the store depends on every loaded word.
__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * PK_BLOCK + threadIdx.x;
  u32x4 v[PK_T];
#pragma unroll
  for (int j = 0; j < PK_T; ++j) v[j] = __builtin_nontemporal_load(src + min(base + 256 * j, n - 1));
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < PK_T; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t base = (size_t)blockIdx.x * PK_BLOCK + threadIdx.x;
  u32x4 v[PK_T];
#pragma unroll
  for (int j = 0; j < PK_T; ++j) v[j] = __builtin_nontemporal_load(src + min(base + 256 * j, n - 1));
#pragma unroll
  for (int j = 0; j < PK_T; ++j)
    if (base + 256 * j < n) __builtin_nontemporal_store(v[j], dst + base + 256 * j);
}

// BIG = false: 16x16x32 (the instruction of the block's fixed summation
// order), sixteen chains per wave; BIG = true: 32x32x16, four chains. Nothing
// reads an accumulator inside the loop: a use after each op (an empty asm
// statement that pins the accumulator to a register file, say) makes the
// compiler wait for that op's result, and the loop then measures latency
// rather than the matrix unit's rate.
template <bool BIG>
__global__ __launch_bounds__(256) void k_mfma(float* __restrict__ sink, int iters) {
  const int t = threadIdx.x;
  s16x8 a, b;
  for (int e = 0; e < 8; ++e) {  // small bf16 values (about 2^-4), so the sums stay finite
    a[e] = (short)(0x3D80 + ((t + e) & 7));
    b[e] = (short)(0x3D80 + ((t * 3 + e) & 7));
  }
  float s = 0.0f;
  if constexpr (!BIG) {
    f32x4 acc[16];
    for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][3];
  } else {
    f32x16 acc[4];
    for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][15];
  }
  if ((t & 63) == 0) sink[blockIdx.x * 4 + (t >> 6)] = s;
}

unsigned blocks_for(size_t n) { return (unsigned)((n + PK_BLOCK - 1) / PK_BLOCK); }

// ---------------------------------------------------------------- floors
// What one decode block cannot go below on this chip: a kernel that does
// nothing, a kernel that streams a given number of bytes once (each piece
// read once, all of a thread's loads in flight together), and a grid-wide
// barrier between the workgroups of one kernel.

__global__ __launch_bounds__(256) void k_empty() {}

constexpr int FL_T = 16;  // 16-byte loads in flight per thread in k_stream

// Workgroup b of G reads pieces b*256 + t + 256*G*j (t its thread, j < FL_T)
// below n: every piece once, coalesced per wave.
__device__ __forceinline__ uint32_t stream_fold(const u32x4* __restrict__ src, size_t n) {
  const size_t T = (size_t)gridDim.x * 256, base = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 v[FL_T];
#pragma unroll
  for (int j = 0; j < FL_T; ++j) v[j] = src[min(base + T * j, n - 1)];
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < FL_T; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  return acc;
}

// Self-resetting grid barrier over the workgroups of one launch: sync[0]
// counts arrivals, sync[64] is a generation word on its own 256-byte line.
// The last arrival zeroes the count and advances the generation; the others
// wait (relaxed agent-scope loads, a short sleep between them) for it to
// change, at most `spin` times: a wait that runs out is counted in err[0]
// and the workgroup goes on, so every wave ends. sync starts zeroed and is
// left with a zero count.
__device__ __forceinline__ void grid_barrier(unsigned* sync, unsigned spin, unsigned* err) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned g0 = __hip_atomic_load(sync + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned prev = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(sync + 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      unsigned it = 0;
      while (__hip_atomic_load(sync + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
        if (++it > spin) {
          __hip_atomic_fetch_add(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __syncthreads();
}

// BAR = false: stream n pieces; BAR = true: stream them, then one grid barrier.
template <bool BAR>
__global__ __launch_bounds__(256) void k_stream(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink,
                                                unsigned* sync, unsigned spin, unsigned* err) {
  const uint32_t acc = n ? stream_fold(src, n) : 0u;
  if (BAR) grid_barrier(sync, spin, err);
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Whether matrix work and vector work share a SIMD's time: two waves per
// SIMD (512-thread workgroups, one per compute unit); a step of a wave is 16
// independent 16x16x32 bf16 matrix ops and/or 64 independent fp32 vector ops
// (eight chains of a multiply and an add). MODE 0: matrix ops in every wave;
// 1: vector ops in every wave; 2: both, interleaved, in every wave; 3: waves
// 0-3 matrix ops only, waves 4-7 vector ops only.
constexpr int OV_NV = 64;
template <int MODE>
__global__ __launch_bounds__(512) void k_overlap(float* __restrict__ sink, int steps, float seed) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && wave < 4);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && wave >= 4);
  s16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (short)(0x3D80 + e);
    b[e] = (short)(0x3D80 + 2 * e);
  }
  f32x4 acc[16];
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float v[8];
  for (int i = 0; i < 8; ++i) v[i] = seed + (float)(i + (int)threadIdx.x);
  for (int st = 0; st < steps; ++st) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (do_m) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      if (do_v) {
#pragma unroll
        for (int q = 0; q < OV_NV / 16; ++q) v[(4 * j + q) & 7] = v[(4 * j + q) & 7] * 1.0001f + 0.5f;
      }
    }
  }
  float t = 0.0f;
  for (int j = 0; j < 16; ++j) t += acc[j][0];
  for (int i = 0; i < 8; ++i) t += v[i];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 8 + wave] = t;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, at most 2^46) from `src`; `sink` is one
// uint32 that is written only if the data fold to a fixed value.
// Returns 0, or a HIP error code (invalid sizes: hipErrorInvalidValue).
int hcpeaks_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || blocks_for(bytes / 16) > 0x7FFFFFFFu)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(blocks_for(bytes / 16)), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16) from `src` to `dst` (non-overlapping).
int hcpeaks_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || blocks_for(bytes / 16) > 0x7FFFFFFFu)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy, dim3(blocks_for(bytes / 16)), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                     (u32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

// `blocks` workgroups of four waves. big = 0: each wave 16 * iters matrix
// ops of 16x16x32 (16,384 FLOP each); big = 1: 4 * iters of 32x32x16
// (32,768 FLOP each). Writes 4 * blocks floats to `sink`.
int hcpeaks_mfma_bf16(float* sink, int blocks, int iters, int big, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  if (big)
    hipLaunchKernelGGL(k_mfma<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, sink, iters);
  else
    hipLaunchKernelGGL(k_mfma<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, sink, iters);
  return (int)hipGetLastError();
}

// Floors. Each enqueues one kernel of `blocks` workgroups of 256 threads.
// hcpeaks_empty: a kernel that does nothing.
int hcpeaks_empty(int blocks, void* stream) {
  if (blocks < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_empty, dim3(blocks), dim3(256), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

// hcpeaks_stream: reads `bytes` (a multiple of 16, at most blocks * 64 KB)
// from src once; barrier != 0 adds one grid barrier after the reads (sync:
// 512 zeroed bytes kept between calls; err: one uint32 counting waits that
// ran out after `spin` polls). With a barrier, all `blocks` workgroups must
// fit on the GPU at once (at most one per compute unit is safe); bytes == 0
// with barrier != 0 times the barrier alone.
int hcpeaks_stream(const void* src, size_t bytes, int blocks, int barrier, uint32_t* sink, unsigned* sync,
                   unsigned spin, unsigned* err, void* stream) {
  if (blocks < 1 || !sink || bytes % 16 != 0 || (bytes && !src) || bytes / 16 > (size_t)blocks * 256 * FL_T)
    return (int)hipErrorInvalidValue;
  if (barrier && (!sync || !err)) return (int)hipErrorInvalidValue;
  if (barrier)
    hipLaunchKernelGGL(k_stream<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, bytes / 16,
                       sink, sync, spin, err);
  else
    hipLaunchKernelGGL(k_stream<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, bytes / 16,
                       sink, sync, spin, err);
  return (int)hipGetLastError();
}

// `blocks` workgroups of 512 threads running k_overlap<mode> for `steps`
// steps; writes 8 * blocks floats to `sink`.
int hcpeaks_overlap(float* sink, int blocks, int steps, int mode, void* stream) {
  if (!sink || blocks < 1 || steps < 1 || mode < 0 || mode > 3) return (int)hipErrorInvalidValue;
  const hipStream_t s = (hipStream_t)stream;
  if (mode == 0) hipLaunchKernelGGL(k_overlap<0>, dim3(blocks), dim3(512), 0, s, sink, steps, 1.0f);
  if (mode == 1) hipLaunchKernelGGL(k_overlap<1>, dim3(blocks), dim3(512), 0, s, sink, steps, 1.0f);
  if (mode == 2) hipLaunchKernelGGL(k_overlap<2>, dim3(blocks), dim3(512), 0, s, sink, steps, 1.0f);
  if (mode == 3) hipLaunchKernelGGL(k_overlap<3>, dim3(blocks), dim3(512), 0, s, sink, steps, 1.0f);
  return (int)hipGetLastError();
}

}  // extern "C"
