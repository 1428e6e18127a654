// Standalone inv_rms: out[r] = 1 / sqrt(mean_d(x[r][d]^2) + eps), one fp32 value
// per row of x [rows, dim] in T (FreeToken PR #101, "compute the
// hyper-connection pre-norm in one kernel", section "The problem": one pass
// over the row, the source read as stored). The work is one streaming read,
// so the arithmetic is taken in fp64 at no cost: a T value's square is exact
// in fp64, the row sum has a relative error far below an fp32 ulp, and the
// result is rounded once to fp32 (the page's section "Accuracy" measures every
// form against exactly that value).
//
// 16-byte aligned rows: one 256-thread workgroup per row. Thread t takes the
// 16-byte chunks t + 256 j of the row in batches of eight, every load of a
// batch issued before any is used (a 16384-wide bf16 row is one batch), as
// non-temporal loads (6.5 against 6.1 TB/s at 8192 x 16384 bf16); each
// wave reduces its lanes in fp64 and the four wave sums are added in order.
// Rows that are not 16-byte aligned (dim * sizeof(T) not a multiple of 16, or
// x itself misaligned) take one wave per row, one element at a time.
#include "hc_device.h"
#include "hc_internal.h"

namespace hc {

constexpr int IR_T = 8;  // chunks per lane per batch

__device__ __forceinline__ double wave_allsum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <DT D> __device__ __forceinline__ double sq_sum_chunk(u32x4 w);
template <> __device__ __forceinline__ double sq_sum_chunk<DT::F32>(u32x4 w) {
  const f32x4 f = __builtin_bit_cast(f32x4, w);
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double v = (double)f[e];
    s = s + v * v;
  }
  return s;
}
template <> __device__ __forceinline__ double sq_sum_chunk<DT::BF16>(u32x4 w) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double lo = (double)widen<DT::BF16>(w[e] & 0xFFFFu), hi = (double)widen<DT::BF16>(w[e] >> 16);
    s = s + lo * lo;
    s = s + hi * hi;
  }
  return s;
}
template <> __device__ __forceinline__ double sq_sum_chunk<DT::F16>(u32x4 w) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double lo = (double)widen<DT::F16>(w[e] & 0xFFFFu), hi = (double)widen<DT::F16>(w[e] >> 16);
    s = s + lo * lo;
    s = s + hi * hi;
  }
  return s;
}

template <DT D>
__global__ __launch_bounds__(256) void k_inv_rms_vec(const void* __restrict__ x, float* __restrict__ out,
                                                     int64_t dim, double eps) {
  __shared__ double wsum[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t r = blockIdx.x;
  constexpr int ES = D == DT::F32 ? 4 : 2;
  const int64_t nq = dim * ES / 16;  // 16-byte chunks of the row
  const unsigned char* row = (const unsigned char*)x + r * dim * ES;
  double acc = 0.0;
  for (int64_t j0 = 0; 256 * j0 < nq; j0 += IR_T) {
    u32x4 v[IR_T];
#pragma unroll
    for (int i = 0; i < IR_T; ++i)  // non-temporal: the row is read once
      v[i] = __builtin_nontemporal_load((const u32x4*)(row + 16 * min((int64_t)tid + 256 * (j0 + i), nq - 1)));
#pragma unroll
    for (int i = 0; i < IR_T; ++i)
      if (tid + 256 * (j0 + i) < nq) acc = acc + sq_sum_chunk<D>(v[i]);
  }
  const double w = wave_allsum_f64(acc);
  if (lane == 0) wsum[tid >> 6] = w;
  __syncthreads();
  if (tid == 0) out[r] = (float)(1.0 / sqrt((((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]) / (double)dim + eps));
}

template <DT D>
__global__ __launch_bounds__(256) void k_inv_rms_elem(const void* __restrict__ x, float* __restrict__ out,
                                                      int64_t rows, int64_t dim, double eps) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  double acc = 0.0;
  for (int64_t d = lane; d < dim; d += 64) {
    const double v = (double)ld<D>(x, r * dim + d);
    acc = acc + v * v;
  }
  const double ss = wave_allsum_f64(acc);
  if (lane == 0) out[r] = (float)(1.0 / sqrt(ss / (double)dim + eps));
}

hipError_t launch_inv_rms(const void* x, float* out, int64_t rows, int64_t dim, int dtype, float eps,
                          hipStream_t s) {
  const int es = dtype == 1 ? 4 : 2;
  const bool vec = ((uintptr_t)x & 15u) == 0 && (dim * es) % 16 == 0;
  const double e = (double)eps;
  if (vec) {
    if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    void* args[] = {(void*)&x, (void*)&out, (void*)&dim, (void*)&e};
    const void* k = dtype == 16 ? (const void*)k_inv_rms_vec<DT::BF16>
                  : dtype == 10 ? (const void*)k_inv_rms_vec<DT::F16>
                                : (const void*)k_inv_rms_vec<DT::F32>;
    return hipLaunchKernel(k, dim3((unsigned)rows), dim3(256), args, 0, s);
  }
  if ((rows + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  void* args[] = {(void*)&x, (void*)&out, (void*)&rows, (void*)&dim, (void*)&e};
  const void* k = dtype == 16 ? (const void*)k_inv_rms_elem<DT::BF16>
                : dtype == 10 ? (const void*)k_inv_rms_elem<DT::F16>
                              : (const void*)k_inv_rms_elem<DT::F32>;
  return hipLaunchKernel(k, dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0, s);
}

}  // namespace hc
