// Device building blocks shared by every path of the HyperConnectionLowRankMix
// block (onnxruntime PR #33384, "Schema summary" and "Numerics contract").
//
// Every function here is the single definition of one arithmetic step. The
// decode and prefill kernels call the same functions in the same order, which
// is what makes a row's bits independent of the row count and of the path
// (onnxruntime PR #33384, "Numerics contract": results per row do not depend
// on how many rows share the call).
//
// The library is compiled with -ffp-contract=off: a multiply followed by an add
// stays two roundings unless written as fmaf().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

enum class DT : int { F32 = 1, F16 = 10, BF16 = 16 };

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ u32x4 to_u32x4(uint4 v) { return u32x4{v.x, v.y, v.z, v.w}; }

template <DT D> struct Store { typedef uint16_t type; };
template <> struct Store<DT::F32> { typedef float type; };

// ------------------------------------------------------------------ codecs

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> bfloat16 with gfx950's conversion instruction (v_cvt_pk_bf16_f32):
// round to nearest even, a NaN keeps its sign and upper payload and becomes
// quiet. Checked against that definition over all 2^32 fp32 inputs.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// fp32 -> binary16, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <DT D> __device__ __forceinline__ float widen(uint32_t bits);
template <> __device__ __forceinline__ float widen<DT::BF16>(uint32_t b) { return bf16_bits_to_f32(b); }
template <> __device__ __forceinline__ float widen<DT::F16>(uint32_t b) { return f16_bits_to_f32(b); }

template <DT D> __device__ __forceinline__ uint32_t to_bits(float x);
template <> __device__ __forceinline__ uint32_t to_bits<DT::BF16>(float x) { return f32_to_bf16_bits(x); }
template <> __device__ __forceinline__ uint32_t to_bits<DT::F16>(float x) { return f32_to_f16_bits(x); }

// rT(x): round an fp32 value to T and widen it back (identity for fp32).
template <DT D> __device__ __forceinline__ float rT(float x) {
  if constexpr (D == DT::F32) return x;
  else return widen<D>(to_bits<D>(x));
}

// Scalar element access.
template <DT D> __device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (D == DT::F32) return ((const float*)p)[i];
  else return widen<D>(((const uint16_t*)p)[i]);
}
// x must already be a T value (rounded); store its encoding.
template <DT D> __device__ __forceinline__ void st(void* p, int64_t i, float x) {
  if constexpr (D == DT::F32) ((float*)p)[i] = x;
  else ((uint16_t*)p)[i] = (uint16_t)to_bits<D>(x);
}

// Eight consecutive 16-bit elements <-> fp32.
template <DT D> __device__ __forceinline__ void unpack8(uint4 v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = widen<D>(w[i] & 0xFFFFu);
    x[2 * i + 1] = widen<D>(w[i] >> 16);
  }
}
// Four consecutive 16-bit elements -> fp32.
template <DT D> __device__ __forceinline__ void unpack4(u32x2 v, float* x) {
  x[0] = widen<D>(v.x & 0xFFFFu);
  x[1] = widen<D>(v.x >> 16);
  x[2] = widen<D>(v.y & 0xFFFFu);
  x[3] = widen<D>(v.y >> 16);
}

// Two fp32 values rounded to T (nearest even) and packed, low half first: one
// v_cvt_pk_{bf16,f16}_f32 for the pair.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <DT D> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2_t v = {a, b};
  if constexpr (D == DT::BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// Eight fp32 values rounded to T and packed.
template <DT D> __device__ __forceinline__ uint4 pack8(const float* x) {
  return make_uint4(pack2<D>(x[0], x[1]), pack2<D>(x[2], x[3]), pack2<D>(x[4], x[5]), pack2<D>(x[6], x[7]));
}
// rT of two values at once (the same bits as two rT calls).
template <DT D> __device__ __forceinline__ void rT2(float& a, float& b) {
  const uint32_t w = pack2<D>(a, b);
  a = widen<D>(w & 0xFFFFu);
  b = widen<D>(w >> 16);
}

// ------------------------------------------------------------------ scalar steps

// "Numerics contract": accurate fp32 exp-based sigmoid (expf is the accurate
// device exponential, the division is correctly rounded).
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// The same function for inputs that are T values (bf16 or fp16): the
// quotient 1 / (1 + e) by the hardware reciprocal and two fused corrections
// (a correctly rounded quotient), with the division itself only where the
// quotient is subnormal or e overflowed. Over all 2^16 bf16 and all 2^16 fp16
// inputs it returns exactly the bits of sigmoid() on gfx950; every sigmoid on
// the hot path except the inject gate's takes a T value.
__device__ __forceinline__ float sigmoid_t(float x) {
  const float y = 1.0f + expf(-x);
  float r = __builtin_amdgcn_rcpf(y);
  const float e = __builtin_fmaf(-y, r, 1.0f);
  r = __builtin_fmaf(e, r, r);
  const float rem = __builtin_fmaf(-y, r, 1.0f);
  r = __builtin_fmaf(rem, r, r);
  if (y >= 0x1p126f) r = 1.0f / y;
  return r;
}

// Prologue ("Schema summary"): S = rT(s + q * p). For 16-bit T the product is
// exact in fp32.
template <DT D> __device__ __forceinline__ float prologue(float s, float q, float p) {
  float prod = q * p;
  return rT<D>(s + prod);
}

// ScaledSiLU(x, a) = x * sigmoid(a * x), rounded at Z, SG and hidden.
template <DT D> __device__ __forceinline__ float scaled_silu(float down, float alpha) {
  float Z = rT<D>(alpha * down);
  float SG = rT<D>(D == DT::F32 ? sigmoid(Z) : sigmoid_t(Z));
  return rT<D>(down * SG);
}

// post_gate = rT(sigmoid(inject / gate_div) * gate_mul) with inject already rounded.
template <DT D> __device__ __forceinline__ float post_gate(float inject, float gate_div, float gate_mul) {
  return rT<D>(sigmoid(inject / gate_div) * gate_mul);
}

// 1 / sqrt(ss / H + eps): the per-branch reciprocal RMS.
__device__ __forceinline__ float rinv_from_ss(float ss, int H, float eps) {
  float den = sqrtf(ss / (float)H + eps);
  return 1.0f / den;
}

// hn = rT((S * rinv) * norm_scale); hnorm_raw is the value before the rounding
// (for callers that round two at a time or pack it straight to T).
__device__ __forceinline__ float hnorm_raw(float S, float rinv, float ns) { return (S * rinv) * ns; }
template <DT D> __device__ __forceinline__ float hnorm(float S, float rinv, float ns) {
  return rT<D>(hnorm_raw(S, rinv, ns));
}

// g = rT(sigmoid(rT(up))) from the fp32 up-projection sum; up_gate_t takes
// up already rounded to T, and up_gate_raw leaves out the final rounding.
template <DT D> __device__ __forceinline__ float up_gate_raw(float up_t) {
  return D == DT::F32 ? sigmoid(up_t) : sigmoid_t(up_t);
}
template <DT D> __device__ __forceinline__ float up_gate(float up_acc) {
  return rT<D>(up_gate_raw<D>(rT<D>(up_acc)));
}

// ------------------------------------------------------------------ wave reductions

// Butterfly over the 64 lanes of a wave. Lanes L and L^d add the same two
// operands, so every lane ends with the same bits.
// The value of lane l ^ d (all 64 lanes active). Inside a row of 16 lanes
// the partner comes from DPP moves: quad permutations for d = 1, 2; for d = 4
// the quad reversed (l ^ 3) and then the half-row mirrored (l ^ 7); for d = 8
// the row rotated by 8. d = 16 is a swizzle inside 32 lanes (xor mask 16),
// d = 32 a permute across the halves. Only the exchange differs from a plain
// shuffle; the value read is the same.
template <int d> __device__ __forceinline__ float xor_partner(float v) {
  const int i = __builtin_bit_cast(int, v);
  int p;
  if constexpr (d == 1) p = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);        // quad_perm [1,0,3,2]
  else if constexpr (d == 2) p = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  else if constexpr (d == 4)
    p = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(i, 0x1B, 0xF, 0xF, false),  // quad_perm [3,2,1,0]
                                 0x141, 0xF, 0xF, false);                             // row_half_mirror
  else if constexpr (d == 8) p = __builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, false);  // row_ror:8
  else if constexpr (d == 16) p = __builtin_amdgcn_ds_swizzle(i, 0x401F);             // and 0x1F, xor 0x10
  else p = __shfl_xor(i, 32, 64);
  return __builtin_bit_cast(float, p);
}

// v + v[l ^ d] for d = 32, 16, ..., 1: every lane ends with the same sum,
// added in a fixed butterfly order.
__device__ __forceinline__ float wave_allsum(float v) {
  v = v + xor_partner<32>(v);
  v = v + xor_partner<16>(v);
  v = v + xor_partner<8>(v);
  v = v + xor_partner<4>(v);
  v = v + xor_partner<2>(v);
  v = v + xor_partner<1>(v);
  return v;
}

// Canonical per-branch sum of squares of one row. The row's 8-element chunks
// q = 0, 1, ... (h = 8q .. 8q+7, h < H) are dealt to 256 virtual lanes, chunk q
// to lane q mod 256; each virtual lane adds x*x from zero over its chunks in
// ascending h. The 64 lanes of each quarter (lanes 64i .. 64i+63) are added by
// the butterfly above, and the four quarter sums as ((t0 + t1) + t2) + t3.
// Every path computes exactly this, whether one wave plays all four quarters
// or four waves play one quarter each.
__device__ __forceinline__ float ss_combine(float t0, float t1, float t2, float t3) {
  return ((t0 + t1) + t2) + t3;
}


// ------------------------------------------------------------------ matrix cores

// D = A(16x32) * B(32x16) + C with fp32 accumulation (v_mfma_f32_16x16x32_{bf16,f16}).
// Fragments: lane l holds A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16], e = 0..7;
// the result lane l holds D[4*(l/16) + r][l%16], r = 0..3.
template <DT D> __device__ __forceinline__ f32x4 mfma(s16x8 a, s16x8 b, f32x4 c) {
  if constexpr (D == DT::BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// B fragment from a row-major [rows][16] tile of 16-bit values in LDS
// (32 bytes per row), chunk rows k0 .. k0+31, via two transposing reads
// (ds_read_b64_tr_b16): within each 16-lane group g, lane 4r+j names the 8-byte
// block (row k0 + 8g + r [+4], columns 4j..4j+3), and lane i of the group gets
// column i of the four rows.
__device__ __forceinline__ s16x8 lds_bfrag(const void* tile, int k0, int lane) {
  const int g = lane >> 4, j = lane & 15, r = j >> 2, cb = j & 3;
  lds_u8* base = (lds_u8*)(tile);
  lds_s16x4* p0 = (lds_s16x4*)(base + (k0 + 8 * g + r) * 32 + cb * 8);
  lds_s16x4* p1 = (lds_s16x4*)(base + (k0 + 8 * g + 4 + r) * 32 + cb * 8);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
  s16x8 v;
  v.s0 = lo.s0; v.s1 = lo.s1; v.s2 = lo.s2; v.s3 = lo.s3;
  v.s4 = hi.s0; v.s5 = hi.s1; v.s6 = hi.s2; v.s7 = hi.s3;
  return v;
}

// The same fragment from 32 row-major rows of pitch_bytes bytes (LDS), columns
// col0 .. col0+15.
__device__ __forceinline__ s16x8 lds_bfrag_pitched(const void* rows, int pitch_bytes, int col0, int lane) {
  const int g = lane >> 4, j = lane & 15, r = j >> 2, cb = j & 3;
  lds_u8* base = (lds_u8*)(rows) + (col0 + 4 * cb) * 2;
  lds_s16x4* p0 = (lds_s16x4*)(base + (8 * g + r) * pitch_bytes);
  lds_s16x4* p1 = (lds_s16x4*)(base + (8 * g + 4 + r) * pitch_bytes);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
  s16x8 v;
  v.s0 = lo.s0; v.s1 = lo.s1; v.s2 = lo.s2; v.s3 = lo.s3;
  v.s4 = hi.s0; v.s5 = hi.s1; v.s6 = hi.s2; v.s7 = hi.s3;
  return v;
}

// A fragment from a row-major [16][ld] tile of 16-bit values in LDS (ld in
// elements, multiple of 8): lane l reads row l%16, elements k0 + 8*(l/16) .. +7.
__device__ __forceinline__ s16x8 lds_afrag(const uint16_t* tile, int ld, int k0, int lane) {
  const uint4 v = *(const uint4*)(tile + (lane & 15) * ld + k0 + 8 * (lane >> 4));
  return __builtin_bit_cast(s16x8, v);
}

}  // namespace hc
