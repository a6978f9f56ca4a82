// Device helpers of the attention kernels (decode and shared-prefix passes):
// vector types, 16-byte loads, exact widening of int8 / E4M3 codes to fp16,
// output stores and cross-row shuffles of the MFMA accumulator layout.
#pragma once

#include <cmath>

#include "kv_write.h"

namespace pkv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// Quantized V: the fp16 operand of the P.V MFMA is the softmax weight times
// the token's V scale times a power-of-two boost b, P' = p * s_v * b (b keeps
// P' clear of fp16's subnormal range; the accumulators are divided by b at the
// end).  Each wave keeps its own b and the largest scale that b admits,
//   s_lim = kFoldMax / (w_max * b),
// where w_max bounds the weights (1 in decode, whose running maximum never
// lags; 2^tau in the multi-query passes).  Every admitted token then has
// P' <= kFoldMax < 65504 = fp16's largest value.  A tile that holds a larger
// scale first lowers b by powers of two (lower_boost) and rescales the
// accumulators by the same power of two, both exact.  b starts at kVBoost0 =
// 64, which admits every scale the cache write produces from fp16 values
// (at most fp16(65504 / 127) = 516 for int8, fp16(65504 / 448) = 146.25 for
// E4M3) in decode; larger scales come only from fp32 sources.
constexpr float kVBoost0 = 64.0f;
constexpr float kFoldMax = 61440.0f;   // 1.875 * 2^15: margin for the weights' rounding

// The largest power of two b' <= b with b' * s * w_max <= kFoldMax, for the
// largest V scale s of a tile (magnitude; an infinite or NaN scale counts as
// fp16's largest finite value -- its output is not finite anyway).
__device__ __forceinline__ float lower_boost(float b, float s, float w_max) {
  s = fminf(s, 65504.0f);
  while (b * s * w_max > kFoldMax) b *= 0.5f;
  return b;
}

template <int KV> struct Kv;
template <> struct Kv<PKV_F32> { static constexpr int EB = 4; };
template <> struct Kv<PKV_F16> { static constexpr int EB = 2; };
template <> struct Kv<PKV_I8> { static constexpr int EB = 1; };
template <> struct Kv<PKV_E4M3> { static constexpr int EB = 1; };

__device__ __forceinline__ u4 load16(const uint8_t *p) {
  return *reinterpret_cast<const u4 *>(p);
}
// K/V tiles are read once per step: non-temporal loads keep them from
// displacing reusable lines (tables, q, shared blocks) and stream faster.
__device__ __forceinline__ u4 load16_stream(const uint8_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u4 *>(p));
}

__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
// Element bit-casts go through a by-value scalar: __builtin_bit_cast applied
// directly to a subscripted ext_vector element (vec[j]) compiled to element 0
// with this compiler.
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u32(h2 x) { return __builtin_bit_cast(uint32_t, x); }

// int8 codes to fp16, biased: a byte u = c + 128 (the code with its sign bit
// flipped) under the exponent byte 0x64 is the fp16 value 1024 + u = c + 1152,
// exact; one v_perm takes two such bytes and the 0x64 bytes from a constant
// register.  V keeps the bias and takes it out of the products:
// sum_t P'_t (c_t + 1152) = P'.c + 1152 * sum_t P'_t, with sum_t P'_t from the
// same fp16 weights the P.V MFMA multiplies.  K does not (k_codes16): its
// codes are made exact (c + 1152 - 1152 in fp16) before the scores.
constexpr uint32_t kExp64 = 0x64646464u;
constexpr float kI8Bias = 1152.0f;
__device__ __forceinline__ h2 i8_pair(uint32_t flipped, uint32_t sel) {
  return as_h2(__builtin_amdgcn_perm(kExp64, flipped, sel));
}
// perm selectors: bytes 0,1 (resp. 2,3) of src1 under 0x64 from src0
constexpr uint32_t kSelLo = 0x04010400u;
constexpr uint32_t kSelHi = 0x04030402u;

// E4M3 codes to exact fp16 with the gfx950 conversion (scale 1.0): two codes
// (the low or high half of a word) per instruction.
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w, bool hi) {
  return as_u32(hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                   : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

// 4 codes of one word (in order) -> h4, exact.
template <int KV>
__device__ __forceinline__ h4 codes4_to_h4(uint32_t w) {
  if constexpr (KV == PKV_I8) {
    const uint32_t f = w ^ 0x80808080u;
    return __builtin_bit_cast(h4, u2{as_u32(i8_pair(f, kSelLo)), as_u32(i8_pair(f, kSelHi))});
  } else {
    return __builtin_bit_cast(h4, u2{e4m3_pair(w, false), e4m3_pair(w, true)});
  }
}

// 16 codes (one K column) -> two h8 (codes 0-7, 8-15), exact.
template <int KV>
__device__ __forceinline__ void codes16_to_h8(u4 w, h8 &lo, h8 &hi) {
  const h4 a = codes4_to_h4<KV>(w[0]), b = codes4_to_h4<KV>(w[1]);
  const h4 c = codes4_to_h4<KV>(w[2]), d = codes4_to_h4<KV>(w[3]);
  lo = h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  hi = h8{c[0], c[1], c[2], c[3], d[0], d[1], d[2], d[3]};
}

// 16 K codes -> two h8 of the codes' exact values (int8: the biased widening
// minus 1152, one packed fp16 add per two codes, exact).  A score computed
// from biased codes, q.(c + 1152) - 1152 * sum(q), would carry fp32 rounding
// of the size of 1152 * sum|q| times the token's K scale: for rows near fp16's
// limit (scale 516) that moves the weights of keys whose scores lie a few
// units apart by tens of percent.
template <int KV>
__device__ __forceinline__ void k_codes16(u4 w, h8 &lo, h8 &hi) {
  codes16_to_h8<KV>(w, lo, hi);
  if constexpr (KV == PKV_I8) {
    lo = lo - (_Float16)kI8Bias;
    hi = hi - (_Float16)kI8Bias;
  }
}

// fp16 outputs: finite values beyond fp16's largest magnitude are stored as
// +-65504 rather than rounded to infinity.  An average of cache values exceeds
// it only through the rounding of the weights at the top of the range, or for
// int8 / E4M3 caches, whose largest dequantized values (127 * 516 = 65532,
// 448 * 146.25 = 65520) lie beyond it.  NaN and infinities are kept.
__device__ __forceinline__ _Float16 to_f16_out(float v) {
  const float a = fabsf(v);
  return (_Float16)((a > 65504.0f && a < INFINITY) ? copysignf(65504.0f, v) : v);
}

template <int OUT>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v) {
  if constexpr (OUT == PKV_F32)
    reinterpret_cast<float *>(out)[idx] = v;
  else
    reinterpret_cast<_Float16 *>(out)[idx] = to_f16_out(v);
}

__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Lane reductions across the four 16-lane rows of a wavefront (lanes r,
// r+16, r+32, r+48), with the gfx950 row swaps: permlane32_swap exchanges the
// two 32-lane halves between its operands and permlane16_swap the odd and
// even rows, so combining the two results of each swap of x with itself
// reduces over the exchanged lanes, without a trip through LDS.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware instruction (about 1 ulp; results below 2^-126 may
// flush to zero, which a softmax weight next to the maximum's 1 never
// notices).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace
}  // namespace pkv
