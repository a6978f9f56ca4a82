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

constexpr float kPvBoost = 64.0f;   // fold factor for quantized V scales

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
// register.  The bias is taken out of the dot products instead of the codes:
// q.(c + 1152) = q.c + 1152 * sum(q) per head, and sum_t P'_t (c_t + 1152) =
// P'.c + 1152 * sum_t P'_t, with sum_t P'_t from one more MFMA on a ones
// operand (it sums exactly the fp16 weights the P.V MFMA multiplies).
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

template <int OUT>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v) {
  if constexpr (OUT == PKV_F32)
    reinterpret_cast<float *>(out)[idx] = v;
  else
    reinterpret_cast<_Float16 *>(out)[idx] = (_Float16)v;
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
