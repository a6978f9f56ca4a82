// Device helpers shared by the cache-write kernel and the fused decode step:
// writing one token's K/V vectors of one kv head into its slot (with int8 /
// E4M3 quantization), and copying one (block, kv head) slice of the pools.
//
// Quantized caches keep one fp16 scale per (token, kv head), separately for
// K and V ("KV Cache scaling factor", "KVcache-learning",
// fairy2021.github.io, s09; int8 / fp8 KV cache, yunthe.com, quantization
// section):  a = max_d |x_d|,  s = fp16(a / 127) or fp16(a / 448) (IEEE fp32
// division, round to nearest even),  code = clamp(rint(x / s), -127, 127) or
// the nearest-even E4M3 value of x / s saturated at +-448; s == 0 gives
// zero codes.
#pragma once

#include <cmath>

#include "pkv_internal.h"

namespace pkv {

template <int KV> constexpr int ebytes() { return KV == PKV_F32 ? 4 : KV == PKV_F16 ? 2 : 1; }

// E4M3 (OCP 8-bit float: bias 7, 3 mantissa bits, max 448, no infinities),
// nearest-even, saturating at +-448.  Works on the binary32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a == a)) return 0x7Fu;                       // NaN
  if (a >= 448.0f) return sign | 0x7Eu;              // saturate
  if (a < 0.015625f)                                 // below 2^-6: step 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t u = __float_as_uint(a);
  uint32_t ex = (u >> 23) - 127u + 7u;               // 1 .. 15
  uint32_t keep = (u >> 20) & 7u;                    // top 3 mantissa bits
  const uint32_t rest = u & 0xFFFFFu;                // 20 dropped bits
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0u; ++ex; }
  return sign | (ex << 3) | keep;
}

__device__ __forceinline__ float wave_max_all(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Byte offsets of element byte j of token t inside a (block, kv head) slice
// of BS tokens (pool layout of pkv.h).  A slice is a run of tiles of
// TB = min(BS, 16) tokens (two for BS = 32).  Inside a tile, K uses 16-byte
// columns, token-minor; V of 2- and 4-byte elements 4-byte columns,
// token-minor; V of 1-byte elements 16-byte groups of 4 elements x 4
// tokens, so that each 4-byte word holds one element of 4 consecutive tokens.
template <int BS> constexpr int tile_rows() { return BS < 16 ? BS : 16; }

template <int BS, int D, int EB>
__device__ __forceinline__ size_t k_byte(int t, int j) {
  constexpr int TB = tile_rows<BS>();
  const int u = t % TB;
  return (size_t)(t / TB) * (TB * D * EB) + (size_t)((j >> 4) * TB + u) * 16 + (j & 15);
}
template <int BS, int D, int EB>
__device__ __forceinline__ size_t v_byte(int t, int j) {
  constexpr int TB = tile_rows<BS>();
  const int u = t % TB;
  const size_t tile = (size_t)(t / TB) * (TB * D * EB);
  if constexpr (EB == 1)
    return tile + (size_t)((j >> 2) * (TB / 4) + (u >> 2)) * 16 + (j & 3) * 4 + (u & 3);
  else
    return tile + (size_t)((j >> 2) * TB + u) * 4 + (j & 3);
}

// The stored form of one token's K and V vectors of one kv head: lane l owns
// elements l*D/64 .. (l+1)*D/64 - 1 as codes of the cache type (fp32 bits,
// fp16 bits or one byte), plus the two fp16 scales of quantized caches.
template <int D> struct TokenCodes {
  uint32_t c[2][D / 64];   // [K, V][element]
  uint16_t sc[2];          // [K, V] fp16 scale bits (quantized caches)
};

// Loads the bits of lane l's elements of the source rows k_row / v_row (D
// elements of SRC type) as they are stored: RW 32-bit words per row (fp16
// pairs share a word; a single fp16 sits in the low half).  Nothing is done
// to them until token_from_raw, so the loads stay in flight until then.
template <int SRC, int D> struct TokenRaw {
  static constexpr int PER = D / 64;
  static constexpr int RW = SRC == PKV_F32 ? PER : (PER + 1) / 2;
  uint32_t w[2][RW];
};

template <int SRC, int D>
__device__ __forceinline__ void load_token_raw(const void *k_row, const void *v_row,
                                               TokenRaw<SRC, D> &raw, int lane) {
  constexpr int PER = D / 64;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint8_t *src = static_cast<const uint8_t *>(which ? v_row : k_row);
    if constexpr (SRC == PKV_F32) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        raw.w[which][k] = reinterpret_cast<const uint32_t *>(src)[lane * PER + k];
    } else if constexpr (PER == 1) {
      raw.w[which][0] = reinterpret_cast<const uint16_t *>(src)[lane];
    } else {
#pragma unroll
      for (int k = 0; k < PER / 2; ++k)
        raw.w[which][k] = reinterpret_cast<const uint32_t *>(src)[lane * (PER / 2) + k];
    }
  }
}

template <int SRC, int D>
__device__ __forceinline__ void token_from_raw(const TokenRaw<SRC, D> &raw,
                                               float (&xs)[2][D / 64]) {
  constexpr int PER = D / 64;
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if constexpr (SRC == PKV_F32) {
        xs[which][k] = __uint_as_float(raw.w[which][k]);
      } else {
        const uint32_t h = (raw.w[which][k / 2] >> (16 * (k % 2))) & 0xFFFFu;
        xs[which][k] = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
      }
    }
}

// Loads lane l's elements of the source rows k_row / v_row (D elements of
// SRC type) as fp32.
template <int SRC, int D>
__device__ __forceinline__ void load_token(const void *k_row, const void *v_row,
                                           float (&xs)[2][D / 64], int lane) {
  TokenRaw<SRC, D> raw;
  load_token_raw<SRC, D>(k_row, v_row, raw, lane);
  token_from_raw<SRC, D>(raw, xs);
}

// Converts (fp32 / fp16 caches) or quantizes (int8 / E4M3, one scale per
// vector) a token held as in load_token.  All 64 lanes take part.
template <int KV, int D>
__device__ __forceinline__ TokenCodes<D> encode_token(const float (&xs)[2][D / 64]) {
  constexpr int PER = D / 64;
  TokenCodes<D> tc;
  tc.sc[0] = tc.sc[1] = 0;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float *x = xs[which];
    if constexpr (KV == PKV_F32) {
#pragma unroll
      for (int k = 0; k < PER; ++k) tc.c[which][k] = __float_as_uint(x[k]);
    } else if constexpr (KV == PKV_F16) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        tc.c[which][k] = __builtin_bit_cast(uint16_t, (_Float16)x[k]);
    } else {
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < PER; ++k) a = fmaxf(a, fabsf(x[k]));
      a = wave_max_all(a);
      const float qmax = (KV == PKV_I8) ? 127.0f : 448.0f;
      const _Float16 s16 = (_Float16)(a / qmax);   // IEEE fp32 division, RNE to fp16
      const float s = (float)s16;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        uint32_t code = 0u;
        if (s != 0.0f) {
          const float y = x[k] / s;
          if constexpr (KV == PKV_I8)
            code = (uint32_t)(int32_t)fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f) & 0xFFu;
          else
            code = e4m3_encode_sat(y);
        }
        tc.c[which][k] = code;
      }
      tc.sc[which] = __builtin_bit_cast(uint16_t, s16);
    }
  }
  return tc;
}

// Stores an encoded token into slot t of the K and V slices of one (block, kv
// head) of BS tokens; the scale pointers address the slot's fp16 scale
// (quantized caches only).
template <int KV, int D, int BS>
__device__ __forceinline__ void store_token(const TokenCodes<D> &tc, uint8_t *k_tile,
                                            uint8_t *v_tile, uint16_t *k_scale,
                                            uint16_t *v_scale, int t, int lane) {
  constexpr int EB = ebytes<KV>();
  constexpr int PER = D / 64;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    uint8_t *tile = which ? v_tile : k_tile;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = (lane * PER + k) * EB;
      const size_t off = which ? v_byte<BS, D, EB>(t, j) : k_byte<BS, D, EB>(t, j);
      if constexpr (EB == 4)
        *reinterpret_cast<uint32_t *>(tile + off) = tc.c[which][k];
      else if constexpr (EB == 2)
        *reinterpret_cast<uint16_t *>(tile + off) = (uint16_t)tc.c[which][k];
      else
        tile[off] = (uint8_t)tc.c[which][k];
    }
    if constexpr (EB == 1)
      if (lane == 0) *(which ? v_scale : k_scale) = tc.sc[which];
  }
}

// One wavefront writes token slot t of the K and V slices of one (block, kv
// head) of BS tokens: src rows k_row / v_row hold D elements of SRC type; the
// scale pointers address the slot's fp16 scale (quantized caches only).  The
// source loads are issued before anything else so they overlap.
template <int SRC, int KV, int D, int BS>
__device__ __forceinline__ void write_token_wave(const void *k_row, const void *v_row,
                                                 uint8_t *k_tile, uint8_t *v_tile,
                                                 uint16_t *k_scale, uint16_t *v_scale, int t,
                                                 int lane) {
  float xs[2][D / 64];
  load_token<SRC, D>(k_row, v_row, xs, lane);
  store_token<KV, D, BS>(encode_token<KV, D>(xs), k_tile, v_tile, k_scale, v_scale, t, lane);
}

// One wavefront copies `bytes` (a multiple of 16) from src to dst with
// 16-byte accesses.
__device__ __forceinline__ void copy_bytes_wave(uint8_t *dst, const uint8_t *src, int bytes,
                                                int lane) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  for (int o = lane * 16; o < bytes; o += 64 * 16)
    *reinterpret_cast<v4 *>(dst + o) = *reinterpret_cast<const v4 *>(src + o);
}

}  // namespace pkv
