// Cache write ("reshape_and_cache") and copy-on-write block copy for gfx950.
//
// Write: token i's K and V vectors for every kv head go to slot
// slot_mapping[i] = physical block * 16 + position ("append the new token's
// K/V to the cache", "KVcache-learning", fairy2021.github.io, s02; slot
// addressing through the block table, "KV Cache and PagedAttention
// (vllm-musa)", 7yue.com, section 5).  int8 and E4M3 caches quantize each
// (token, kv head) vector with its own fp16 scale (KV-cache scaling factor,
// KVcache-learning s09; int8 / fp8 KV, yunthe.com quantization section).
// One wavefront handles one (token, kv head): lane l owns head_dim/64
// consecutive elements; the absolute maximum is a wavefront reduction.
//
// Copy: whole physical blocks (K and V tiles of every kv head, and scales)
// are copied src -> dst with 16-byte loads and stores (copy-on-write,
// KVcache-learning s05 and s06).
#include <cmath>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// byte offsets inside a (block, kv head) tile, see include/pkv.h
__device__ __forceinline__ size_t k_byte(int t, int j) { return (size_t)((j >> 4) * 16 + t) * 16 + (j & 15); }
__device__ __forceinline__ size_t v_byte(int t, int j) { return (size_t)((j >> 2) * 16 + t) * 4 + (j & 3); }

template <int SRC, int KV, int D>
__global__ __launch_bounds__(64) void write_kernel(WriteParams p) {
  constexpr int EB = ebytes<KV>();
  constexpr int PER = D / 64;   // elements per lane
  constexpr int TILE = kBlockSize * D * EB;
  const int i = blockIdx.x;
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t ks = p.key_stride, vs = p.value_stride;

  // The source rows and the slot are independent loads: issue all of them
  // before the slot is examined.
  float xs[2][PER];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const void *src = which ? p.value : p.key;
    const size_t row = (size_t)i * (which ? vs : ks) + (size_t)kvh * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane * PER + k;
      if constexpr (SRC == PKV_F32)
        xs[which][k] = reinterpret_cast<const float *>(src)[row + d];
      else
        xs[which][k] = (float)reinterpret_cast<const _Float16 *>(src)[row + d];
    }
  }
  const int64_t slot = p.slots[i];
  if (slot < 0 || slot >= (int64_t)p.num_blocks * kBlockSize) return;
  const int64_t blk = slot / kBlockSize;
  const int t = (int)(slot % kBlockSize);
  const size_t tile = ((size_t)blk * p.num_kv_heads + kvh) * TILE;

#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float *x = xs[which];
    uint8_t *pool = (which ? p.v_cache : p.k_cache) + tile;
    if constexpr (KV == PKV_F32 || KV == PKV_F16) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = (lane * PER + k) * EB;
        const size_t off = which ? v_byte(t, j) : k_byte(t, j);
        if constexpr (KV == PKV_F32)
          *reinterpret_cast<float *>(pool + off) = x[k];
        else
          *reinterpret_cast<_Float16 *>(pool + off) = (_Float16)x[k];
      }
    } else {
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < PER; ++k) a = fmaxf(a, fabsf(x[k]));
      a = wave_max(a);
      const float qmax = (KV == PKV_I8) ? 127.0f : 448.0f;
      const _Float16 s16 = (_Float16)(a / qmax);   // IEEE fp32 division, RNE to fp16
      const float s = (float)s16;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = lane * PER + k;
        uint32_t code = 0u;
        if (s != 0.0f) {
          const float y = x[k] / s;
          if constexpr (KV == PKV_I8)
            code = (uint32_t)(int32_t)fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f) & 0xFFu;
          else
            code = e4m3_encode_sat(y);
        }
        pool[which ? v_byte(t, j) : k_byte(t, j)] = (uint8_t)code;
      }
      if (lane == 0) {
        uint16_t *sc = which ? p.v_scale : p.k_scale;
        sc[((size_t)blk * p.num_kv_heads + kvh) * kBlockSize + t] =
            __builtin_bit_cast(uint16_t, s16);
      }
    }
  }
}

__global__ __launch_bounds__(256) void copy_kernel(CopyParams p) {
  const int32_t src = p.pairs[2 * blockIdx.x];
  const int32_t dst = p.pairs[2 * blockIdx.x + 1];
  if (src < 0 || dst < 0 || src >= p.num_blocks || dst >= p.num_blocks || src == dst) return;
  const int64_t n16 = p.block_bytes / 16;
  const u4 *ks = reinterpret_cast<const u4 *>(p.k_cache + (size_t)src * p.block_bytes);
  const u4 *vs = reinterpret_cast<const u4 *>(p.v_cache + (size_t)src * p.block_bytes);
  u4 *kd = reinterpret_cast<u4 *>(p.k_cache + (size_t)dst * p.block_bytes);
  u4 *vd = reinterpret_cast<u4 *>(p.v_cache + (size_t)dst * p.block_bytes);
  for (int64_t e = threadIdx.x; e < n16; e += blockDim.x) {
    kd[e] = ks[e];
    vd[e] = vs[e];
  }
  if (p.scale_elems > 0) {
    for (int64_t e = threadIdx.x; e < p.scale_elems; e += blockDim.x) {
      p.k_scale[(size_t)dst * p.scale_elems + e] = p.k_scale[(size_t)src * p.scale_elems + e];
      p.v_scale[(size_t)dst * p.scale_elems + e] = p.v_scale[(size_t)src * p.scale_elems + e];
    }
  }
}

template <int SRC, int KV>
hipError_t launch_write_d(const WriteParams &p, int head_dim, hipStream_t stream) {
  dim3 grid(p.num_tokens, p.num_kv_heads);
  if (head_dim == 64)
    hipLaunchKernelGGL((write_kernel<SRC, KV, 64>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((write_kernel<SRC, KV, 128>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int SRC>
hipError_t launch_write_kv(const WriteParams &p, int cache_dtype, int head_dim,
                           hipStream_t stream) {
  switch (cache_dtype) {
    case PKV_F32: return launch_write_d<SRC, PKV_F32>(p, head_dim, stream);
    case PKV_F16: return launch_write_d<SRC, PKV_F16>(p, head_dim, stream);
    case PKV_I8: return launch_write_d<SRC, PKV_I8>(p, head_dim, stream);
    default: return launch_write_d<SRC, PKV_E4M3>(p, head_dim, stream);
  }
}

}  // namespace

hipError_t launch_write(const WriteParams &p, int src_dtype, int cache_dtype, int head_dim,
                        hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  return src_dtype == PKV_F32 ? launch_write_kv<PKV_F32>(p, cache_dtype, head_dim, stream)
                              : launch_write_kv<PKV_F16>(p, cache_dtype, head_dim, stream);
}

hipError_t launch_copy(const CopyParams &p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(p.num_pairs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
