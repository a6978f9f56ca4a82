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
#include "kv_write.h"

namespace pkv {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <int SRC, int KV, int D, int BS>
__global__ __launch_bounds__(64) void write_kernel(WriteParams p) {
  constexpr int TILE = BS * D * ebytes<KV>();
  const int i = blockIdx.x;
  const int kvh = blockIdx.y;
  const int64_t slot = p.slots[i];
  if (slot < 0 || slot >= (int64_t)p.num_blocks * BS) return;
  const int64_t blk = slot / BS;
  const int t = (int)(slot % BS);
  const size_t tile = ((size_t)blk * p.num_kv_heads + kvh) * TILE;
  const size_t esz = SRC == PKV_F32 ? 4 : 2;
  const uint8_t *k_row = static_cast<const uint8_t *>(p.key) + ((size_t)i * p.key_stride + (size_t)kvh * D) * esz;
  const uint8_t *v_row = static_cast<const uint8_t *>(p.value) + ((size_t)i * p.value_stride + (size_t)kvh * D) * esz;
  const size_t sidx = ((size_t)blk * p.num_kv_heads + kvh) * BS + t;
  write_token_wave<SRC, KV, D, BS>(k_row, v_row, p.k_cache + tile, p.v_cache + tile,
                               p.k_scale ? p.k_scale + sidx : nullptr,
                               p.v_scale ? p.v_scale + sidx : nullptr, t, threadIdx.x);
}

// fp16 caches, sources on 16-byte rows: a workgroup takes TB = min(BS, 16)
// consecutive tokens of one kv head.  When their slots fill one aligned tile
// (a chunk of consecutive tokens, as a prefill writes) it gathers the tile's
// 16-byte K columns and 4-byte V columns from the token rows and stores the
// tile as whole 16-byte words, consecutive lanes on consecutive words (the
// layout of k_byte / v_byte).  Otherwise it writes the tokens one by one as
// write_kernel does.
template <int D, int BS>
__global__ __launch_bounds__(64) void write_tiles_kernel(WriteParams p) {
  constexpr int TB = tile_rows<BS>();
  constexpr int SLICE = BS * D * 2;     // bytes of a (block, kv head) slice
  constexpr int TBYTES = TB * D * 2;    // bytes of a tile
  constexpr int NW = TBYTES / 16 / 64;  // 16-byte words per lane, K and V each
  static_assert(NW >= 1 && TBYTES % (16 * 64) == 0, "tile words");
  const int i0 = blockIdx.x * TB;
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = min(TB, p.num_tokens - i0);   // >= 1
  const int64_t my = lane < n ? p.slots[i0 + lane] : -1;
  const int64_t slot0 =
      (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(my >> 32)) << 32) |
                (uint32_t)__builtin_amdgcn_readfirstlane((int)my));
  const bool lane_ok = lane >= TB || my == slot0 + lane;
  const bool full = n == TB && __builtin_amdgcn_ballot_w64(!lane_ok) == 0 && slot0 >= 0 &&
                    slot0 % TB == 0 && slot0 + TB <= (int64_t)p.num_blocks * BS;
  if (full) {
    const size_t base = ((size_t)(slot0 / BS) * p.num_kv_heads + kvh) * SLICE +
                        (size_t)((slot0 % BS) / TB) * TBYTES;
    const size_t kst = (size_t)p.key_stride * 2, vst = (size_t)p.value_stride * 2;
    const uint8_t *k0 = static_cast<const uint8_t *>(p.key) + (size_t)i0 * kst + (size_t)kvh * D * 2;
    const uint8_t *v0 = static_cast<const uint8_t *>(p.value) + (size_t)i0 * vst + (size_t)kvh * D * 2;
    u4 kw[NW], vw[NW];
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      const int e = lane + 64 * r;
      // K word e: 16-byte column e / TB of token e % TB
      kw[r] = *reinterpret_cast<const u4 *>(k0 + (size_t)(e % TB) * kst + 16 * (e / TB));
      // V word e: 4-byte column e / (TB/4) of tokens 4 (e % (TB/4)) .. + 3
      const int pc = e / (TB / 4), u = 4 * (e % (TB / 4));
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vw[r][k] = *reinterpret_cast<const uint32_t *>(v0 + (size_t)(u + k) * vst + 4 * pc);
    }
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      reinterpret_cast<u4 *>(p.k_cache + base)[lane + 64 * r] = kw[r];
      reinterpret_cast<u4 *>(p.v_cache + base)[lane + 64 * r] = vw[r];
    }
    return;
  }
  for (int j = 0; j < n; ++j) {
    const int i = i0 + j;
    const int64_t slot = p.slots[i];
    if (slot < 0 || slot >= (int64_t)p.num_blocks * BS) continue;
    const int64_t blk = slot / BS;
    const int t = (int)(slot % BS);
    const size_t tile = ((size_t)blk * p.num_kv_heads + kvh) * SLICE;
    const uint8_t *k_row = static_cast<const uint8_t *>(p.key) + ((size_t)i * p.key_stride + (size_t)kvh * D) * 2;
    const uint8_t *v_row = static_cast<const uint8_t *>(p.value) + ((size_t)i * p.value_stride + (size_t)kvh * D) * 2;
    write_token_wave<PKV_F16, PKV_F16, D, BS>(k_row, v_row, p.k_cache + tile, p.v_cache + tile,
                                              nullptr, nullptr, t, lane);
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

// Whole-block copy between a device pool and a host pool (one workgroup per
// pair): row [src, dst] of the pairs, device -> host when to_host, else
// host -> device.  Out-of-range rows are skipped.
__global__ __launch_bounds__(256) void swap_kernel(SwapParams p) {
  const int32_t a = p.pairs[2 * blockIdx.x];
  const int32_t b = p.pairs[2 * blockIdx.x + 1];
  const int32_t dev = p.to_host ? a : b, host = p.to_host ? b : a;
  if (dev < 0 || host < 0 || dev >= p.num_blocks || host >= p.num_host_blocks) return;
  const int64_t n16 = p.block_bytes / 16;
  u4 *dk = reinterpret_cast<u4 *>(p.dev_k + (size_t)dev * p.block_bytes);
  u4 *dv = reinterpret_cast<u4 *>(p.dev_v + (size_t)dev * p.block_bytes);
  u4 *hk = reinterpret_cast<u4 *>(p.host_k + (size_t)host * p.block_bytes);
  u4 *hv = reinterpret_cast<u4 *>(p.host_v + (size_t)host * p.block_bytes);
  const u4 *sk = p.to_host ? dk : hk;
  const u4 *sv = p.to_host ? dv : hv;
  u4 *tk = p.to_host ? hk : dk;
  u4 *tv = p.to_host ? hv : dv;
  for (int64_t e = threadIdx.x; e < n16; e += blockDim.x) {
    tk[e] = sk[e];
    tv[e] = sv[e];
  }
  if (p.scale_elems > 0) {
    uint16_t *dks = p.dev_ks + (size_t)dev * p.scale_elems;
    uint16_t *dvs = p.dev_vs + (size_t)dev * p.scale_elems;
    uint16_t *hks = p.host_ks + (size_t)host * p.scale_elems;
    uint16_t *hvs = p.host_vs + (size_t)host * p.scale_elems;
    for (int64_t e = threadIdx.x; e < p.scale_elems; e += blockDim.x) {
      if (p.to_host) {
        hks[e] = dks[e];
        hvs[e] = dvs[e];
      } else {
        dks[e] = hks[e];
        dvs[e] = hvs[e];
      }
    }
  }
}

template <int D>
hipError_t launch_write_tiles(const WriteParams &p, hipStream_t stream) {
  const int tb = p.block_size < 16 ? p.block_size : 16;
  dim3 grid((p.num_tokens + tb - 1) / tb, p.num_kv_heads);
  switch (p.block_size) {
    case 8: hipLaunchKernelGGL((write_tiles_kernel<D, 8>), grid, dim3(64), 0, stream, p); break;
    case 32: hipLaunchKernelGGL((write_tiles_kernel<D, 32>), grid, dim3(64), 0, stream, p); break;
    default: hipLaunchKernelGGL((write_tiles_kernel<D, 16>), grid, dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

template <int SRC, int KV, int D>
hipError_t launch_write_bs(const WriteParams &p, hipStream_t stream) {
  if constexpr (SRC == PKV_F16 && KV == PKV_F16) {
    const auto on16 = [](const void *a) { return (reinterpret_cast<uintptr_t>(a) & 15u) == 0; };
    if (on16(p.key) && on16(p.value) && p.key_stride % 8 == 0 && p.value_stride % 8 == 0)
      return launch_write_tiles<D>(p, stream);
  }
  dim3 grid(p.num_tokens, p.num_kv_heads);
  switch (p.block_size) {
    case 8: hipLaunchKernelGGL((write_kernel<SRC, KV, D, 8>), grid, dim3(64), 0, stream, p); break;
    case 32: hipLaunchKernelGGL((write_kernel<SRC, KV, D, 32>), grid, dim3(64), 0, stream, p); break;
    default: hipLaunchKernelGGL((write_kernel<SRC, KV, D, 16>), grid, dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

template <int SRC, int KV>
hipError_t launch_write_d(const WriteParams &p, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_write_bs<SRC, KV, 64>(p, stream)
                        : launch_write_bs<SRC, KV, 128>(p, stream);
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

hipError_t launch_swap(const SwapParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(swap_kernel, dim3(p.num_pairs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
