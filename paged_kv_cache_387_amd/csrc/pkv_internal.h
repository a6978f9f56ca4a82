// Internal declarations shared by the HIP translation units of libpkv.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

constexpr int kTile = 16;        // tokens per decode tile (the MFMA row count)
#ifndef PKV_WAVES
#define PKV_WAVES 4
#endif
constexpr int kWaves = PKV_WAVES;  // wavefronts per decode workgroup
constexpr int kMaxGroup = 16;    // query heads per kv head (MFMA column count)
constexpr int kXcds = 8;         // accelerator complex dies: workgroup i runs on die i % 8

inline int elem_bytes(int dtype) {
  return dtype == PKV_F32 ? 4 : dtype == PKV_F16 ? 2 : 1;
}

struct DecodeParams {
  void *out;
  const void *q;
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const uint16_t *k_scale;
  const uint16_t *v_scale;
  const int32_t *block_tables;
  const int32_t *seq_lens;
  float *ws_o;      // [S][H][num_parts][D] normalized partial outputs
  float *ws_lse;    // [S][H][num_parts] base-2 log-sum-exp of the partial
  int num_blocks;
  int max_blocks;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;        // num_heads / num_kv_heads
  int block_size;   // tokens per physical block: 8, 16 or 32
  int part_tiles;   // 16-token tiles per partition (whole blocks)
  int num_parts;    // partitions in the grid (>= ceil(max tokens / 16 / part_tiles))
  int num_units;    // num_seqs * num_kv_heads
  float qk_scale;   // scale * log2(e): scores are kept in base 2
  // Fused decode step only: the new token of each sequence (row s of
  // key_new / value_new, [S][Hkv][D]) is written at position seq_len - 1
  // after copying block cow_src[s] into the tail block (cow_src nullable).
  const void *key_new;
  const void *value_new;
  const int32_t *cow_src;
  uint8_t *k_cache_w;
  uint8_t *v_cache_w;
  uint16_t *k_scale_w;
  uint16_t *v_scale_w;
};

// Workgroups land on a die's compute units roughly round robin by id, and
// the die and compute-unit counts are powers of two.  A count that strides
// the grid (partitions per unit, unit groups per die) is therefore padded to
// an odd number: a unit's partitions then spread over different compute units
// instead of aliasing onto the same ones.  Padding slots are empty
// workgroups that exit at once.
__host__ __device__ inline int odd_up(int n) { return n > 1 && n % 2 == 0 ? n + 1 : n; }

// Unit groups per die: units are dealt to dies u % kXcds.
__host__ __device__ inline int unit_groups(int num_units) { return odd_up((num_units + kXcds - 1) / kXcds); }

// Grid of the decode kernel: one workgroup per (unit group, die, partition).
inline int64_t decode_grid(int num_units, int num_parts) {
  return (int64_t)unit_groups(num_units) * kXcds * num_parts;
}

struct WriteParams {
  const void *key;
  const void *value;
  int64_t key_stride;
  int64_t value_stride;
  const int64_t *slots;
  uint8_t *k_cache;
  uint8_t *v_cache;
  uint16_t *k_scale;
  uint16_t *v_scale;
  int num_tokens;
  int num_blocks;
  int num_kv_heads;
  int block_size;
};

struct CopyParams {
  uint8_t *k_cache;
  uint8_t *v_cache;
  uint16_t *k_scale;
  uint16_t *v_scale;
  const int32_t *pairs;
  int num_pairs;
  int num_blocks;
  int64_t block_bytes;   // K (or V) bytes of one physical block, all kv heads
  int64_t scale_elems;   // fp16 scales of one physical block, all kv heads (0: none)
};

hipError_t launch_decode(const DecodeParams &p, int cache_dtype, int out_dtype, int head_dim,
                         hipStream_t stream);
hipError_t launch_decode_step(const DecodeParams &p, int cache_dtype, int src_dtype,
                              int out_dtype, int head_dim, hipStream_t stream);
hipError_t launch_write(const WriteParams &p, int src_dtype, int cache_dtype, int head_dim,
                        hipStream_t stream);
hipError_t launch_copy(const CopyParams &p, hipStream_t stream);

}  // namespace pkv
