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
constexpr int kWaves = PKV_WAVES;  // wavefronts per workgroup of the multi-query passes
// Modes of the multi-query passes: queries of a shared prefix's group
// (partials out), or a sequence's own query tokens with causal limits.
constexpr int kModeShared = 0;
constexpr int kModePrefill = 1;
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = PKV_DECODE_WAVES;   // wavefronts per decode workgroup
constexpr int kMaxGroup = 16;    // query heads per kv head (MFMA column count)
constexpr int kXcds = 8;         // accelerator complex dies: workgroup i runs on die i % 8

// How the decode kernel's waves share the tiles (see decode_kernel.h).
constexpr int kWalkSplit = 0;    // one workgroup per (unit, partition), waves interleave tiles
constexpr int kWalkRuns = 1;     // one workgroup per (unit, run of partitions), waves interleave tiles
constexpr int kWalkStream = 2;   // equal shares of the batch's tiles per wave
// Waves the stream walk deals the batch's tiles to: two 4-wave workgroups on
// each of 256 compute units (also fixes the stream workspace's size).
constexpr int kStreamWaves = 2048;
// Fewest tiles in a stream share (a smaller batch uses fewer waves).
constexpr int kStreamMinShare = 16;

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
  float *ws_o;      // [S][H][ws_stride][D] normalized partial outputs (stream walk:
                    // [2 * stream_waves][group][D])
  float *ws_lse;    // [S][H][ws_stride] base-2 log-sum-exp of the partial (stream walk:
                    // [2 * stream_waves][group])
  int32_t *ws_info; // stream walk: [num_units][2] first wave and piece count of each unit
  int num_blocks;
  int max_blocks;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;        // num_heads / num_kv_heads
  int block_size;   // tokens per physical block: 8, 16 or 32
  int part_tiles;   // 16-token tiles per partition (whole blocks)
  int num_parts;    // partition slots per (sequence, head) workspace row (>= ceil(max tokens / 16 / part_tiles))
  int walk;         // kWalkSplit, kWalkRuns or kWalkStream
  int run_parts;    // runs walk: consecutive partitions one workgroup walks (> 1, with
                    // part_tiles a multiple of kDecodeWaves)
  int num_runs;     // split / runs walks: workgroup slots per unit in the grid
  int stream_waves; // stream walk: waves the batch's tiles are dealt to
  int min_share;    // stream walk: fewest tiles per share
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
  // Shared prefixes only (seq_group null otherwise): block_tables /
  // seq_lens then describe each sequence's suffix, and a sequence s with
  // seq_group[s] = g in [0, num_groups) and a prefix of at least one tile also
  // has the partials of its group's prefix in workspace slots ws_pre .. of its
  // row; its suffix partials always go to the workspace and the merge writes
  // `out`.
  const int32_t *seq_group;
  const int32_t *group_prefix_lens;
  int num_groups;
  int max_prefix_blocks;
  int pp_tiles;     // tiles per prefix partition
  int ws_stride;    // partial slots per (sequence, head) row of the workspace
  int ws_pre;       // first slot of the prefix partials
};

// Shared-prefix pass: for each group of sequences whose block tables begin
// with the same blocks, attention of all the group's queries over those
// blocks, read once per (group, kv head).
struct PrefixParams {
  const void *q;
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const uint16_t *k_scale;
  const uint16_t *v_scale;
  const int32_t *offsets;      // [num_groups + 1] CSR offsets into members
  const int32_t *members;      // [num_members] sequence indices
  const int32_t *tables;       // [num_groups][max_prefix_blocks]
  const int32_t *prefix_lens;  // [num_groups] tokens
  float *ws_o;
  float *ws_lse;
  int num_blocks;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;                   // query heads per kv head
  int num_groups;
  int num_members;
  int max_prefix_blocks;
  int num_units;               // num_groups * num_kv_heads
  int col_blocks;              // workgroups across one group's query columns
  int pp_tiles;                // tiles per prefix partition
  int num_pparts;              // prefix partitions in the grid
  int ws_stride;
  int ws_pre;
  float qk_scale;
  // Multi-token queries (prefill mode of the same pass): unit = (sequence,
  // kv head); sequence s has query rows query_offsets[s] .. query_offsets[s+1]
  // - 1, the last of its seq_lens[s] tokens, each attending causally.
  const int32_t *block_tables;   // [num_seqs][max_blocks]
  const int32_t *seq_lens;
  const int32_t *query_offsets;  // [num_seqs + 1]
  int max_blocks;
  int num_query_tokens;
  int block_size;
  void *out;                     // written directly when num_pparts == 1
};

// Prefix partials of sequence s (0: none).  Used identically by the decode
// kernel (which then never writes `out` directly) and the merge; the merge
// reads s's group (its seq_group entry, -1 for none) itself, with the length.
__device__ inline int prefix_parts_of_group(const DecodeParams &p, int g) {
  if ((unsigned)g >= (unsigned)p.num_groups) return 0;
  int len = p.group_prefix_lens[g];
  const int cap = p.max_prefix_blocks * p.block_size;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int tiles = len / kTile;
  return (tiles + p.pp_tiles - 1) / p.pp_tiles;
}
__device__ inline int prefix_parts_of(const DecodeParams &p, int s) {
  return p.seq_group == nullptr ? 0 : prefix_parts_of_group(p, p.seq_group[s]);
}

// Workgroups land on a die's compute units roughly round robin by id, and
// the die and compute-unit counts are powers of two.  A count that strides
// the grid (partitions per unit, unit groups per die) is therefore padded to
// an odd number: a unit's partitions then spread over different compute units
// instead of aliasing onto the same ones.  Padding slots are empty
// workgroups that exit at once.
__host__ __device__ inline int odd_up(int n) { return n > 1 && n % 2 == 0 ? n + 1 : n; }

// Unit groups per die: units are dealt to dies u % kXcds.
__host__ __device__ inline int unit_groups(int num_units) { return odd_up((num_units + kXcds - 1) / kXcds); }

// Grid of the decode kernel: one workgroup per (unit group, die, run of
// partitions).
inline int64_t decode_grid(int num_units, int num_runs) {
  return (int64_t)unit_groups(num_units) * kXcds * num_runs;
}

// LDS floats a runs-walk workgroup sets aside for the finished partials of a
// run (all but its last partition, which is stored directly): a row of
// D + 4 floats (the normalized output, its log-sum-exp, padding to 16 bytes)
// per query head and staged partition.  Room for 7 partitions of 8 heads.
__host__ __device__ constexpr int stage_floats(int head_dim) { return 7 * 8 * (head_dim + 4); }

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
// The decode kernel of the runs and stream walks (decode only, or the fused
// step when `step`); the caller launches the merge.
hipError_t launch_decode_runs(const DecodeParams &p, int cache_dtype, bool step, int out_dtype,
                              int head_dim, hipStream_t stream);
hipError_t launch_decode_stream(const DecodeParams &p, int cache_dtype, bool step, int out_dtype,
                                int head_dim, hipStream_t stream);
// Columns (query vectors) one prefix workgroup handles: 16 per MFMA chunk.
inline int prefix_chunks(int cache_dtype) { return cache_dtype == PKV_F32 ? 2 : 4; }
inline int64_t prefix_grid(const PrefixParams &p) {
  return (int64_t)unit_groups(p.num_units) * kXcds * p.col_blocks * p.num_pparts;
}
hipError_t launch_prefix(const PrefixParams &p, int cache_dtype, int head_dim, int block_size,
                         hipStream_t stream);
hipError_t launch_merge(const DecodeParams &p, int out_dtype, int head_dim, hipStream_t stream);
// The pipelined pass of fp16 caches (shared prefixes or multi-token
// queries): 64 * 4 / token_groups columns per workgroup, token_groups 1 or 2.
hipError_t launch_pipe(const PrefixParams &p, bool prefill, int out_dtype, int head_dim,
                       int block_size, int token_groups, hipStream_t stream);
// Columns of a workgroup of the pipelined pass with one token group
// (multi-token queries) and with two (shared prefixes), and of
// prefix32_kernel (quantized caches).
constexpr int kPipeCols = 256;
constexpr int kPipeSharedCols = 128;
constexpr int kPrefixCols = 64;
// Multi-token queries: the pass (and, with several partitions, the merge).
hipError_t launch_prefill(const PrefixParams &p, int cache_dtype, int out_dtype, int head_dim,
                          int block_size, hipStream_t stream);

// Block swap between device pools and device-addressable host pools.
struct SwapParams {
  uint8_t *dev_k, *dev_v;
  uint16_t *dev_ks, *dev_vs;
  uint8_t *host_k, *host_v;
  uint16_t *host_ks, *host_vs;
  const int32_t *pairs;
  int num_pairs;
  int num_blocks;
  int num_host_blocks;
  int to_host;
  int64_t block_bytes;
  int64_t scale_elems;
};
hipError_t launch_swap(const SwapParams &p, hipStream_t stream);

hipError_t launch_write(const WriteParams &p, int src_dtype, int cache_dtype, int head_dim,
                        hipStream_t stream);
hipError_t launch_copy(const CopyParams &p, hipStream_t stream);

}  // namespace pkv
