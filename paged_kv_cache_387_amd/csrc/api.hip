// C ABI of libpkv: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <cstring>
#include <mutex>

#include "pkv_internal.h"

namespace {

using namespace pkv;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool is_cache_dtype(int t) { return t == PKV_F32 || t == PKV_F16 || t == PKV_I8 || t == PKV_E4M3; }
bool is_quant(int t) { return t == PKV_I8 || t == PKV_E4M3; }

// The kernels are built for gfx950 only: refuse any other device instead of
// failing at launch.  Cached per device id.
int check_device() {
  static std::mutex mu;
  static int state[64] = {0};   // 0 unknown, 1 ok, -1 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EDEVICE;
  if (dev < 0 || dev >= 64) return PKV_ENOTSUP;
  std::lock_guard<std::mutex> lock(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PKV_EDEVICE;
    state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return state[dev] == 1 ? PKV_OK : PKV_ENOTSUP;
}

int status_of(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_EDEVICE; }

bool valid_block_size(int32_t bs) { return bs == 8 || bs == 16 || bs == 32; }

// Decode tiles (16 tokens) a table row of max_blocks blocks can hold.
int64_t max_tiles_of(int32_t max_blocks, int32_t block_size) {
  return ((int64_t)max_blocks * block_size + kTile - 1) / kTile;
}

// Partition sizes in tokens must be whole tiles and whole blocks.
bool valid_partition(int32_t tokens, int32_t block_size) {
  const int32_t unit = block_size > kTile ? block_size : kTile;
  return tokens >= 0 && tokens % unit == 0;
}

// Automatic partition choice: a quarter of the table's width, clamped to
// [kMinPartTiles, kMaxPartTiles] tiles and rounded up to a multiple of the
// wave count (which keeps 32-token blocks whole).  Short sequences (up to
// 1024 tokens) run in a single pass; long ones are split into pieces of at
// most 4096 tokens so that sequences of very different lengths still spread
// evenly over the compute units.
constexpr int64_t kMinPartTiles = 64;
constexpr int64_t kMaxPartTiles = 256;

int32_t choose_part_tiles(int32_t max_blocks, int32_t block_size, int32_t requested_tokens) {
  const int64_t mt = max_tiles_of(max_blocks, block_size);
  int64_t pt;
  if (requested_tokens > 0) {
    pt = requested_tokens / kTile;
  } else {
    pt = (mt + 3) / 4;
    if (pt < kMinPartTiles) pt = kMinPartTiles;
    if (pt > kMaxPartTiles) pt = kMaxPartTiles;
    pt = (pt + kDecodeWaves - 1) / kDecodeWaves * kDecodeWaves;
  }
  return pt >= mt ? (int32_t)mt : (int32_t)pt;
}

// The decode plan for a table width and partition request: how the kernel's
// waves share the tiles (see decode_kernel.h) and the partition slots of the
// workspace.
//  * An automatic choice that splits the table, with no shared-prefix
//    partials to merge: the stream walk, equal shares of the batch's tiles
//    per wave, whatever the lengths.
//  * Explicit partitions that are whole multiples of the wave count: the runs
//    walk, one workgroup walking run_parts consecutive partitions of its
//    unit, keeping its load ring primed across their boundaries and ending
//    each in its own partial.  A run spans about as many tiles as an
//    automatic partition would, so small explicit partitions keep the long
//    per-workgroup walks that stream well; its finished partials wait in LDS
//    (stage_floats) until its last load has been issued.
//  * Otherwise one workgroup per partition (the split walk), which for a
//    table of one partition is the single pass.
// Stream grid.  Two workgroups that share a compute unit do not stream at
// the same rate: the hardware favours the older one's waves, the younger
// one's first tiles arrive late and it finishes last.  Where every share is
// one long piece (few units), a grid of one workgroup per compute unit
// (kWavesOneRound waves) finishes first; where shares hold the short pieces
// of many units, a second workgroup per compute unit hides the start of each
// piece and pays for itself.
constexpr int64_t kWavesOneRound = 1024;   // 4 waves on each of 256 compute units
constexpr int64_t kFewUnits = 256;

struct DecodePlan {
  int walk = kWalkSplit;
  int32_t part_tiles = 0;      // tiles per partition (split and runs walks)
  int32_t num_parts = 0;       // partition slots per (sequence, head) row
  int32_t run_parts = 1;       // runs walk
  int32_t num_runs = 0;        // workgroup slots per unit (split and runs walks)
  int32_t stream_waves = 0;    // stream walk: waves the batch's tiles are dealt to
};

DecodePlan plan_decode(int64_t num_units, int32_t max_blocks, int32_t block_size,
                       int32_t requested, int32_t extra_parts, int32_t group,
                       int32_t head_dim) {
  DecodePlan pl;
  const int64_t mt = max_tiles_of(max_blocks, block_size);
  pl.part_tiles = choose_part_tiles(max_blocks, block_size, requested);
  const int64_t parts = (mt + pl.part_tiles - 1) / pl.part_tiles;
  pl.num_parts = odd_up((int32_t)parts);
  if (requested == 0 && extra_parts == 0 && parts > 1) {
    pl.walk = kWalkStream;
    pl.stream_waves = num_units <= kFewUnits ? (int32_t)kWavesOneRound : kStreamWaves;
    return pl;
  }
  if (pl.part_tiles % kDecodeWaves == 0 && parts > 1) {
    int64_t rp = choose_part_tiles(max_blocks, block_size, 0) / pl.part_tiles;
    const int64_t cap = 1 + stage_floats(head_dim) / ((int64_t)(group > 1 ? group : 1) * (head_dim + 4));
    rp = rp < cap ? rp : cap;
    rp = rp < parts ? rp : parts;
    if (rp > 1) {
      pl.walk = kWalkRuns;
      pl.run_parts = (int32_t)rp;
      pl.num_runs = odd_up((int32_t)((parts + rp - 1) / rp));
      return pl;
    }
  }
  pl.num_runs = pl.num_parts;
  return pl;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace: [partial outputs][partial lse][stream walk: unit records], each
// part 256-byte aligned.
struct WorkspaceLayout {
  size_t o_off, lse_off, info_off, total;
};

// Split and runs walks: a row of partials per (sequence, head), num_parts
// suffix (or whole-sequence) partitions, then `extra` shared-prefix
// partitions.  Stream walk: two partial slots per wave (a unit's first piece,
// and a piece that began in an earlier share), each holding the rows of a
// kv head's group of query heads, and per unit its first wave and piece count.
WorkspaceLayout rows_layout(int32_t num_rows, int32_t num_heads, int32_t head_dim,
                            int32_t num_parts, int32_t extra = 0) {
  WorkspaceLayout w{0, 0, 0, 0};
  if (num_parts <= 1 && extra == 0) return w;
  const size_t rows = (size_t)num_rows * num_heads * (num_parts + extra);
  w.lse_off = round256(rows * head_dim * sizeof(float));
  w.total = w.lse_off + rows * sizeof(float);
  w.info_off = w.total;
  return w;
}

WorkspaceLayout workspace_layout(const DecodePlan &pl, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t extra = 0) {
  if (pl.walk != kWalkStream)
    return rows_layout(num_seqs, num_heads, head_dim, pl.num_parts, extra);
  WorkspaceLayout w{0, 0, 0, 0};
  const size_t rows = (size_t)2 * kStreamWaves * (num_heads / num_kv_heads);
  w.lse_off = round256(rows * head_dim * sizeof(float));
  w.info_off = round256(w.lse_off + rows * sizeof(float));
  w.total = w.info_off + (size_t)num_seqs * num_kv_heads * 2 * sizeof(int32_t);
  return w;
}

// Shared-prefix partitioning: enough (group, kv head, column block,
// partition) workgroups to give every compute unit one, with partitions of
// at least 16 tiles and a multiple of the wave count.  Planned for the
// 128-column blocks of the pipelined pass (fp16 caches) whatever the cache
// type, so that the workspace size does not depend on it.
constexpr int64_t kPrefixTargetWgs = 256;
constexpr int64_t kPrefixMinTiles = 16;
constexpr int kPrefixNominalCols = kPipeSharedCols;

struct PrefixPlan {
  int32_t pp_tiles = 0, num_pparts = 0;
};

bool valid_groups(const pkv_prefix_groups *gr, int32_t block_size) {
  if (!gr || gr->num_groups < 0) return false;
  if (gr->num_groups == 0) return true;
  return gr->num_members >= 0 && gr->max_group_size >= 1 && gr->max_prefix_blocks >= 1 &&
         (int64_t)gr->max_prefix_blocks * block_size <= (1 << 30);
}

PrefixPlan plan_prefix(const pkv_prefix_groups *gr, int32_t num_heads, int32_t num_kv_heads,
                       int32_t block_size) {
  PrefixPlan pl;
  if (!gr || gr->num_groups <= 0) return pl;
  const int64_t tiles = (int64_t)gr->max_prefix_blocks * block_size / kTile;
  if (tiles <= 0) return pl;
  const int64_t cols = (int64_t)gr->max_group_size * (num_heads / num_kv_heads);
  const int64_t per_part =
      (int64_t)gr->num_groups * num_kv_heads * ((cols + kPrefixNominalCols - 1) / kPrefixNominalCols);
  int64_t parts = (kPrefixTargetWgs + per_part - 1) / per_part;
  const int64_t max_parts = (tiles + kPrefixMinTiles - 1) / kPrefixMinTiles;
  parts = parts < 1 ? 1 : (parts > max_parts ? max_parts : parts);
  int64_t pt = (tiles + parts - 1) / parts;
  pt = (pt + kWaves - 1) / kWaves * kWaves;
  pl.pp_tiles = (int32_t)pt;
  pl.num_pparts = (int32_t)((tiles + pt - 1) / pt);
  return pl;
}

// Multi-token queries: partitions of the table's tokens.  One pass per
// (sequence, kv head, column block) when there are enough of them for the
// compute units, else partitions of at least 32 tiles; explicit sizes must
// be whole 32-token steps and whole blocks.  The partitions are planned for
// the pipelined pass's 256-column blocks whatever the cache type, so that the
// workspace size does not depend on it.

struct PrefillPlan {
  int64_t col_blocks = 0;
  int32_t pp_tiles = 0, num_pparts = 0;
};

bool valid_prefill_partition(int32_t tokens, int32_t block_size) {
  const int32_t unit = block_size > 32 ? block_size : 32;
  return tokens >= 0 && tokens % unit == 0;
}

PrefillPlan plan_prefill(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t max_query_len, int32_t max_blocks, int32_t block_size,
                         int32_t requested) {
  PrefillPlan pl;
  const int64_t cols = (int64_t)max_query_len * (num_heads / num_kv_heads);
  pl.col_blocks = (cols + kPipeCols - 1) / kPipeCols;
  const int64_t tiles = max_tiles_of(max_blocks, block_size);
  int64_t pt;
  if (requested > 0) {
    pt = requested / kTile;
  } else {
    const int64_t wgs = (int64_t)num_seqs * num_kv_heads * pl.col_blocks;
    int64_t parts = (kPrefixTargetWgs + wgs - 1) / (wgs > 0 ? wgs : 1);
    const int64_t max_parts = (tiles + 31) / 32;
    parts = parts < 1 ? 1 : (parts > max_parts ? max_parts : parts);
    pt = (tiles + parts - 1) / parts;
    pt = (pt + 7) / 8 * 8;
  }
  if (pt >= tiles) pt = (tiles + 1) / 2 * 2;   // one partition (whole steps)
  pl.pp_tiles = (int32_t)pt;
  pl.num_pparts = (int32_t)((tiles + pt - 1) / pt);
  return pl;
}

}  // namespace

extern "C" {

const char *pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_ENOMEM: return "block pool exhausted";
    case PKV_ENOENT: return "unknown sequence id";
    case PKV_EEXIST: return "sequence id already exists";
    case PKV_EDEVICE: return "HIP device error";
    case PKV_ENOTSUP: return "unsupported configuration or device";
    case PKV_ESCRATCH: return "more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 100; }

int32_t paged_attention_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t requested) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      !valid_block_size(block_size) || !valid_partition(requested, block_size))
    return PKV_EINVAL;
  return choose_part_tiles(max_blocks_per_seq, block_size, requested) * kTile;
}

int32_t paged_attention_decode_walk(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads ||
      head_dim <= 0 || max_blocks_per_seq <= 0 || !valid_block_size(block_size) ||
      !valid_partition(partition_size, block_size))
    return PKV_EINVAL;
  const DecodePlan pl = plan_decode((int64_t)num_seqs * num_kv_heads, max_blocks_per_seq,
                                    block_size, partition_size, 0, num_heads / num_kv_heads,
                                    head_dim);
  return pl.walk == kWalkStream ? PKV_WALK_STREAM
         : pl.walk == kWalkRuns ? PKV_WALK_RUNS
                                : PKV_WALK_SPLIT;
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || !valid_block_size(block_size) ||
      !valid_partition(partition_size, block_size))
    return 0;
  const DecodePlan pl = plan_decode((int64_t)num_seqs * num_kv_heads, max_blocks_per_seq,
                                    block_size, partition_size, 0, num_heads / num_kv_heads,
                                    head_dim);
  return workspace_layout(pl, num_seqs, num_heads, num_kv_heads, head_dim).total;
}

size_t paged_attention_prefill_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens,
                                               int32_t max_query_len, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_blocks_per_seq, int32_t block_size,
                                               int32_t partition_size) {
  if (num_seqs <= 0 || num_query_tokens <= 0 || max_query_len <= 0 || num_heads <= 0 ||
      num_kv_heads <= 0 || num_heads % num_kv_heads || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || !valid_block_size(block_size) ||
      !valid_prefill_partition(partition_size, block_size))
    return 0;
  const PrefillPlan pl = plan_prefill(num_seqs, num_heads, num_kv_heads, max_query_len,
                                      max_blocks_per_seq, block_size, partition_size);
  if (pl.num_pparts <= 1) return 0;
  return rows_layout(num_query_tokens, num_heads, head_dim, pl.num_pparts).total;
}

size_t paged_attention_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              int32_t partition_size,
                                              const pkv_prefix_groups *groups) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_heads % num_kv_heads || max_blocks_per_seq <= 0 || !valid_block_size(block_size) ||
      !valid_partition(partition_size, block_size) || !valid_groups(groups, block_size))
    return 0;
  const PrefixPlan pre = plan_prefix(groups, num_heads, num_kv_heads, block_size);
  const DecodePlan pl = plan_decode((int64_t)num_seqs * num_kv_heads, max_blocks_per_seq,
                                    block_size, partition_size, pre.num_pparts,
                                    num_heads / num_kv_heads, head_dim);
  return workspace_layout(pl, num_seqs, num_heads, num_kv_heads, head_dim, pre.num_pparts)
      .total;
}

}  // extern "C"

namespace {

// Validation and parameter set-up shared by paged_attention_decode and
// paged_decode_step.  Returns PKV_OK and fills *pp, or an error status.
int prepare_decode(DecodeParams *pp, void *out, int32_t out_dtype, const void *query,
                   int32_t q_dtype, const void *k_cache, const void *v_cache,
                   const void *k_scale, const void *v_scale, int32_t cache_dtype,
                   int32_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                   int32_t partition_size, void *workspace, size_t workspace_bytes,
                   int32_t extra_parts = 0) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || partition_size < 0)
    return PKV_EINVAL;
  if (num_heads % num_kv_heads) return PKV_EINVAL;
  if (!valid_block_size(block_size)) return PKV_ENOTSUP;
  if (head_dim != 64 && head_dim != 128) return PKV_ENOTSUP;
  if (num_heads / num_kv_heads > kMaxGroup) return PKV_ENOTSUP;
  // token counts stay in int32
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return PKV_ENOTSUP;
  if (!is_cache_dtype(cache_dtype)) return PKV_EINVAL;
  if (out_dtype != PKV_F32 && out_dtype != PKV_F16) return PKV_EINVAL;
  if (q_dtype != (cache_dtype == PKV_F32 ? PKV_F32 : PKV_F16)) return PKV_ENOTSUP;
  if (!valid_partition(partition_size, block_size)) return PKV_EINVAL;
  if (!(scale == scale)) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens) return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (!aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, elem_bytes(out_dtype)) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4))
    return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!aligned(k_scale, 8) || !aligned(v_scale, 8)))
    return PKV_EINVAL;

  const DecodePlan pl = plan_decode((int64_t)num_seqs * num_kv_heads, max_blocks_per_seq,
                                    block_size, partition_size, extra_parts,
                                    num_heads / num_kv_heads, head_dim);
  const int32_t pt = pl.part_tiles;
  const int32_t parts = pl.num_parts;
  if ((int64_t)num_seqs * num_heads > INT32_MAX ||
      (int64_t)num_seqs * num_kv_heads * 2 > INT32_MAX ||
      (pl.walk != kWalkStream && decode_grid(num_seqs * num_kv_heads, pl.num_runs) > INT32_MAX))
    return PKV_ENOTSUP;
  const WorkspaceLayout wl =
      workspace_layout(pl, num_seqs, num_heads, num_kv_heads, head_dim, extra_parts);
  const size_t need = wl.total;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return PKV_EINVAL;
  const int dev = check_device();
  if (dev != PKV_OK) return dev;

  DecodeParams p{};
  p.out = out;
  p.q = query;
  p.k_cache = static_cast<const uint8_t *>(k_cache);
  p.v_cache = static_cast<const uint8_t *>(v_cache);
  p.k_scale = static_cast<const uint16_t *>(k_scale);
  p.v_scale = static_cast<const uint16_t *>(v_scale);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  char *ws = static_cast<char *>(workspace);
  p.ws_o = need ? reinterpret_cast<float *>(ws + wl.o_off) : nullptr;
  p.ws_lse = need ? reinterpret_cast<float *>(ws + wl.lse_off) : nullptr;
  p.ws_info = need && pl.walk == kWalkStream ? reinterpret_cast<int32_t *>(ws + wl.info_off)
                                             : nullptr;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_heads / num_kv_heads;
  p.block_size = block_size;
  p.part_tiles = pt;
  p.num_parts = parts;
  p.walk = pl.walk;
  p.run_parts = pl.run_parts;
  p.num_runs = pl.num_runs;
  p.stream_waves = pl.stream_waves;
  p.min_share = kStreamMinShare;
  // stream walk: a unit's piece count is known on the device only; the merge
  // sizes its partial groups for about one piece per 64 tiles of the table
  p.ws_stride = pl.walk == kWalkStream
                    ? (int32_t)((max_tiles_of(max_blocks_per_seq, block_size) + 63) / 64 + 2)
                    : parts + extra_parts;
  p.ws_pre = parts;
  p.num_units = num_seqs * num_kv_heads;
  p.qk_scale = scale * 1.4426950408889634f;
  *pp = p;
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_attention_decode(void *out, int32_t out_dtype, const void *query, int32_t q_dtype,
                           const void *k_cache, const void *v_cache, const void *k_scale,
                           const void *v_scale, int32_t cache_dtype, int32_t num_blocks,
                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           float scale, int32_t partition_size, void *workspace,
                           size_t workspace_bytes, void *stream) {
  DecodeParams p{};
  const int st = prepare_decode(&p, out, out_dtype, query, q_dtype, k_cache, v_cache, k_scale,
                                v_scale, cache_dtype, num_blocks, block_tables,
                                max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads,
                                head_dim, block_size, scale, partition_size, workspace,
                                workspace_bytes);
  if (st != PKV_OK || num_seqs == 0) return st;
  return status_of(launch_decode(p, cache_dtype, out_dtype, head_dim,
                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Scratch of paged_attention_decode_noalloc: the split-K partials live in
// this file-scope device array instead of a caller's workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  On the host the
// name `scratch` is only a stand-in for the symbol, never a device address:
// host code uses the address scratch_ptr looks up.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

// This device's address of `scratch`, looked up with hipGetSymbolAddress the
// first time a device calls (with that device current) and kept per device.
int scratch_ptr(void **out) {
  static std::mutex mu;
  static void *ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EDEVICE;
  if (dev < 0 || dev >= 64) return PKV_ENOTSUP;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return PKV_EDEVICE;
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_attention_decode_noalloc(void *out, int32_t out_dtype, const void *query,
                                   int32_t q_dtype, const void *k_cache, const void *v_cache,
                                   const void *k_scale, const void *v_scale,
                                   int32_t cache_dtype, int32_t num_blocks,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   float scale, int32_t partition_size, void *stream) {
  // the partials this call needs (0 for one pass per sequence, and for
  // arguments paged_attention_decode rejects)
  const size_t need = paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                                      head_dim, max_blocks_per_seq, block_size,
                                                      partition_size);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ESCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    const int dev = check_device();
    if (dev != PKV_OK) return dev;
    const int st = scratch_ptr(&ws);
    if (st != PKV_OK) return st;
  }
  return paged_attention_decode(out, out_dtype, query, q_dtype, k_cache, v_cache, k_scale,
                                v_scale, cache_dtype, num_blocks, block_tables,
                                max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads,
                                head_dim, block_size, scale, partition_size, ws,
                                need > 0 ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int paged_decode_step(void *out, int32_t out_dtype, const void *query, int32_t q_dtype,
                      const void *key, const void *value, int32_t src_dtype,
                      const int32_t *cow_src, void *k_cache, void *v_cache, void *k_scale,
                      void *v_scale, int32_t cache_dtype, int32_t num_blocks,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *stream) {
  DecodeParams p{};
  const int st = prepare_decode(&p, out, out_dtype, query, q_dtype, k_cache, v_cache, k_scale,
                                v_scale, cache_dtype, num_blocks, block_tables,
                                max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads,
                                head_dim, block_size, scale, partition_size, workspace,
                                workspace_bytes);
  if (st != PKV_OK) return st;
  if (src_dtype != (cache_dtype == PKV_F32 ? PKV_F32 : PKV_F16)) return PKV_ENOTSUP;
  if (num_seqs == 0) return PKV_OK;
  if (!key || !value) return PKV_EINVAL;
  if (!aligned(key, elem_bytes(src_dtype)) || !aligned(value, elem_bytes(src_dtype)) ||
      !aligned(cow_src, 4))
    return PKV_EINVAL;
  p.key_new = key;
  p.value_new = value;
  p.cow_src = cow_src;
  p.k_cache_w = static_cast<uint8_t *>(k_cache);
  p.v_cache_w = static_cast<uint8_t *>(v_cache);
  p.k_scale_w = static_cast<uint16_t *>(k_scale);
  p.v_scale_w = static_cast<uint16_t *>(v_scale);
  return status_of(launch_decode_step(p, cache_dtype, src_dtype, out_dtype, head_dim,
                                      static_cast<hipStream_t>(stream)));
}

int paged_attention_decode_shared(void *out, int32_t out_dtype, const void *query,
                                  int32_t q_dtype, const void *key, const void *value,
                                  int32_t src_dtype, const int32_t *cow_src, void *k_cache,
                                  void *v_cache, void *k_scale, void *v_scale,
                                  int32_t cache_dtype, int32_t num_blocks,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  float scale, const pkv_prefix_groups *groups,
                                  int32_t partition_size, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  if (!groups || groups->num_groups < 0) return PKV_EINVAL;
  if (!valid_block_size(block_size)) return PKV_ENOTSUP;
  if (!valid_groups(groups, block_size)) return PKV_EINVAL;
  const pkv_prefix_groups &gr = *groups;
  if (gr.num_groups > 0 &&
      (!gr.offsets || !gr.members || !gr.tables || !gr.prefix_lens || !gr.seq_group ||
       !aligned(gr.offsets, 4) || !aligned(gr.members, 4) || !aligned(gr.tables, 4) ||
       !aligned(gr.prefix_lens, 4) || !aligned(gr.seq_group, 4)))
    return PKV_EINVAL;
  if (num_heads > 0 && num_kv_heads > 0 && num_heads % num_kv_heads) return PKV_EINVAL;
  const bool step = key != nullptr || value != nullptr;
  PrefixPlan pl;
  if (num_heads > 0 && num_kv_heads > 0)
    pl = plan_prefix(groups, num_heads, num_kv_heads, block_size);
  DecodeParams p{};
  int st = prepare_decode(&p, out, out_dtype, query, q_dtype, k_cache, v_cache, k_scale, v_scale,
                          cache_dtype, num_blocks, block_tables, max_blocks_per_seq, seq_lens,
                          num_seqs, num_heads, num_kv_heads, head_dim, block_size, scale,
                          partition_size, workspace, workspace_bytes, pl.num_pparts);
  if (st != PKV_OK) return st;
  if (step && src_dtype != (cache_dtype == PKV_F32 ? PKV_F32 : PKV_F16)) return PKV_ENOTSUP;
  if (num_seqs == 0) return PKV_OK;
  if (step) {
    if (!key || !value) return PKV_EINVAL;
    if (!aligned(key, elem_bytes(src_dtype)) || !aligned(value, elem_bytes(src_dtype)) ||
        !aligned(cow_src, 4))
      return PKV_EINVAL;
  }
  PrefixParams pp{};
  if (gr.num_groups > 0 && pl.num_pparts > 0) {
    const int64_t units = (int64_t)gr.num_groups * num_kv_heads;
    const int wg_cols = cache_dtype == PKV_F16 ? kPipeSharedCols : 16 * prefix_chunks(cache_dtype);
    const int64_t cols = (int64_t)gr.max_group_size * (num_heads / num_kv_heads);
    const int64_t col_blocks = (cols + wg_cols - 1) / wg_cols;
    if (units > INT32_MAX || col_blocks > INT32_MAX ||
        (int64_t)unit_groups((int)units) * kXcds * col_blocks * pl.num_pparts > INT32_MAX)
      return PKV_ENOTSUP;
    p.seq_group = gr.seq_group;
    p.group_prefix_lens = gr.prefix_lens;
    p.num_groups = gr.num_groups;
    p.max_prefix_blocks = gr.max_prefix_blocks;
    p.pp_tiles = pl.pp_tiles;
    pp.q = query;
    pp.k_cache = p.k_cache;
    pp.v_cache = p.v_cache;
    pp.k_scale = p.k_scale;
    pp.v_scale = p.v_scale;
    pp.offsets = gr.offsets;
    pp.members = gr.members;
    pp.tables = gr.tables;
    pp.prefix_lens = gr.prefix_lens;
    pp.ws_o = p.ws_o;
    pp.ws_lse = p.ws_lse;
    pp.num_blocks = num_blocks;
    pp.num_seqs = num_seqs;
    pp.num_heads = num_heads;
    pp.num_kv_heads = num_kv_heads;
    pp.group = p.group;
    pp.num_groups = gr.num_groups;
    pp.num_members = gr.num_members;
    pp.max_prefix_blocks = gr.max_prefix_blocks;
    pp.num_units = (int)units;
    pp.col_blocks = (int)col_blocks;
    pp.pp_tiles = pl.pp_tiles;
    pp.num_pparts = pl.num_pparts;
    pp.ws_stride = p.ws_stride;
    pp.ws_pre = p.ws_pre;
    pp.qk_scale = p.qk_scale;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (step) {
    p.key_new = key;
    p.value_new = value;
    p.cow_src = cow_src;
    p.k_cache_w = static_cast<uint8_t *>(k_cache);
    p.v_cache_w = static_cast<uint8_t *>(v_cache);
    p.k_scale_w = static_cast<uint16_t *>(k_scale);
    p.v_scale_w = static_cast<uint16_t *>(v_scale);
    err = launch_decode_step(p, cache_dtype, src_dtype, out_dtype, head_dim, s);
  } else {
    err = launch_decode(p, cache_dtype, out_dtype, head_dim, s);
  }
  if (err != hipSuccess || p.seq_group == nullptr) return status_of(err);
  // The prefix pass reads only prefix blocks, which the step neither copies
  // into nor writes; the merge then combines suffix and prefix partials.
  err = launch_prefix(pp, cache_dtype, head_dim, block_size, s);
  if (err != hipSuccess) return status_of(err);
  return status_of(launch_merge(p, out_dtype, head_dim, s));
}

int paged_attention_prefill(void *out, int32_t out_dtype, const void *query, int32_t q_dtype,
                            const void *k_cache, const void *v_cache, const void *k_scale,
                            const void *v_scale, int32_t cache_dtype, int32_t num_blocks,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, const int32_t *query_offsets,
                            int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, float scale, int32_t partition_size,
                            void *workspace, size_t workspace_bytes, void *stream) {
  if (num_seqs < 0 || num_query_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || partition_size < 0)
    return PKV_EINVAL;
  if (num_heads % num_kv_heads) return PKV_EINVAL;
  if (!valid_block_size(block_size)) return PKV_ENOTSUP;
  if (head_dim != 64 && head_dim != 128) return PKV_ENOTSUP;
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return PKV_ENOTSUP;
  if (!is_cache_dtype(cache_dtype)) return PKV_EINVAL;
  if (cache_dtype == PKV_F32) return PKV_ENOTSUP;   // the pass runs on fp16 MFMAs
  if (out_dtype != PKV_F32 && out_dtype != PKV_F16) return PKV_EINVAL;
  if (q_dtype != PKV_F16) return PKV_ENOTSUP;
  if (!valid_prefill_partition(partition_size, block_size)) return PKV_EINVAL;
  if (!(scale == scale)) return PKV_EINVAL;
  if (num_seqs == 0 || num_query_tokens == 0) return PKV_OK;
  if (max_query_len <= 0) return PKV_EINVAL;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens || !query_offsets)
    return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (!aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 4 * elem_bytes(out_dtype)) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4) || !aligned(query_offsets, 4))
    return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!aligned(k_scale, 4) || !aligned(v_scale, 4))) return PKV_EINVAL;
  const PrefillPlan pl = plan_prefill(num_seqs, num_heads, num_kv_heads, max_query_len,
                                      max_blocks_per_seq, block_size, partition_size);
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int wg_cols = cache_dtype == PKV_F16 ? kPipeCols : kPrefixCols;
  const int64_t col_blocks =
      ((int64_t)max_query_len * (num_heads / num_kv_heads) + wg_cols - 1) / wg_cols;
  if ((int64_t)num_query_tokens * num_heads > INT32_MAX || units > INT32_MAX ||
      (int64_t)unit_groups((int)std::min<int64_t>(units, INT32_MAX)) * kXcds * col_blocks *
              pl.num_pparts > INT32_MAX)
    return PKV_ENOTSUP;
  WorkspaceLayout wl{0, 0, 0};
  if (pl.num_pparts > 1) {
    wl = rows_layout(num_query_tokens, num_heads, head_dim, pl.num_pparts);
    if (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256)) return PKV_EINVAL;
  }
  const int dev = check_device();
  if (dev != PKV_OK) return dev;
  PrefixParams pp{};
  pp.q = query;
  pp.k_cache = static_cast<const uint8_t *>(k_cache);
  pp.v_cache = static_cast<const uint8_t *>(v_cache);
  pp.k_scale = static_cast<const uint16_t *>(k_scale);
  pp.v_scale = static_cast<const uint16_t *>(v_scale);
  char *ws = static_cast<char *>(workspace);
  pp.ws_o = wl.total ? reinterpret_cast<float *>(ws + wl.o_off) : nullptr;
  pp.ws_lse = wl.total ? reinterpret_cast<float *>(ws + wl.lse_off) : nullptr;
  pp.num_blocks = num_blocks;
  pp.num_seqs = num_seqs;
  pp.num_heads = num_heads;
  pp.num_kv_heads = num_kv_heads;
  pp.group = num_heads / num_kv_heads;
  pp.num_units = (int)units;
  pp.col_blocks = (int)col_blocks;
  pp.pp_tiles = pl.pp_tiles;
  pp.num_pparts = pl.num_pparts;
  pp.ws_stride = pl.num_pparts;
  pp.ws_pre = 0;
  pp.qk_scale = scale * 1.4426950408889634f;
  pp.block_tables = block_tables;
  pp.seq_lens = seq_lens;
  pp.query_offsets = query_offsets;
  pp.max_blocks = max_blocks_per_seq;
  pp.num_query_tokens = num_query_tokens;
  pp.block_size = block_size;
  pp.out = out;
  return status_of(launch_prefill(pp, cache_dtype, out_dtype, head_dim, block_size,
                                  static_cast<hipStream_t>(stream)));
}

int paged_kv_write(const void *key, const void *value, int32_t src_dtype, int64_t key_stride,
                   int64_t value_stride, const int64_t *slot_mapping, int32_t num_tokens,
                   void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                   int32_t cache_dtype, int32_t num_blocks, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, void *stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || key_stride < 0 ||
      value_stride < 0)
    return PKV_EINVAL;
  if (num_kv_heads > 65535) return PKV_ENOTSUP;
  if (!valid_block_size(block_size)) return PKV_ENOTSUP;
  if (head_dim != 64 && head_dim != 128) return PKV_ENOTSUP;
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16) return PKV_EINVAL;
  if (!is_cache_dtype(cache_dtype)) return PKV_EINVAL;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (key_stride == 0) key_stride = row;
  if (value_stride == 0) value_stride = row;
  if (key_stride < row || value_stride < row) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  const size_t se = elem_bytes(src_dtype);
  if (!aligned(key, se) || !aligned(value, se) || !aligned(slot_mapping, 8) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!aligned(k_scale, 2) || !aligned(v_scale, 2))) return PKV_EINVAL;
  const int dev = check_device();
  if (dev != PKV_OK) return dev;
  WriteParams p;
  p.key = key;
  p.value = value;
  p.key_stride = key_stride;
  p.value_stride = value_stride;
  p.slots = slot_mapping;
  p.k_cache = static_cast<uint8_t *>(k_cache);
  p.v_cache = static_cast<uint8_t *>(v_cache);
  p.k_scale = static_cast<uint16_t *>(k_scale);
  p.v_scale = static_cast<uint16_t *>(v_scale);
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  return status_of(launch_write(p, src_dtype, cache_dtype, head_dim,
                                static_cast<hipStream_t>(stream)));
}

int paged_copy_blocks(void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                      int32_t cache_dtype, int32_t num_blocks, const int32_t *block_pairs,
                      int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, void *stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_EINVAL;
  if (!valid_block_size(block_size)) return PKV_ENOTSUP;
  if (head_dim != 64 && head_dim != 128) return PKV_ENOTSUP;
  if (!is_cache_dtype(cache_dtype)) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 4))
    return PKV_EINVAL;
  const int dev = check_device();
  if (dev != PKV_OK) return dev;
  CopyParams p;
  p.k_cache = static_cast<uint8_t *>(k_cache);
  p.v_cache = static_cast<uint8_t *>(v_cache);
  p.k_scale = static_cast<uint16_t *>(k_scale);
  p.v_scale = static_cast<uint16_t *>(v_scale);
  p.pairs = block_pairs;
  p.num_pairs = num_pairs;
  p.num_blocks = num_blocks;
  p.block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(cache_dtype);
  p.scale_elems = is_quant(cache_dtype) ? (int64_t)num_kv_heads * block_size : 0;
  return status_of(launch_copy(p, static_cast<hipStream_t>(stream)));
}

int paged_swap_blocks(void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                      void *host_k, void *host_v, void *host_k_scale, void *host_v_scale,
                      int32_t cache_dtype, int32_t num_blocks, int32_t num_host_blocks,
                      const int32_t *block_pairs, int32_t num_pairs, int32_t to_host,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      void *stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_host_blocks < 0 || num_kv_heads <= 0 ||
      (to_host != 0 && to_host != 1))
    return PKV_EINVAL;
  if (!valid_block_size(block_size)) return PKV_ENOTSUP;
  if (head_dim != 64 && head_dim != 128) return PKV_ENOTSUP;
  if (!is_cache_dtype(cache_dtype)) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !host_k || !host_v || !block_pairs) return PKV_EINVAL;
  if (is_quant(cache_dtype) && (!k_scale || !v_scale || !host_k_scale || !host_v_scale))
    return PKV_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(host_k, 16) ||
      !aligned(host_v, 16) || !aligned(block_pairs, 4))
    return PKV_EINVAL;
  const int dev = check_device();
  if (dev != PKV_OK) return dev;
  SwapParams p{};
  p.dev_k = static_cast<uint8_t *>(k_cache);
  p.dev_v = static_cast<uint8_t *>(v_cache);
  p.dev_ks = static_cast<uint16_t *>(k_scale);
  p.dev_vs = static_cast<uint16_t *>(v_scale);
  p.host_k = static_cast<uint8_t *>(host_k);
  p.host_v = static_cast<uint8_t *>(host_v);
  p.host_ks = static_cast<uint16_t *>(host_k_scale);
  p.host_vs = static_cast<uint16_t *>(host_v_scale);
  p.pairs = block_pairs;
  p.num_pairs = num_pairs;
  p.num_blocks = num_blocks;
  p.num_host_blocks = num_host_blocks;
  p.to_host = to_host;
  p.block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(cache_dtype);
  p.scale_elems = is_quant(cache_dtype) ? (int64_t)num_kv_heads * block_size : 0;
  return status_of(launch_swap(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
