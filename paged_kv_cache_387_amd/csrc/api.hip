// C ABI of libpkv: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is enqueued.
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
    pt = (pt + kWaves - 1) / kWaves * kWaves;
  }
  return pt >= mt ? (int32_t)mt : (int32_t)pt;
}

int32_t num_parts_of(int32_t max_blocks, int32_t block_size, int32_t part_tiles) {
  const int64_t mt = max_tiles_of(max_blocks, block_size);
  return odd_up((int32_t)((mt + part_tiles - 1) / part_tiles));
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace: [partial outputs][partial lse], each part 256-byte aligned.
struct WorkspaceLayout {
  size_t o_off, lse_off, total;
};

WorkspaceLayout workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t num_parts) {
  WorkspaceLayout w{0, 0, 0};
  if (num_parts <= 1) return w;
  const size_t rows = (size_t)num_seqs * num_heads * num_parts;
  w.o_off = 0;
  w.lse_off = round256(rows * head_dim * sizeof(float));
  w.total = w.lse_off + rows * sizeof(float);
  return w;
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

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || !valid_block_size(block_size) ||
      !valid_partition(partition_size, block_size))
    return 0;
  const int32_t pt = choose_part_tiles(max_blocks_per_seq, block_size, partition_size);
  const int32_t parts = num_parts_of(max_blocks_per_seq, block_size, pt);
  return workspace_layout(num_seqs, num_heads, head_dim, parts).total;
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
                   int32_t partition_size, void *workspace, size_t workspace_bytes) {
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

  const int32_t pt = choose_part_tiles(max_blocks_per_seq, block_size, partition_size);
  const int32_t parts = num_parts_of(max_blocks_per_seq, block_size, pt);
  if ((int64_t)num_seqs * num_heads > INT32_MAX || (int64_t)num_seqs * num_kv_heads > INT32_MAX ||
      decode_grid(num_seqs * num_kv_heads, parts) > INT32_MAX)
    return PKV_ENOTSUP;
  const WorkspaceLayout wl = workspace_layout(num_seqs, num_heads, head_dim, parts);
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
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_heads / num_kv_heads;
  p.block_size = block_size;
  p.part_tiles = pt;
  p.num_parts = parts;
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

}  // extern "C"
