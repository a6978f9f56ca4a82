/*
 * pkv.h -- C ABI of libpkv: paged KV cache and PagedAttention decode for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (pages cited by title/site and section):
 *  [7yue]   "KV Cache and PagedAttention (vllm-musa)", 7yue.com, m8-l2
 *  [jsqmd]  "vLLM PagedAttention deep dive and engineering practice", jsqmd.com
 *  [yunthe] "KV cache quantization and PagedAttention memory configuration", yunthe.com
 *  [fairy]  "KVcache-learning" tutorial, fairy2021.github.io (chapters s01..s13)
 *
 * Conventions for every entry point
 *  - Plain C types only.  Pointers documented "device" must point to device
 *    memory of the current HIP device; "host" pointers to host memory.
 *  - The caller owns every buffer.  The library never allocates device memory
 *    (its one device array, the fixed scratch of the allocation-free decode
 *    entry point, exists from the library's load) and keeps no pointer after
 *    a call returns.  Device work is enqueued
 *    asynchronously on `stream` (a hipStream_t passed as void*, NULL = the
 *    default stream); buffers must stay alive until that work completes.
 *  - Arguments are validated on the host before anything is launched; a
 *    negative status means nothing was enqueued (except PKV_EDEVICE, which
 *    reports a launch failure).  No C++ exception crosses this ABI.
 *  - Device-side contents (block tables, slot mappings, sequence lengths) are
 *    the caller's contract; the kernels clamp or skip out-of-range values so
 *    that no access leaves the buffers, but the numbers produced for such
 *    entries are unspecified.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK        0
#define PKV_EINVAL   (-1)  /* bad argument (shape, pointer, alignment, size) */
#define PKV_ENOMEM   (-2)  /* block pool exhausted; allocator state unchanged */
#define PKV_ENOENT   (-3)  /* unknown sequence id */
#define PKV_EEXIST   (-4)  /* sequence id already exists */
#define PKV_EDEVICE  (-5)  /* HIP error while launching */
#define PKV_ENOTSUP  (-6)  /* valid but unsupported (dtype combination, head_dim, GPU arch) */
#define PKV_ESCRATCH (-7)  /* needs more scratch than an allocation-free entry point holds */

/* Static text for a status code. */
const char *pkv_strerror(int status);

/* ---- element types ----------------------------------------------------- */
#define PKV_F32   0   /* IEEE binary32 */
#define PKV_F16   1   /* IEEE binary16 */
#define PKV_I8    3   /* int8 code, symmetric [-127, 127], fp16 scale per (token, kv head) */
#define PKV_E4M3  4   /* OCP 8-bit float E4M3 (bias 7, max 448), fp16 scale per (token, kv head) */

/* Library version as 10000*major + 100*minor + patch. */
int pkv_version(void);

/* ========================================================================
 * KV block pool layout (part of the ABI)
 *
 * A physical block holds block_size (8, 16 or 32) token slots of K and of V
 * for every kv head: "16 tokens x head_dim x num_kv_heads x 2 (K+V) x dtype
 * bytes" [7yue, section 2].  The K pool and the V pool are separate buffers,
 * each [num_blocks][num_kv_heads][slice], slice = block_size * head_dim * eb
 * bytes (eb = element bytes: 4, 2 or 1).  A slice is a run of tiles of
 * TB = min(block_size, 16) tokens (two tiles for 32-token blocks), each
 * TB * head_dim * eb bytes; token t of the block is position u = t % TB of
 * tile t / TB.  Inside a tile, let j be a byte index into the token's
 * head_dim-vector (j = d * eb + byte of element d):
 *   K tile: byte j of token u at ((j / 16) * TB + u) * 16 + j % 16
 *           (16-byte columns, token-minor: the split of the K cache into
 *           [head_dim*eb/16][block_size][16 bytes] of [7yue, section 5])
 *   V tile, PKV_F32 / PKV_F16: byte j of token u at
 *           ((j / 4) * TB + u) * 4 + j % 4   (4-byte columns, token-minor)
 *   V tile, PKV_I8 / PKV_E4M3 (one byte per element, j = d): element d of
 *           token u at ((d / 4) * (TB / 4) + u / 4) * 16 + (d % 4) * 4 + u % 4
 *           (16-byte groups of 4 elements x 4 tokens; each 4-byte word holds
 *           one element of 4 consecutive tokens)
 * Scales (PKV_I8 / PKV_E4M3 only): fp16 [num_blocks][num_kv_heads][block_size],
 * one array for K and one for V.  Slot s of the cache is token position
 * s % block_size of physical block s / block_size.
 * ======================================================================== */

/* ========================================================================
 * Host block allocator (the "Block Manager")
 *
 * Fixed-size blocks allocated on demand, returned when a sequence ends
 * [7yue, section 2]; ceil(n / block_size) blocks for n tokens, capacity checked
 * before anything is taken, blocks taken from the head of the free list and
 * freed blocks appended at its tail [jsqmd, section 3.2]; blocks shared between
 * sequences with copy-on-write: a sequence about to write into a shared block
 * copies it, writes into the copy and repoints its own table, the others keep
 * the original [fairy, s05 copy-on-write; s06 alloc / cow / free].  A block's
 * reference count is the number of table entries that point at it; it returns
 * to the free list when that count reaches zero.
 *
 * Host memory only, no GPU calls.  Not thread-safe: the caller serializes
 * calls on one allocator.  Every failing call leaves the state unchanged.
 * ======================================================================== */
typedef struct pkv_alloc pkv_alloc;

/* Create an allocator over blocks 0 .. num_blocks-1.  free_order (host,
 * nullable) is a permutation of 0 .. num_blocks-1 giving the initial free-list
 * order (NULL: ascending).  block_size is 8, 16 or 32 tokens.  *out receives
 * the handle. */
int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order,
                     pkv_alloc **out);
void pkv_alloc_destroy(pkv_alloc *a);
/* Number of free blocks (>= 0), or PKV_EINVAL for a NULL handle. */
int32_t pkv_alloc_num_free(const pkv_alloc *a);
/* Copy up to cap free-list entries (head first) into out (host); returns the
 * free-list length. */
int32_t pkv_alloc_free_list(const pkv_alloc *a, int32_t *out, int32_t cap);
/* Reference count of a block (0 = free), or PKV_EINVAL if out of range. */
int32_t pkv_block_refcount(const pkv_alloc *a, int32_t block);

/* Grow sequence seq_id (created if new) to num_tokens filled tokens, taking
 * ceil(num_tokens/block_size) - (blocks held) new blocks ("allocate(seq_id, num_tokens)"
 * of [jsqmd, section 3.2]).  If the sequence's partly filled tail block is shared
 * and the call adds tokens to it, that block is first replaced by a private
 * copy: *cow_src / *cow_dst (host, nullable) receive the pair to copy with
 * paged_copy_blocks before any write; both are -1 when no copy is needed.
 * num_tokens <= current length is a no-op.  PKV_ENOMEM if the free list is too
 * short. */
int pkv_seq_allocate(pkv_alloc *a, int64_t seq_id, int32_t num_tokens, int32_t *cow_src,
                     int32_t *cow_dst);
/* Reserve the slot of the next token of an existing sequence (a new block
 * every block_size-th token [fairy, s06 decode-phase allocation]); *slot (host)
 * receives it.  Copy-on-write as for pkv_seq_allocate. */
int pkv_seq_append_slot(pkv_alloc *a, int64_t seq_id, int64_t *slot, int32_t *cow_src,
                        int32_t *cow_dst);
/* pkv_seq_append_slot for n sequences in order (host arrays).  slots[i]
 * receives sequence i's slot; the copy pairs are written to cow_pairs as
 * [src, dst] rows and their count to *num_cow (cow_pairs needs room for n
 * rows); cow_src (nullable, [n]) receives for each sequence the source block
 * of its copy (the destination is its new tail block), -1 if none -- the form
 * paged_decode_step takes.  All or nothing: the blocks the whole batch takes
 * (a new block at each block boundary, a copy for each shared partly filled
 * tail; a sequence may appear more than once) are counted first, and a
 * failing call (PKV_ENOENT, PKV_EINVAL for a swapped-out sequence, PKV_ENOMEM)
 * changes nothing.  *num_done (nullable) receives how many sequences were
 * appended: n on success, 0 on failure. */
int pkv_seq_append_slots(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int64_t *slots,
                         int32_t *cow_pairs, int32_t *num_cow, int32_t *cow_src,
                         int32_t *num_done);
/* One decode step of the allocator in one call: pkv_seq_append_slots for the
 * n sequences (all or nothing, as there), then their block tables and lengths
 * as pkv_export_tables writes them -- the inputs of paged_decode_step
 * (block_tables, seq_lens, cow_src) for a batch whose every sequence gains
 * one token [fairy, s06 decode-phase allocation].  slots (host [n], nullable)
 * receives the new tokens' slots, cow_src (host [n]) each sequence's copy
 * source block or -1, out_block_tables (host [n][max_blocks_per_seq], padded
 * with -1) and out_seq_lens (host [n]) the state after the appends.
 * PKV_EINVAL, and no change, also when a table would outgrow
 * max_blocks_per_seq. */
int pkv_seq_step(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int32_t max_blocks_per_seq,
                 int64_t *slots, int32_t *cow_src, int32_t *out_block_tables,
                 int32_t *out_seq_lens);
/* Make child share every block of parent (reference counts + 1). */
int pkv_seq_fork(pkv_alloc *a, int64_t parent, int64_t child);
/* Release a sequence; blocks whose count drops to zero go to the free-list tail
 * in logical order. */
int pkv_seq_free(pkv_alloc *a, int64_t seq_id);
/* Current length in tokens. */
int pkv_seq_len(const pkv_alloc *a, int64_t seq_id, int32_t *len);
/* Slots of token positions [start, start+count) of a sequence (host out);
 * the positions must be < the sequence length. */
int pkv_seq_slots(const pkv_alloc *a, int64_t seq_id, int32_t start, int32_t count,
                  int64_t *out_slots);
/* Block tables of n sequences as rows of max_blocks_per_seq int32 entries
 * (host [n][max_blocks_per_seq], padded with -1) and their lengths (host [n]).
 * PKV_EINVAL if a table is longer than max_blocks_per_seq. */
int pkv_export_tables(const pkv_alloc *a, const int64_t *seq_ids, int32_t n,
                      int32_t max_blocks_per_seq, int32_t *out_block_tables,
                      int32_t *out_seq_lens);
/* ---- swapping to a host block pool ("swap_out(blocks, cpu_blocks) /
 * swap_in(blocks, gpu_blocks)" when device memory runs short [fairy, s06];
 * swapped-out KV kept in CPU memory [yunthe, preemption / swap_space]) ----
 * The allocator keeps a second pool of num_host_blocks host blocks with its
 * own FIFO free list and reference counts.  A swapped-out sequence's table
 * holds host blocks; it may only be freed or swapped back in (other calls on
 * it return PKV_EINVAL).  Data moves with paged_swap_blocks. */
/* Set the host pool size (free list 0 .. n-1); PKV_EINVAL while a sequence
 * is swapped out. */
int pkv_alloc_set_host_blocks(pkv_alloc *a, int32_t num_host_blocks);
int32_t pkv_alloc_num_free_host(const pkv_alloc *a);
int32_t pkv_alloc_free_list_host(const pkv_alloc *a, int32_t *out, int32_t cap);
int32_t pkv_host_block_refcount(const pkv_alloc *a, int32_t block);
/* *on_host (host) = 1 if the sequence is swapped out. */
int pkv_seq_on_host(const pkv_alloc *a, int64_t seq_id, int32_t *on_host);
/* Move n sequences (distinct, on the device) to the host pool, all or
 * nothing.  Each distinct device block of their tables, in order of first
 * appearance, gets one host block from the head of the host free list (so
 * blocks the sequences share stay shared); pairs (host, [cap][2]) receives
 * [device, host] rows -- copy them with paged_swap_blocks(to_host = 1) -- and
 * *num_pairs their count.  The sequences' references to the device blocks are
 * dropped (blocks other sequences still use stay).  PKV_ENOMEM if the host
 * free list is too short, PKV_EINVAL if cap is. */
int pkv_seq_swap_out(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int32_t *pairs,
                     int32_t cap, int32_t *num_pairs);
/* The reverse for n swapped-out sequences: each distinct host block gets a
 * device block (prefix-cache blocks are evicted if the free list is short);
 * pairs receives [host, device] rows (paged_swap_blocks(to_host = 0)); host
 * blocks whose count drops to zero return to the host free-list tail. */
int pkv_seq_swap_in(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int32_t *pairs,
                    int32_t cap, int32_t *num_pairs);

/* ---- automatic prefix caching [fairy, s08 APC: "each physical block is
 * indexed by the hash of its content" and a request whose prompt starts with
 * a cached block sequence reuses those blocks; jsqmd, section 4.2] ----
 * Reading of the pages' per-block hash: a block's K/V depend on every token
 * before it, so its key is the whole token prefix through that block -- a
 * chained 64-bit hash, and a hit is verified exactly (the block's own tokens
 * and its parent cached block).  Only full blocks are cached.  The cache holds
 * one reference to each cached block; blocks that only the cache holds are
 * evictable, least recently released first, and every allocating call evicts
 * them (to the free-list tail) when the free list is too short. */
/* Create seq_id (must be new) for a prompt of n tokens (host int32 token ids):
 * the longest run of leading full blocks found in the cache is shared, the
 * rest is taken from the free list.  *num_cached_tokens receives the shared
 * tokens (a multiple of block_size), whose K/V need not be computed.
 * PKV_ENOMEM (nothing changed) if the blocks cannot be found. */
int pkv_seq_allocate_cached(pkv_alloc *a, int64_t seq_id, const int32_t *tokens, int32_t n,
                            int32_t *num_cached_tokens);
/* Register the full blocks of the first n tokens of seq_id (their K/V
 * written; tokens = the sequence's token ids) in the cache, from the first
 * block on; stops at a block whose prefix is cached as another block's or
 * whose block is cached under another prefix. */
int pkv_seq_cache_blocks(pkv_alloc *a, int64_t seq_id, const int32_t *tokens, int32_t n);
/* Evict up to max_blocks cache-only blocks (least recently released first). */
int pkv_prefix_cache_evict(pkv_alloc *a, int32_t max_blocks, int32_t *num_evicted);
/* Number of cached blocks. */
int32_t pkv_prefix_cache_size(const pkv_alloc *a);
/* The evictable blocks, least recently released first (up to cap into out);
 * returns their count. */
int32_t pkv_prefix_cache_evictable(const pkv_alloc *a, int32_t *out, int32_t cap);

/* Tables of n sequences split into shared prefixes and private suffixes, the
 * input of paged_attention_decode_shared.  Sequences forked from one parent
 * share the physical blocks of their common beginning [fairy, s05
 * copy-on-write, s08 prefix sharing]; a group is every sequence (two or more
 * of seq_ids) whose first table entry is the same physical block, numbered in
 * order of its first member.  The group's prefix is the longest run of leading
 * entries common to all members, cut to blocks every member has filled, to
 * max_prefix_blocks and to a multiple of 16 tokens; a group whose prefix is
 * shorter than max(16, min_prefix_tokens) tokens is not formed.  One level of
 * sharing: sequences that share more than their group's common run still
 * read the rest as suffix.  Host outputs:
 *   suffix_tables [n][max_suffix_blocks] (padded with -1): each table without
 *       its group's prefix entries; suffix_lens [n]: length minus prefix.
 *   seq_group [n]: group of each sequence, -1 for none.
 *   group_offsets [n/2 + 1 or more], group_members [n]: the members of group g
 *       (indices into seq_ids, ascending) are group_members[group_offsets[g]
 *       .. group_offsets[g+1]).
 *   group_tables [n/2 or more][max_prefix_blocks] (padded with -1) and
 *       group_prefix_lens [n/2 or more] (tokens): each group's prefix.
 *   *num_groups, *max_group_size (0 without groups).
 * PKV_ENOENT for an unknown id, PKV_EINVAL if a suffix is longer than
 * max_suffix_blocks (nothing is written then). */
int pkv_export_shared_tables(const pkv_alloc *a, const int64_t *seq_ids, int32_t n,
                             int32_t min_prefix_tokens, int32_t max_prefix_blocks,
                             int32_t max_suffix_blocks, int32_t *suffix_tables,
                             int32_t *suffix_lens, int32_t *seq_group, int32_t *group_offsets,
                             int32_t *group_members, int32_t *group_tables,
                             int32_t *group_prefix_lens, int32_t *num_groups,
                             int32_t *max_group_size);

/* ========================================================================
 * Device operations (gfx950 HIP kernels)
 * ======================================================================== */

/* Cache write ("append the new token's K/V to the cache" [fairy, s02]; the
 * per-token slot addressing of the block table [7yue, section 5]).
 *   key, value:  device, [num_tokens][num_kv_heads][head_dim] of src_dtype
 *                (PKV_F32 or PKV_F16); row i starts at element i*key_stride
 *                (value_stride for value); a stride of 0 means num_kv_heads*head_dim.
 *   slot_mapping: device int64 [num_tokens]; token i goes to slot
 *                slot_mapping[i]; a negative or >= num_blocks*block_size slot
 *                skips the token (padding).
 *   k_cache, v_cache: device pools of cache_dtype in the layout above.
 *   k_scale, v_scale: device fp16 scale arrays, required for PKV_I8 / PKV_E4M3
 *                (NULL otherwise).
 * Conversion: F16<-F16 and F32<-F32 copy bits; F16<-F32 rounds to nearest even;
 * F32<-F16 widens.  Quantized caches (one scale per (token, kv head), separately
 * for K and V; "KV Cache scaling factor" [fairy, s09], int8 / fp8 KV [yunthe,
 * quantization section]):
 *   a = max_d |x_d|;  s32 = a / 127 (int8) or a / 448 (E4M3), IEEE fp32 division;
 *   s = fp16(s32) rounded to nearest even, stored as the scale;
 *   s == 0 -> all codes 0;  int8 code = clamp(rint_even(x_d / s), -127, 127);
 *   E4M3 code = nearest-even E4M3 of x_d / s, saturating at +-448.
 *   The dequantized value code * s is exact in fp32.  Source values must be
 *   finite (and, for PKV_F32 sources, a / 127 or a / 448 must fit in fp16).
 * Destination slots must be distinct within one call. */
int paged_kv_write(const void *key, const void *value, int32_t src_dtype,
                   int64_t key_stride, int64_t value_stride,
                   const int64_t *slot_mapping, int32_t num_tokens,
                   void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                   int32_t cache_dtype, int32_t num_blocks, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, void *stream);

/* Copy-on-write block copy [fairy, s05 copy-on-write; s06 "cow(seq_group,
 * block_id) -> new_physical_block"]: for each row [src, dst] of block_pairs
 * (device int32 [num_pairs][2]) copy the whole physical block src to dst -- the
 * K and V tiles of every kv head and, for quantized caches, their scales.
 * Rows with src or dst outside [0, num_blocks) or src == dst are skipped.
 * Destinations must be distinct and must not be sources of the same call.
 * Enqueue it before the paged_kv_write of the same step, on the same stream. */
int paged_copy_blocks(void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                      int32_t cache_dtype, int32_t num_blocks, const int32_t *block_pairs,
                      int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, void *stream);

/* Block swap between the device pools and host pools of the same layout
 * (swap_out / swap_in [fairy, s06]): for each row of pairs (device int32
 * [num_pairs][2]) copy the whole block -- K and V of every kv head and, for
 * quantized caches, the scales -- from device block row[0] to host block
 * row[1] (to_host = 1) or from host block row[0] to device block row[1]
 * (to_host = 0).  host_k, host_v (and host_k_scale, host_v_scale) are host
 * pools of num_host_blocks blocks in pinned memory that the device can
 * address (hipHostMalloc / torch pin_memory); the copy runs as a kernel over
 * the host link.  Rows with an index out of range are skipped; destinations
 * must be distinct. */
int paged_swap_blocks(void *k_cache, void *v_cache, void *k_scale, void *v_scale,
                      void *host_k, void *host_v, void *host_k_scale, void *host_v_scale,
                      int32_t cache_dtype, int32_t num_blocks, int32_t num_host_blocks,
                      const int32_t *block_pairs, int32_t num_pairs, int32_t to_host,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, void *stream);

/* Partition size (tokens) paged_attention_decode uses for these shapes when
 * asked for `requested` (0 = the library's choice); a value >=
 * max_blocks_per_seq*block_size means one pass per (sequence, kv head).
 * With requested = 0 and a smaller value the call does not cut fixed
 * partitions: it deals the batch's tiles to the GPU's waves in equal shares
 * (PKV_WALK_STREAM below), and the value only records that it splits. */
int32_t paged_attention_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t requested);

/* How paged_attention_decode (and paged_decode_step) spreads the work for
 * these shapes; returns one of the values below, or PKV_EINVAL.
 *   PKV_WALK_SPLIT:  one workgroup per (sequence, kv head, partition); a
 *                    table of one partition is the single pass.
 *   PKV_WALK_RUNS:   explicit partitions of a multiple of 64 tokens: one
 *                    workgroup walks a run of consecutive partitions of a
 *                    (sequence, kv head), each ending in its own partial.
 *   PKV_WALK_STREAM: the library's choice for tables of several partitions:
 *                    the batch's 16-token tiles, in (sequence, kv head, tile)
 *                    order, are dealt to the waves in equal shares of whole
 *                    blocks, so ragged lengths still give every wave the same
 *                    bytes; a (sequence, kv head) split between shares is
 *                    merged by the log-sum-exp reduction.
 * The results do not depend on the walk beyond fp32 rounding order. */
#define PKV_WALK_SPLIT 0
#define PKV_WALK_RUNS 1
#define PKV_WALK_STREAM 2
int32_t paged_attention_decode_walk(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_size);

/* Bytes of device workspace paged_attention_decode needs for these shapes
 * (0 when every sequence fits one partition): the partial outputs and their
 * log-sum-exps, fp32 (PKV_WALK_STREAM: two slots of a kv head's query rows
 * per wave, and an 8-byte record per (sequence, kv head)). */
size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size);

/* PagedAttention decode: each sequence's single query token attends over its
 * cached K/V, reached through its block table [7yue, section 5 kernel entry:
 * q [num_seqs, num_heads, head_size], block_tables [num_seqs,
 * max_num_blocks_per_seq], seq_lens [num_seqs]; fairy, s05]:
 *   out[s][h][:] = softmax_t(scale * q[s][h] . K[s][t]) V[s][t],  t < seq_lens[s]
 * (the attention formula of [fairy, s01]; paging does not change the math
 * [jsqmd, section 9]).  Query head h uses kv head h / (num_heads/num_kv_heads)
 * (grouped-query attention, num_kv_heads <= num_heads [fairy, s11]).
 *   out:     device [num_seqs][num_heads][head_dim] of out_dtype (F32 or F16),
 *            aligned to its element size (written with 4-element vector
 *            stores when 16-byte (F32) or 8-byte (F16) aligned).
 *   query:   device [num_seqs][num_heads][head_dim], q_dtype = F32 when
 *            cache_dtype is F32, else F16; 16-byte aligned.
 *   k_cache, v_cache, k_scale, v_scale, cache_dtype, num_blocks: the pools.
 *   block_tables: device int32 [num_seqs][max_blocks_per_seq]; entry i is the
 *            physical block of tokens i*block_size .. (i+1)*block_size - 1.
 *            Entries past ceil(seq_len/block_size) are never read.
 *   seq_lens: device int32 [num_seqs], tokens already in the cache including
 *            the one just written; 0 gives a zero output row.
 *   head_dim 64 or 128; block_size 8, 16 or 32; num_heads/num_kv_heads <= 16.
 *   partition_size: tokens per partition along the sequence (a multiple of
 *            16 and of block_size; 0 = library choice).  Longer sequences are split;
 *            the partial results (max, sum, weighted V) of the partitions are
 *            merged by a log-sum-exp reduction ("partial accumulate, then
 *            merge", paged_attention_v2 of [jsqmd, section 4.1]).  When the
 *            size is a multiple of 64 tokens, one workgroup may walk several
 *            consecutive partitions of a sequence (up to the library's own
 *            partition size); that changes the schedule, not the partials.
 *            The library's choice splits at share boundaries instead of
 *            fixed partitions (paged_attention_decode_walk).
 *   workspace: device, >= paged_attention_workspace_bytes(...) bytes,
 *            256-byte aligned (may be NULL when that size is 0); its contents
 *            on entry do not matter.  Calls that share a workspace must not
 *            run concurrently (same stream, or otherwise ordered).
 * Arithmetic: fp32 scores, softmax and accumulation; q.k products on MFMA from
 * the stored values; int8/E4M3 values are dequantized exactly (code*scale). */
int paged_attention_decode(void *out, int32_t out_dtype, const void *query, int32_t q_dtype,
                           const void *k_cache, const void *v_cache, const void *k_scale,
                           const void *v_scale, int32_t cache_dtype, int32_t num_blocks,
                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           float scale, int32_t partition_size, void *workspace,
                           size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it): the same call as
 * paged_attention_decode, with the same results and the same kernels, but the
 * split-K partials go to the library's own scratch array instead of a caller
 * workspace -- one static device array of PKV_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends.  Nothing is allocated or freed.  A call whose
 * partials need more than that (paged_attention_workspace_bytes of the same
 * arguments) returns PKV_ESCRATCH and enqueues nothing.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, not otherwise ordered) race and must not be issued; calls on one
 * stream are ordered and safe.  The array's contents on entry do not matter.
 * Other arguments and errors as paged_attention_decode. */
#define PKV_NOALLOC_SCRATCH_BYTES (48u << 20)
int paged_attention_decode_noalloc(void *out, int32_t out_dtype, const void *query,
                                   int32_t q_dtype, const void *k_cache, const void *v_cache,
                                   const void *k_scale, const void *v_scale,
                                   int32_t cache_dtype, int32_t num_blocks,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   float scale, int32_t partition_size, void *stream);

/* Fused decode step: for every sequence s with L = seq_lens[s] > 0,
 *   1. if cow_src (nullable, device int32 [num_seqs]) has cow_src[s] >= 0,
 *      copy block cow_src[s] into the sequence's tail block
 *      block_tables[s][(L-1)/block_size] (copy-on-write [fairy, s05]);
 *   2. write the sequence's new token -- row s of key / value, device
 *      [num_seqs][num_kv_heads][head_dim] of src_dtype -- at position L - 1,
 *      i.e. slot block_tables[s][(L-1)/bs] * bs + (L-1) % bs (bs =
 *      block_size), quantizing as
 *      paged_kv_write does ("append the new token's K/V" [fairy, s02]);
 *   3. compute out exactly as paged_attention_decode does, over all L tokens
 *      including the new one.
 * One launch (plus the merge when sequences are split) instead of
 * paged_copy_blocks + paged_kv_write + paged_attention_decode, with the same
 * results.  The copy and write of a sequence's kv head are done by the
 * workgroup that reads that tail block.  src_dtype is PKV_F32 for an fp32
 * cache and PKV_F16 otherwise.  The tail blocks written must be distinct
 * sequences' own blocks (the allocator guarantees this: a shared tail is
 * copied first); other sequences may share the copy sources.  Other arguments
 * and errors as paged_attention_decode (the pools are written here). */
int paged_decode_step(void *out, int32_t out_dtype, const void *query, int32_t q_dtype,
                      const void *key, const void *value, int32_t src_dtype,
                      const int32_t *cow_src, void *k_cache, void *v_cache, void *k_scale,
                      void *v_scale, int32_t cache_dtype, int32_t num_blocks,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Groups of sequences that share the physical blocks of a prefix (as
 * pkv_export_shared_tables produces them).  A host struct; the arrays are
 * device int32 memory. */
typedef struct pkv_prefix_groups {
  int32_t num_groups;          /* 0: no sharing (plain decode) */
  int32_t num_members;         /* entries of members */
  int32_t max_group_size;      /* >= the member count of every group */
  int32_t max_prefix_blocks;   /* row stride of tables */
  const int32_t *offsets;      /* [num_groups + 1]: group g is members[offsets[g] .. offsets[g+1]) */
  const int32_t *members;      /* [num_members]: sequence indices (rows of query / tables) */
  const int32_t *tables;       /* [num_groups][max_prefix_blocks]: the prefix's physical blocks */
  const int32_t *prefix_lens;  /* [num_groups]: prefix tokens, a multiple of 16 and of block_size */
  const int32_t *seq_group;    /* [num_seqs]: group of each sequence, -1 for none */
} pkv_prefix_groups;

/* Workspace bytes of paged_attention_decode_shared (max_blocks_per_seq: the
 * suffix tables' width).  0 for invalid arguments. */
size_t paged_attention_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              int32_t partition_size,
                                              const pkv_prefix_groups *groups);

/* Shared-prefix decode: the output of paged_attention_decode (or, with key /
 * value, of paged_decode_step) for sequences whose tables are split into a
 * shared prefix and a private suffix, reading each prefix block once per
 * (group, kv head) instead of once per sequence.  Sequence s attends over its
 * group's prefix (groups->tables[g], groups->prefix_lens[g] tokens, g =
 * groups->seq_group[s]) followed by its suffix (block_tables[s],
 * seq_lens[s] tokens): the token order of its full table.  Sharing of blocks
 * between requests with reference counts is the page's [7yue, section 2;
 * fairy, s05, s08]; that each sharer's softmax over prefix + suffix is the
 * log-sum-exp merge of the softmaxes over the two pieces is the same identity
 * as the split-K merge of paged_attention_v2 [jsqmd, section 4.1].
 *   key, value, src_dtype, cow_src: as paged_decode_step, applied to the
 *       suffix (the new token is position seq_lens[s] - 1 of the suffix);
 *       both NULL for decode only.
 *   block_tables, max_blocks_per_seq, seq_lens: the suffixes.
 *   groups: host struct (see above); num_groups = 0 runs the plain path.
 *       Contract: each member's full table is the group's prefix followed by
 *       its suffix table, and every sequence is a member of its seq_group.
 *       The prefix kernels read the blocks of groups->tables only.
 *   workspace: >= paged_attention_shared_workspace_bytes(...) bytes, 256-byte
 *       aligned.
 * Other arguments, arithmetic and errors as paged_attention_decode.  Three
 * launches: the (suffix) decode or step kernel, the prefix kernel (all of a
 * group's query heads of one kv head against each prefix tile, on MFMA), and
 * the merge. */
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
                                  size_t workspace_bytes, void *stream);

/* Multi-token queries over the paged cache (prefill and chunked prefill):
 * sequence s has the query rows query_offsets[s] .. query_offsets[s+1] - 1
 * (q_len of them); they are the last q_len of its seq_lens[s] tokens, whose
 * K/V are already in the cache (paged_kv_write first).  Query i sits at
 * position P = seq_lens[s] - q_len + i and attends over tokens 0 .. P -- the
 * cached context and the new tokens up to itself [fairy, s01 attention, s04
 * incremental generation; prefill then decode, 7yue, section 1]:
 *   out[query_offsets[s] + i][h] = softmax_{t <= P}(scale * q . K_t) V_t
 *   out:     device [num_query_tokens][num_heads][head_dim], F32 or F16.
 *   query:   device [num_query_tokens][num_heads][head_dim], F16, 16-byte aligned.
 *   query_offsets: device int32 [num_seqs + 1], non-decreasing, last =
 *            num_query_tokens; q_len <= seq_lens[s] and <= max_query_len (host
 *            bound that sizes the launch; rows of longer queries are not
 *            written).
 *   cache_dtype F16, I8 or E4M3 (the pass runs on fp16 MFMAs; F32 caches give
 *   PKV_ENOTSUP); head_dim 64 or 128; block_size 8, 16 or 32.
 *   partition_size: tokens per partition of the keys (a multiple of 32 and
 *            of block_size; 0 = library choice: one pass per (sequence, kv
 *            head, 64 query columns) unless that leaves compute units idle).
 *            With several partitions the partial results go through the
 *            workspace and a log-sum-exp merge.
 *   workspace: >= paged_attention_prefill_workspace_bytes(...) bytes (0 with
 *            one partition), 256-byte aligned.
 * Arithmetic and errors as paged_attention_decode. */
size_t paged_attention_prefill_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens,
                                               int32_t max_query_len, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_blocks_per_seq, int32_t block_size,
                                               int32_t partition_size);
int paged_attention_prefill(void *out, int32_t out_dtype, const void *query, int32_t q_dtype,
                            const void *k_cache, const void *v_cache, const void *k_scale,
                            const void *v_scale, int32_t cache_dtype, int32_t num_blocks,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, const int32_t *query_offsets,
                            int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, float scale, int32_t partition_size,
                            void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
