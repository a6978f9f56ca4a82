// Host block allocator: free list, per-sequence block tables, reference
// counts and copy-on-write.
//
// Behaviour (see include/pkv.h for the contract):
//  - blocks for n tokens: ceil(n / block_size); capacity is checked before any
//    block is taken, so a failing call changes nothing; blocks are taken from
//    the head of the free list and released blocks are appended at its tail
//    ("vLLM PagedAttention deep dive", jsqmd.com, section 3.2 BlockManager);
//  - allocation on demand, release at the end of a request, sharing of blocks
//    between requests ("KV Cache and PagedAttention (vllm-musa)", 7yue.com,
//    section 2);
//  - copy-on-write: a sequence about to add tokens to a shared, partly filled
//    tail block gets a private copy first and repoints its table; the other
//    sharers keep the original ("KVcache-learning", fairy2021.github.io, s05).
//
// The free list is a ring buffer of capacity num_blocks (every block is either
// free or referenced, so it never overflows).  Sequences live in a hash map.
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"

struct pkv_seq {
  std::vector<int32_t> blocks;   // device blocks, or host blocks while swapped out
  int32_t len = 0;
  bool on_host = false;
};

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::vector<int32_t> ring;   // free list storage
  int32_t head = 0;            // index of the first free entry
  int32_t count = 0;           // number of free blocks
  std::vector<int32_t> ref;    // table entries (+1 when cached) pointing at each block
  std::unordered_map<int64_t, pkv_seq> seqs;

  // host block pool for swapped-out sequences (FIFO free list like the device one)
  int32_t num_host = 0;
  std::deque<int32_t> host_free;
  std::vector<int32_t> host_ref;

  // prefix cache: full blocks indexed by the hash of the token prefix through
  // them (chained block by block); each cached block keeps its own tokens and
  // the key of the prefix before it, which a hit must match -- exact up to a
  // 64-bit collision of that preceding key.  The cache holds one reference to
  // each cached block; blocks only the cache holds are evictable, least
  // recently released first.
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::vector<char> cached;
  std::vector<uint64_t> key;
  std::vector<uint64_t> parent_key;
  std::vector<std::vector<int32_t>> block_tokens;
  std::list<int32_t> lru;
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<char> in_lru;

  int32_t pop_front() {
    int32_t b = ring[head];
    head = (head + 1 == num_blocks) ? 0 : head + 1;
    --count;
    return b;
  }
  void push_back(int32_t b) {
    int32_t pos = head + count;
    if (pos >= num_blocks) pos -= num_blocks;
    ring[pos] = b;
    ++count;
  }
  int32_t blocks_for(int32_t n) const { return (n + block_size - 1) / block_size; }

  // k table entries (or the cache's reference) of block b are gone
  void unref(int32_t b, int32_t k = 1) {
    ref[b] -= k;
    if (ref[b] == 0) {
      push_back(b);
    } else if (ref[b] == 1 && cached[b] && !in_lru[b]) {
      lru_pos[b] = lru.insert(lru.end(), b);
      in_lru[b] = 1;
    }
  }
  void addref(int32_t b) {
    ref[b] += 1;
    if (in_lru[b]) {
      lru.erase(lru_pos[b]);
      in_lru[b] = 0;
    }
  }
  // Drop the least recently released cache-only block: uncached, freed.
  void evict_one() {
    const int32_t b = lru.front();
    lru.pop_front();
    in_lru[b] = 0;
    by_hash.erase(key[b]);
    cached[b] = 0;
    block_tokens[b].clear();
    unref(b);
  }
  // Room for `need` new blocks: evicts as many cache-only blocks as the free
  // list lacks.  False (nothing changed) if even that is not enough.
  bool make_room(int32_t need) {
    if ((int64_t)count + (int64_t)lru.size() < need) return false;
    while (count < need) evict_one();
    return true;
  }
};

namespace {

void set_pair(int32_t *src, int32_t *dst, int32_t s, int32_t d) {
  if (src) *src = s;
  if (dst) *dst = d;
}

// Grow `seq` to n tokens; see pkv_seq_allocate.
int grow(pkv_alloc *a, int64_t seq_id, int32_t n, bool create, int32_t *cow_src,
         int32_t *cow_dst) {
  set_pair(cow_src, cow_dst, -1, -1);
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) {
    if (!create) return PKV_ENOENT;
  } else if (it->second.on_host) {
    return PKV_EINVAL;   // swapped out: swap in first
  }
  const int32_t cur = (it == a->seqs.end()) ? 0 : it->second.len;
  const int32_t held = (it == a->seqs.end()) ? 0 : (int32_t)it->second.blocks.size();
  if (n <= cur) {
    if (it == a->seqs.end()) a->seqs.emplace(seq_id, pkv_seq{});
    return PKV_OK;
  }
  int32_t need = a->blocks_for(n) - held;
  if (need < 0) need = 0;
  const bool cow = (it != a->seqs.end()) && (cur % a->block_size != 0) &&
                   a->ref[it->second.blocks.back()] > 1;
  if (!a->make_room(need + (cow ? 1 : 0))) return PKV_ENOMEM;
  if (it == a->seqs.end()) it = a->seqs.emplace(seq_id, pkv_seq{}).first;
  pkv_seq &s = it->second;
  s.blocks.reserve((size_t)held + need);
  if (cow) {
    const int32_t src = s.blocks.back();
    const int32_t dst = a->pop_front();
    a->ref[dst] = 1;
    a->unref(src);
    s.blocks.back() = dst;
    set_pair(cow_src, cow_dst, src, dst);
  }
  for (int32_t i = 0; i < need; ++i) {
    const int32_t b = a->pop_front();
    a->ref[b] = 1;
    s.blocks.push_back(b);
  }
  s.len = n;
  return PKV_OK;
}

// The check that makes a batch of appends all or nothing: what the whole
// batch takes is found before anything changes.  A sequence's append takes a
// new block at a block boundary; its first append of the batch copies a
// partly filled tail that is shared (counting the copies earlier sequences of
// the batch made of the same block); after that its tail is its own.  Appends
// only take blocks (a copied tail keeps another holder, and partly filled
// blocks are never cached), so the batch succeeds exactly when the free list
// plus the evictable cached blocks cover the total.  With max_blocks > 0 every
// sequence's table must also still fit that width afterwards.
int check_append_batch(const pkv_alloc *a, const int64_t *seq_ids, int32_t n,
                       int32_t max_blocks) {
  try {
    int64_t need = 0;
    std::unordered_map<int64_t, int32_t> seen;   // appends per sequence so far
    std::unordered_map<int32_t, int32_t> moved;  // references copies have taken off a block
    for (int32_t i = 0; i < n; ++i) {
      auto it = a->seqs.find(seq_ids[i]);
      if (it == a->seqs.end()) return PKV_ENOENT;
      if (it->second.on_host) return PKV_EINVAL;
      int32_t &k = seen[seq_ids[i]];
      const int64_t pos = (int64_t)it->second.len + k;
      if (pos >= INT32_MAX) return PKV_EINVAL;
      if (max_blocks > 0 && a->blocks_for((int32_t)pos + 1) > max_blocks) return PKV_EINVAL;
      if (pos % a->block_size == 0) {
        ++need;
      } else if (k == 0) {
        const int32_t tail = it->second.blocks.back();
        int32_t &mv = moved[tail];
        if (a->ref[tail] - mv > 1) {
          ++need;
          ++mv;
        }
      }
      ++k;
    }
    if ((int64_t)a->count + (int64_t)a->lru.size() < need) return PKV_ENOMEM;
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order,
                     pkv_alloc **out) {
  if (!out || num_blocks <= 0 || (block_size != 8 && block_size != 16 && block_size != 32))
    return PKV_EINVAL;
  *out = nullptr;
  pkv_alloc *a = new (std::nothrow) pkv_alloc();
  if (!a) return PKV_ENOMEM;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ring.resize(num_blocks);
    a->ref.assign(num_blocks, 0);
    a->cached.assign(num_blocks, 0);
    a->key.assign(num_blocks, 0);
    a->parent_key.assign(num_blocks, 0);
    a->block_tokens.resize(num_blocks);
    a->lru_pos.resize(num_blocks);
    a->in_lru.assign(num_blocks, 0);
    if (free_order) {
      std::vector<char> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        const int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) {
          delete a;
          return PKV_EINVAL;
        }
        seen[b] = 1;
        a->ring[i] = b;
      }
    } else {
      for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
    }
    a->head = 0;
    a->count = num_blocks;
  } catch (...) {
    delete a;
    return PKV_ENOMEM;
  }
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_alloc *a) { delete a; }

int32_t pkv_alloc_num_free(const pkv_alloc *a) { return a ? a->count : PKV_EINVAL; }

int32_t pkv_alloc_free_list(const pkv_alloc *a, int32_t *out, int32_t cap) {
  if (!a || (cap > 0 && !out)) return PKV_EINVAL;
  for (int32_t i = 0; i < a->count && i < cap; ++i) {
    int32_t pos = a->head + i;
    if (pos >= a->num_blocks) pos -= a->num_blocks;
    out[i] = a->ring[pos];
  }
  return a->count;
}

int32_t pkv_block_refcount(const pkv_alloc *a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return PKV_EINVAL;
  return a->ref[block];
}

int pkv_seq_allocate(pkv_alloc *a, int64_t seq_id, int32_t num_tokens, int32_t *cow_src,
                     int32_t *cow_dst) {
  if (!a || num_tokens < 0) return PKV_EINVAL;
  try {
    return grow(a, seq_id, num_tokens, true, cow_src, cow_dst);
  } catch (...) {
    return PKV_ENOMEM;
  }
}

int pkv_seq_append_slot(pkv_alloc *a, int64_t seq_id, int64_t *slot, int32_t *cow_src,
                        int32_t *cow_dst) {
  if (!a || !slot) return PKV_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ENOENT;
  if (it->second.on_host) return PKV_EINVAL;
  const int32_t pos = it->second.len;
  if (pos == INT32_MAX) return PKV_EINVAL;
  int st;
  try {
    st = grow(a, seq_id, pos + 1, false, cow_src, cow_dst);
  } catch (...) {
    return PKV_ENOMEM;
  }
  if (st != PKV_OK) return st;
  const pkv_seq &s = a->seqs.find(seq_id)->second;
  *slot = (int64_t)s.blocks[pos / a->block_size] * a->block_size + pos % a->block_size;
  return PKV_OK;
}

int pkv_seq_append_slots(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int64_t *slots,
                         int32_t *cow_pairs, int32_t *num_cow, int32_t *cow_src,
                         int32_t *num_done) {
  if (num_done) *num_done = 0;
  if (num_cow) *num_cow = 0;
  if (!a || n < 0 || (n > 0 && (!seq_ids || !slots || !cow_pairs || !num_cow)))
    return PKV_EINVAL;
  const int chk = check_append_batch(a, seq_ids, n, 0);
  if (chk != PKV_OK) return chk;
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    const int st = pkv_seq_append_slot(a, seq_ids[i], &slots[i], &src, &dst);
    if (st != PKV_OK) return st;   // not reached: the batch was checked above
    if (cow_src) cow_src[i] = src;
    if (src >= 0) {
      cow_pairs[2 * ncow] = src;
      cow_pairs[2 * ncow + 1] = dst;
      ++ncow;
      *num_cow = ncow;
    }
    if (num_done) *num_done = i + 1;
  }
  return PKV_OK;
}

int pkv_seq_step(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int32_t max_blocks_per_seq,
                 int64_t *slots, int32_t *cow_src, int32_t *out_block_tables,
                 int32_t *out_seq_lens) {
  if (!a || n < 0 || max_blocks_per_seq <= 0 ||
      (n > 0 && (!seq_ids || !cow_src || !out_block_tables || !out_seq_lens)))
    return PKV_EINVAL;
  const int chk = check_append_batch(a, seq_ids, n, max_blocks_per_seq);
  if (chk != PKV_OK) return chk;
  for (int32_t i = 0; i < n; ++i) {
    int64_t slot;
    int32_t dst;
    const int st = pkv_seq_append_slot(a, seq_ids[i], &slot, &cow_src[i], &dst);
    if (st != PKV_OK) return st;   // not reached: the batch was checked above
    if (slots) slots[i] = slot;
  }
  return pkv_export_tables(a, seq_ids, n, max_blocks_per_seq, out_block_tables, out_seq_lens);
}

int pkv_seq_fork(pkv_alloc *a, int64_t parent, int64_t child) {
  if (!a) return PKV_EINVAL;
  auto p = a->seqs.find(parent);
  if (p == a->seqs.end()) return PKV_ENOENT;
  if (a->seqs.count(child)) return PKV_EEXIST;
  if (p->second.on_host) return PKV_EINVAL;
  try {
    pkv_seq copy = p->second;
    for (int32_t b : copy.blocks) a->addref(b);
    a->seqs.emplace(child, std::move(copy));
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

int pkv_seq_free(pkv_alloc *a, int64_t seq_id) {
  if (!a) return PKV_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ENOENT;
  if (it->second.on_host) {
    for (int32_t c : it->second.blocks)
      if (--a->host_ref[c] == 0) a->host_free.push_back(c);
  } else {
    for (int32_t b : it->second.blocks) a->unref(b);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_seq_len(const pkv_alloc *a, int64_t seq_id, int32_t *len) {
  if (!a || !len) return PKV_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ENOENT;
  *len = it->second.len;
  return PKV_OK;
}

int pkv_seq_slots(const pkv_alloc *a, int64_t seq_id, int32_t start, int32_t count,
                  int64_t *out_slots) {
  if (!a || start < 0 || count < 0 || (count > 0 && !out_slots)) return PKV_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ENOENT;
  const pkv_seq &s = it->second;
  if (s.on_host || (int64_t)start + count > s.len) return PKV_EINVAL;
  const int32_t bs = a->block_size;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t p = start + i;
    out_slots[i] = (int64_t)s.blocks[p / bs] * bs + p % bs;
  }
  return PKV_OK;
}

int pkv_export_tables(const pkv_alloc *a, const int64_t *seq_ids, int32_t n,
                      int32_t max_blocks_per_seq, int32_t *out_block_tables,
                      int32_t *out_seq_lens) {
  if (!a || n < 0 || max_blocks_per_seq <= 0 ||
      (n > 0 && (!seq_ids || !out_block_tables || !out_seq_lens)))
    return PKV_EINVAL;
  for (int32_t i = 0; i < n; ++i) {  // validate everything before writing
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ENOENT;
    if (it->second.on_host) return PKV_EINVAL;
    if ((int32_t)it->second.blocks.size() > max_blocks_per_seq) return PKV_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_seq &s = a->seqs.find(seq_ids[i])->second;
    int32_t *row = out_block_tables + (size_t)i * max_blocks_per_seq;
    const int32_t nb = (int32_t)s.blocks.size();
    if (nb) std::memcpy(row, s.blocks.data(), sizeof(int32_t) * nb);
    for (int32_t j = nb; j < max_blocks_per_seq; ++j) row[j] = -1;
    out_seq_lens[i] = s.len;
  }
  return PKV_OK;
}

int pkv_export_shared_tables(const pkv_alloc *a, const int64_t *seq_ids, int32_t n,
                             int32_t min_prefix_tokens, int32_t max_prefix_blocks,
                             int32_t max_suffix_blocks, int32_t *suffix_tables,
                             int32_t *suffix_lens, int32_t *seq_group, int32_t *group_offsets,
                             int32_t *group_members, int32_t *group_tables,
                             int32_t *group_prefix_lens, int32_t *num_groups,
                             int32_t *max_group_size) {
  if (!a || n < 0 || min_prefix_tokens < 0 || max_prefix_blocks <= 0 || max_suffix_blocks <= 0 ||
      !num_groups || !max_group_size || !group_offsets)
    return PKV_EINVAL;
  if (n > 0 && (!seq_ids || !suffix_tables || !suffix_lens || !seq_group || !group_members ||
                !group_tables || !group_prefix_lens))
    return PKV_EINVAL;
  std::vector<const pkv_seq *> sq(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ENOENT;
    if (it->second.on_host) return PKV_EINVAL;
    sq[i] = &it->second;
  }
  const int32_t bs = a->block_size;
  // a prefix is whole 16-token tiles: an even number of 8-token blocks
  const int32_t step = bs < 16 ? 16 / bs : 1;
  const int64_t min_tokens = min_prefix_tokens > 16 ? min_prefix_tokens : 16;

  // candidate groups: sequences whose first block is the same physical block,
  // numbered in order of their first member
  std::unordered_map<int32_t, int32_t> by_first;
  std::vector<std::vector<int32_t>> cand;
  for (int32_t i = 0; i < n; ++i) {
    if (sq[i]->blocks.empty()) continue;
    auto ins = by_first.emplace(sq[i]->blocks[0], (int32_t)cand.size());
    if (ins.second) cand.emplace_back();
    cand[ins.first->second].push_back(i);
  }
  std::vector<int32_t> grp_of(n, -1), pre_blocks(n, 0);
  std::vector<int32_t> kept, kept_blocks;
  for (size_t c = 0; c < cand.size(); ++c) {
    const std::vector<int32_t> &mem = cand[c];
    if (mem.size() < 2) continue;
    // longest common run of leading entries, limited to blocks every member
    // has filled
    int64_t k = max_prefix_blocks;
    for (int32_t i : mem) {
      const int64_t filled = sq[i]->len / bs;
      if (filled < k) k = filled;
    }
    const std::vector<int32_t> &t0 = sq[mem[0]]->blocks;
    int64_t common = 0;
    while (common < k) {
      bool same = true;
      for (int32_t i : mem)
        if (sq[i]->blocks[common] != t0[common]) { same = false; break; }
      if (!same) break;
      ++common;
    }
    common -= common % step;
    if (common * bs < min_tokens) continue;
    for (int32_t i : mem) {
      grp_of[i] = (int32_t)kept.size();
      pre_blocks[i] = (int32_t)common;
    }
    kept.push_back((int32_t)c);
    kept_blocks.push_back((int32_t)common);
  }
  for (int32_t i = 0; i < n; ++i)
    if ((int64_t)sq[i]->blocks.size() - pre_blocks[i] > max_suffix_blocks) return PKV_EINVAL;

  // outputs
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t> &t = sq[i]->blocks;
    int32_t *row = suffix_tables + (size_t)i * max_suffix_blocks;
    const int32_t ns = (int32_t)t.size() - pre_blocks[i];
    for (int32_t j = 0; j < max_suffix_blocks; ++j) row[j] = j < ns ? t[pre_blocks[i] + j] : -1;
    suffix_lens[i] = sq[i]->len - pre_blocks[i] * bs;
    seq_group[i] = grp_of[i];
  }
  int32_t pos = 0, biggest = 0;
  for (size_t g = 0; g < kept.size(); ++g) {
    const std::vector<int32_t> &mem = cand[kept[g]];
    group_offsets[g] = pos;
    for (int32_t i : mem) group_members[pos++] = i;
    if ((int32_t)mem.size() > biggest) biggest = (int32_t)mem.size();
    const std::vector<int32_t> &t0 = sq[mem[0]]->blocks;
    int32_t *row = group_tables + g * (size_t)max_prefix_blocks;
    for (int32_t j = 0; j < max_prefix_blocks; ++j) row[j] = j < kept_blocks[g] ? t0[j] : -1;
    group_prefix_lens[g] = kept_blocks[g] * bs;
  }
  group_offsets[kept.size()] = pos;
  *num_groups = (int32_t)kept.size();
  *max_group_size = biggest;
  return PKV_OK;
}

// ---- host pool and swapping -------------------------------------------------

int pkv_alloc_set_host_blocks(pkv_alloc *a, int32_t num_host_blocks) {
  if (!a || num_host_blocks < 0) return PKV_EINVAL;
  for (const auto &kv : a->seqs)
    if (kv.second.on_host) return PKV_EINVAL;
  try {
    a->num_host = num_host_blocks;
    a->host_free.clear();
    for (int32_t i = 0; i < num_host_blocks; ++i) a->host_free.push_back(i);
    a->host_ref.assign(num_host_blocks, 0);
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

int32_t pkv_alloc_num_free_host(const pkv_alloc *a) {
  return a ? (int32_t)a->host_free.size() : PKV_EINVAL;
}

int32_t pkv_alloc_free_list_host(const pkv_alloc *a, int32_t *out, int32_t cap) {
  if (!a || (cap > 0 && !out)) return PKV_EINVAL;
  int32_t i = 0;
  for (int32_t c : a->host_free) {
    if (i >= cap) break;
    out[i++] = c;
  }
  return (int32_t)a->host_free.size();
}

int32_t pkv_host_block_refcount(const pkv_alloc *a, int32_t block) {
  if (!a || block < 0 || block >= a->num_host) return PKV_EINVAL;
  return a->host_ref[block];
}

int pkv_seq_on_host(const pkv_alloc *a, int64_t seq_id, int32_t *on_host) {
  if (!a || !on_host) return PKV_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ENOENT;
  *on_host = it->second.on_host ? 1 : 0;
  return PKV_OK;
}

namespace {

// The sequences of a swap call: known, all on the same side, no repeats.
int collect(pkv_alloc *a, const int64_t *seq_ids, int32_t n, bool on_host,
            std::vector<pkv_seq *> *out) {
  std::unordered_set<int64_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ENOENT;
    if (it->second.on_host != on_host || !seen.insert(seq_ids[i]).second) return PKV_EINVAL;
    out->push_back(&it->second);
  }
  return PKV_OK;
}

// Distinct blocks of the sequences' tables in order of first appearance, and
// how many of those table entries point at each.
void distinct_blocks(const std::vector<pkv_seq *> &sq, std::vector<int32_t> *order,
                     std::unordered_map<int32_t, int32_t> *count) {
  for (const pkv_seq *q : sq)
    for (int32_t b : q->blocks)
      if ((*count)[b]++ == 0) order->push_back(b);
}

}  // namespace

int pkv_seq_swap_out(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int32_t *pairs,
                     int32_t cap, int32_t *num_pairs) {
  if (num_pairs) *num_pairs = 0;
  if (!a || n < 0 || !num_pairs || (n > 0 && !seq_ids) || cap < 0 || (cap > 0 && !pairs))
    return PKV_EINVAL;
  try {
    std::vector<pkv_seq *> sq;
    const int st = collect(a, seq_ids, n, false, &sq);
    if (st != PKV_OK) return st;
    std::vector<int32_t> order;
    std::unordered_map<int32_t, int32_t> cnt;
    distinct_blocks(sq, &order, &cnt);
    if ((int64_t)order.size() > cap) return PKV_EINVAL;
    if (order.size() > a->host_free.size()) return PKV_ENOMEM;
    std::unordered_map<int32_t, int32_t> to_host;
    for (size_t i = 0; i < order.size(); ++i) {
      const int32_t b = order[i], c = a->host_free.front();
      a->host_free.pop_front();
      a->host_ref[c] = cnt[b];
      to_host[b] = c;
      pairs[2 * i] = b;
      pairs[2 * i + 1] = c;
    }
    for (int32_t b : order) a->unref(b, cnt[b]);
    for (pkv_seq *q : sq) {
      for (int32_t &b : q->blocks) b = to_host[b];
      q->on_host = true;
    }
    *num_pairs = (int32_t)order.size();
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

int pkv_seq_swap_in(pkv_alloc *a, const int64_t *seq_ids, int32_t n, int32_t *pairs,
                    int32_t cap, int32_t *num_pairs) {
  if (num_pairs) *num_pairs = 0;
  if (!a || n < 0 || !num_pairs || (n > 0 && !seq_ids) || cap < 0 || (cap > 0 && !pairs))
    return PKV_EINVAL;
  try {
    std::vector<pkv_seq *> sq;
    const int st = collect(a, seq_ids, n, true, &sq);
    if (st != PKV_OK) return st;
    std::vector<int32_t> order;
    std::unordered_map<int32_t, int32_t> cnt;
    distinct_blocks(sq, &order, &cnt);
    if ((int64_t)order.size() > cap) return PKV_EINVAL;
    if (!a->make_room((int32_t)order.size())) return PKV_ENOMEM;
    std::unordered_map<int32_t, int32_t> to_dev;
    for (size_t i = 0; i < order.size(); ++i) {
      const int32_t c = order[i], b = a->pop_front();
      a->ref[b] = cnt[c];
      to_dev[c] = b;
      pairs[2 * i] = c;
      pairs[2 * i + 1] = b;
    }
    for (int32_t c : order) {
      a->host_ref[c] -= cnt[c];
      if (a->host_ref[c] == 0) a->host_free.push_back(c);
    }
    for (pkv_seq *q : sq) {
      for (int32_t &c : q->blocks) c = to_dev[c];
      q->on_host = false;
    }
    *num_pairs = (int32_t)order.size();
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

// ---- automatic prefix caching -------------------------------------------------

namespace {

// Hash of the token prefix through one more block, chained from the previous
// block's (0 before the first): a 64-bit multiply-xorshift mix per token.
uint64_t chain_hash(uint64_t h, const int32_t *tok, int32_t n) {
  h ^= 0x9E3779B97F4A7C15ull;
  for (int32_t i = 0; i < n; ++i) {
    h ^= (uint32_t)tok[i];
    h *= 0xBF58476D1CE4E5B9ull;
    h ^= h >> 31;
  }
  return h;
}

// The cached block whose prefix key is h, preceded by the prefix with key
// hprev, holding tokens tok; or -1.
int32_t lookup(const pkv_alloc *a, uint64_t h, const int32_t *tok, uint64_t hprev) {
  auto it = a->by_hash.find(h);
  if (it == a->by_hash.end()) return -1;
  const int32_t b = it->second;
  if (a->parent_key[b] != hprev) return -1;
  const std::vector<int32_t> &t = a->block_tokens[b];
  if (std::memcmp(t.data(), tok, sizeof(int32_t) * a->block_size) != 0) return -1;
  return b;
}

}  // namespace

int pkv_seq_allocate_cached(pkv_alloc *a, int64_t seq_id, const int32_t *tokens, int32_t n,
                            int32_t *num_cached_tokens) {
  if (num_cached_tokens) *num_cached_tokens = 0;
  if (!a || n < 0 || (n > 0 && !tokens) || !num_cached_tokens) return PKV_EINVAL;
  if (a->seqs.count(seq_id)) return PKV_EEXIST;
  try {
    const int32_t bs = a->block_size;
    std::vector<int32_t> hit;
    uint64_t h = 0;
    for (int32_t i = 0; (int64_t)(i + 1) * bs <= n; ++i) {
      const uint64_t hp = h;
      h = chain_hash(h, tokens + (size_t)i * bs, bs);
      const int32_t b = lookup(a, h, tokens + (size_t)i * bs, hp);
      if (b < 0) break;
      hit.push_back(b);
    }
    const int32_t need = a->blocks_for(n) - (int32_t)hit.size();
    // capacity: the free list plus the evictable blocks other than the hits
    int32_t hit_evictable = 0;
    for (int32_t b : hit) hit_evictable += a->in_lru[b] ? 1 : 0;
    if ((int64_t)a->count + (int64_t)a->lru.size() - hit_evictable < need) return PKV_ENOMEM;
    pkv_seq s;
    s.blocks.reserve(a->blocks_for(n));
    for (int32_t b : hit) {
      a->addref(b);
      s.blocks.push_back(b);
    }
    a->make_room(need);
    for (int32_t i = 0; i < need; ++i) {
      const int32_t b = a->pop_front();
      a->ref[b] = 1;
      s.blocks.push_back(b);
    }
    s.len = n;
    a->seqs.emplace(seq_id, std::move(s));
    *num_cached_tokens = (int32_t)hit.size() * bs;
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

int pkv_seq_cache_blocks(pkv_alloc *a, int64_t seq_id, const int32_t *tokens, int32_t n) {
  if (!a || n < 0 || (n > 0 && !tokens)) return PKV_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ENOENT;
  pkv_seq &s = it->second;
  if (s.on_host || n > s.len) return PKV_EINVAL;
  try {
    const int32_t bs = a->block_size;
    uint64_t h = 0;
    for (int32_t i = 0; (int64_t)(i + 1) * bs <= n; ++i) {
      const int32_t *tok = tokens + (size_t)i * bs;
      const uint64_t hp = h;
      h = chain_hash(h, tok, bs);
      if (lookup(a, h, tok, hp) >= 0) continue;   // this prefix is cached already
      if (a->by_hash.count(h)) break;             // a different prefix holds this hash
      const int32_t b = s.blocks[i];
      if (a->cached[b]) break;                    // cached under another prefix
      a->by_hash[h] = b;
      a->cached[b] = 1;
      a->key[b] = h;
      a->parent_key[b] = hp;
      a->block_tokens[b].assign(tok, tok + bs);
      a->addref(b);                               // the cache's reference
    }
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

int pkv_prefix_cache_evict(pkv_alloc *a, int32_t max_blocks, int32_t *num_evicted) {
  if (num_evicted) *num_evicted = 0;
  if (!a || max_blocks < 0) return PKV_EINVAL;
  int32_t k = 0;
  while (k < max_blocks && !a->lru.empty()) {
    a->evict_one();
    ++k;
  }
  if (num_evicted) *num_evicted = k;
  return PKV_OK;
}

int32_t pkv_prefix_cache_size(const pkv_alloc *a) {
  return a ? (int32_t)a->by_hash.size() : PKV_EINVAL;
}

int32_t pkv_prefix_cache_evictable(const pkv_alloc *a, int32_t *out, int32_t cap) {
  if (!a || (cap > 0 && !out)) return PKV_EINVAL;
  int32_t i = 0;
  for (int32_t b : a->lru) {
    if (i >= cap) break;
    out[i++] = b;
  }
  return (int32_t)a->lru.size();
}

}  // extern "C"
