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
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_seq {
  std::vector<int32_t> blocks;
  int32_t len = 0;
};

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::vector<int32_t> ring;   // free list storage
  int32_t head = 0;            // index of the first free entry
  int32_t count = 0;           // number of free blocks
  std::vector<int32_t> ref;    // table entries pointing at each block
  std::unordered_map<int64_t, pkv_seq> seqs;

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
  if (a->count < need + (cow ? 1 : 0)) return PKV_ENOMEM;
  if (it == a->seqs.end()) it = a->seqs.emplace(seq_id, pkv_seq{}).first;
  pkv_seq &s = it->second;
  s.blocks.reserve((size_t)held + need);
  if (cow) {
    const int32_t src = s.blocks.back();
    const int32_t dst = a->pop_front();
    a->ref[dst] = 1;
    a->ref[src] -= 1;
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
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    const int st = pkv_seq_append_slot(a, seq_ids[i], &slots[i], &src, &dst);
    if (st != PKV_OK) return st;
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

int pkv_seq_fork(pkv_alloc *a, int64_t parent, int64_t child) {
  if (!a) return PKV_EINVAL;
  auto p = a->seqs.find(parent);
  if (p == a->seqs.end()) return PKV_ENOENT;
  if (a->seqs.count(child)) return PKV_EEXIST;
  try {
    pkv_seq copy = p->second;
    for (int32_t b : copy.blocks) a->ref[b] += 1;
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
  for (int32_t b : it->second.blocks) {
    if (--a->ref[b] == 0) a->push_back(b);
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
  if ((int64_t)start + count > s.len) return PKV_EINVAL;
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

}  // extern "C"
