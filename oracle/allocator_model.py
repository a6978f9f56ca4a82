"""Block allocator model -- TEST INFRASTRUCTURE ONLY (part of the oracle).

A plain Python model of the KV block manager, written from the pages:

* fixed 16-token blocks, allocated on demand and returned to a free pool when
  a request ends ("KV Cache and PagedAttention (vllm-musa)", 7yue.com, section 2);
* the number of blocks for n tokens is ceil(n / block_size), and allocation
  checks capacity before it takes anything, so an out-of-memory request
  changes nothing; blocks are taken from the head of the free list and freed
  blocks go to its tail ("vLLM PagedAttention deep dive", jsqmd.com, section 3.2);
* requests may share physical blocks; before a request writes into a shared
  block it copies the block, writes into the copy and repoints its own table,
  while the others keep the original ("KVcache-learning", fairy2021.github.io,
  chapter s05, copy-on-write; chapter s06 lists alloc / cow / free).

Reference counts (how many table entries point at a block) are this model's
reading of "shared": a block returns to the free list when its count reaches
zero.  Statuses are strings ("ok", "enomem", "enoent", "eexist", "einval").
"""
from __future__ import annotations

from collections import deque


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks))
        self.free = deque(order)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.ref = [0] * num_blocks

    def _blocks_for(self, n: int) -> int:
        return -(-n // self.block_size)

    def allocate(self, seq: int, n_tokens: int):
        """Grow seq (created if new) to n_tokens filled tokens.
        Returns (status, cow_pair or None)."""
        if n_tokens < 0:
            return "einval", None
        table = self.tables.get(seq, [])
        cur = self.lens.get(seq, 0)
        if n_tokens <= cur:
            self.tables.setdefault(seq, table)
            self.lens.setdefault(seq, cur)
            return "ok", None
        new_blocks = max(0, self._blocks_for(n_tokens) - len(table))
        # the partly filled tail block receives new tokens: copy it first if shared
        cow = cur % self.block_size != 0 and self.ref[table[-1]] > 1
        if len(self.free) < new_blocks + (1 if cow else 0):
            return "enomem", None
        pair = None
        if cow:
            src = table[-1]
            dst = self.free.popleft()
            self.ref[dst] = 1
            self.ref[src] -= 1
            table = table[:-1] + [dst]
            pair = (src, dst)
        for _ in range(new_blocks):
            b = self.free.popleft()
            self.ref[b] = 1
            table = table + [b]
        self.tables[seq] = table
        self.lens[seq] = n_tokens
        return "ok", pair

    def append(self, seq: int):
        """Reserve the next token's slot.  Returns (status, slot, cow_pair or None)."""
        if seq not in self.tables:
            return "enoent", -1, None
        pos = self.lens[seq]
        st, pair = self.allocate(seq, pos + 1)
        if st != "ok":
            return st, -1, None
        b = self.tables[seq][pos // self.block_size]
        return "ok", b * self.block_size + pos % self.block_size, pair

    def fork(self, parent: int, child: int) -> str:
        if parent not in self.tables:
            return "enoent"
        if child in self.tables:
            return "eexist"
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return "ok"

    def release(self, seq: int) -> str:
        if seq not in self.tables:
            return "enoent"
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]
        return "ok"

    def slots(self, seq: int, start: int, count: int):
        """Slots (block * block_size + offset) of positions [start, start + count)."""
        if seq not in self.tables:
            return "enoent", None
        if start < 0 or count < 0 or start + count > self.lens[seq]:
            return "einval", None
        t = self.tables[seq]
        bs = self.block_size
        return "ok", [t[p // bs] * bs + p % bs for p in range(start, start + count)]

    def export(self, seqs, max_blocks: int):
        """Block-table rows padded with -1, and seq lens."""
        rows, lens = [], []
        for s in seqs:
            if s not in self.tables:
                return "enoent", None, None
            t = self.tables[s]
            if len(t) > max_blocks:
                return "einval", None, None
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return "ok", rows, lens

    def export_shared(self, seqs, min_prefix_tokens: int, max_prefix_blocks: int,
                      max_suffix_blocks: int):
        """Tables split into shared prefixes and private suffixes.

        Sequences forked from one parent share the physical blocks of their
        common beginning (s05 copy-on-write and s08 of "KVcache-learning").  A
        group is every sequence (two or more) whose first table entry is the
        same physical block, taken in the order of its first member; its prefix
        is the longest run of leading entries all members have in common,
        limited to blocks every member has filled, to max_prefix_blocks and to
        whole 16-token tiles.  Groups whose prefix is shorter than
        max(16, min_prefix_tokens) tokens are not formed.  Returns status and a
        dict of the host arrays the C call fills.
        """
        for s in seqs:
            if s not in self.tables:
                return "enoent", None
        bs = self.block_size
        firsts = {}
        for i, s in enumerate(seqs):
            if self.tables[s]:
                firsts.setdefault(self.tables[s][0], []).append(i)
        groups = []
        for members in sorted(firsts.values(), key=lambda mem: mem[0]):
            if len(members) < 2:
                continue
            tabs = [self.tables[seqs[i]] for i in members]
            limit = min([max_prefix_blocks] + [self.lens[seqs[i]] // bs for i in members])
            k = 0
            while k < limit and all(t[k] == tabs[0][k] for t in tabs):
                k += 1
            while (k * bs) % 16:
                k -= 1
            if k * bs >= max(16, min_prefix_tokens):
                groups.append((members, k))
        n = len(seqs)
        seq_group, pre = [-1] * n, [0] * n
        for gi, (members, k) in enumerate(groups):
            for i in members:
                seq_group[i], pre[i] = gi, k
        suffix_tables, suffix_lens = [], []
        for i, s in enumerate(seqs):
            rest = self.tables[s][pre[i]:]
            if len(rest) > max_suffix_blocks:
                return "einval", None
            suffix_tables.append(rest + [-1] * (max_suffix_blocks - len(rest)))
            suffix_lens.append(self.lens[s] - pre[i] * bs)
        offsets, members_flat, group_tables, prefix_lens = [0], [], [], []
        for members, k in groups:
            members_flat += members
            offsets.append(len(members_flat))
            head = self.tables[seqs[members[0]]][:k]
            group_tables.append(head + [-1] * (max_prefix_blocks - k))
            prefix_lens.append(k * bs)
        return "ok", dict(suffix_tables=suffix_tables, suffix_lens=suffix_lens,
                          seq_group=seq_group, group_offsets=offsets,
                          group_members=members_flat, group_tables=group_tables,
                          group_prefix_lens=prefix_lens, num_groups=len(groups),
                          max_group_size=max([len(m) for m, _ in groups], default=0))

    # invariants ---------------------------------------------------------------
    def check_invariants(self):
        counts = [0] * self.num_blocks
        for seq, t in self.tables.items():
            assert len(t) == self._blocks_for(self.lens[seq]), "table length != ceil(len/bs)"
            assert len(t) * self.block_size - self.lens[seq] < self.block_size, "tail waste"
            for b in t:
                counts[b] += 1
        assert counts == self.ref, "refcount != number of table entries"
        free = set(self.free)
        assert len(free) == len(self.free), "duplicate free block"
        for b in range(self.num_blocks):
            assert (b in free) == (self.ref[b] == 0), "free iff unreferenced"
        assert sum(1 for r in self.ref if r > 0) + len(self.free) == self.num_blocks
