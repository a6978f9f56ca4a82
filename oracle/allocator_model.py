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

Swapping ("swap_out(blocks, cpu_blocks) / swap_in(blocks, gpu_blocks)" of the
Block Manager, KVcache-learning s06; KV moved to CPU memory under
preemption, yunthe.com): a host pool with its own FIFO free list; a set of
sequences moves as a whole, blocks they share staying shared.

Automatic prefix caching (KVcache-learning s08; jsqmd.com section 4.2): a full
block is indexed by the token prefix through it (this model keys by the exact
token tuple); the cache holds a reference; blocks only the cache holds are
evicted least recently released first when an allocation finds the free list
short.
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
        self.on_host: set[int] = set()
        self.host_free: deque = deque()
        self.host_ref: list[int] = []
        self.cache: dict[tuple, int] = {}      # token prefix -> cached block
        self.cached_as: dict[int, tuple] = {}  # cached block -> its prefix
        self.lru: list[int] = []               # blocks only the cache holds, oldest first

    # references ---------------------------------------------------------------
    def _drop(self, b: int, k: int = 1):
        self.ref[b] -= k
        if self.ref[b] == 0:
            self.free.append(b)
        elif self.ref[b] == 1 and b in self.cached_as and b not in self.lru:
            self.lru.append(b)

    def _take(self, b: int):
        self.ref[b] += 1
        if b in self.lru:
            self.lru.remove(b)

    def _room(self, need: int) -> bool:
        """Evict cache-only blocks (oldest release first) until `need` are free."""
        if len(self.free) + len(self.lru) < need:
            return False
        while len(self.free) < need:
            b = self.lru.pop(0)
            del self.cache[self.cached_as.pop(b)]
            self._drop(b)
        return True

    def _blocks_for(self, n: int) -> int:
        return -(-n // self.block_size)

    def allocate(self, seq: int, n_tokens: int):
        """Grow seq (created if new) to n_tokens filled tokens.
        Returns (status, cow_pair or None)."""
        if n_tokens < 0 or seq in self.on_host:
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
        if not self._room(new_blocks + (1 if cow else 0)):
            return "enomem", None
        pair = None
        if cow:
            src = table[-1]
            dst = self.free.popleft()
            self.ref[dst] = 1
            self._drop(src)
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
        if seq in self.on_host:
            return "einval", -1, None
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
        if parent in self.on_host:
            return "einval"
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self._take(b)
        return "ok"

    def release(self, seq: int) -> str:
        if seq not in self.tables:
            return "enoent"
        if seq in self.on_host:
            for c in self.tables.pop(seq):
                self.host_ref[c] -= 1
                if self.host_ref[c] == 0:
                    self.host_free.append(c)
            self.on_host.discard(seq)
        else:
            for b in self.tables.pop(seq):
                self._drop(b)
        del self.lens[seq]
        return "ok"

    # swapping ----------------------------------------------------------------------
    def set_host_blocks(self, n: int) -> str:
        if self.on_host or n < 0:
            return "einval"
        self.host_free = deque(range(n))
        self.host_ref = [0] * n
        return "ok"

    def _group(self, seqs, on_host: bool):
        if len(set(seqs)) != len(seqs):
            return "einval", None, None
        for s in seqs:
            if s not in self.tables:
                return "enoent", None, None
            if (s in self.on_host) != on_host:
                return "einval", None, None
        order, count = [], {}
        for s in seqs:
            for b in self.tables[s]:
                if b not in count:
                    order.append(b)
                    count[b] = 0
                count[b] += 1
        return "ok", order, count

    def swap_out(self, seqs):
        """Move a set of device sequences to the host pool.  Returns (status,
        [(device, host), ...])."""
        st, order, count = self._group(seqs, False)
        if st != "ok":
            return st, None
        if len(self.host_free) < len(order):
            return "enomem", None
        pairs = [(b, self.host_free.popleft()) for b in order]
        where = dict(pairs)
        for b, c in pairs:
            self.host_ref[c] = count[b]
        for b in order:
            self._drop(b, count[b])
        for s in seqs:
            self.tables[s] = [where[b] for b in self.tables[s]]
            self.on_host.add(s)
        return "ok", pairs

    def swap_in(self, seqs):
        """Bring a set of swapped-out sequences back.  Returns (status,
        [(host, device), ...])."""
        st, order, count = self._group(seqs, True)
        if st != "ok":
            return st, None
        if not self._room(len(order)):
            return "enomem", None
        pairs = [(c, self.free.popleft()) for c in order]
        where = dict(pairs)
        for c, b in pairs:
            self.ref[b] = count[c]
        for c in order:
            self.host_ref[c] -= count[c]
            if self.host_ref[c] == 0:
                self.host_free.append(c)
        for s in seqs:
            self.tables[s] = [where[c] for c in self.tables[s]]
            self.on_host.discard(s)
        return "ok", pairs

    # automatic prefix caching ------------------------------------------------------
    def allocate_cached(self, seq: int, tokens):
        """New sequence for a prompt: the longest run of leading full blocks
        whose prefixes are cached is shared.  Returns (status, cached tokens)."""
        if seq in self.tables:
            return "eexist", 0
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        hits = []
        while (len(hits) + 1) * bs <= len(tokens):
            key = tuple(tokens[:(len(hits) + 1) * bs])
            if key not in self.cache:
                break
            hits.append(self.cache[key])
        need = self._blocks_for(len(tokens)) - len(hits)
        if len(self.free) + len([b for b in self.lru if b not in hits]) < need:
            return "enomem", 0
        for b in hits:
            self._take(b)
        self._room(need)
        table = list(hits)
        for _ in range(need):
            b = self.free.popleft()
            self.ref[b] = 1
            table.append(b)
        self.tables[seq] = table
        self.lens[seq] = len(tokens)
        return "ok", len(hits) * bs

    def cache_blocks(self, seq: int, tokens, n: int) -> str:
        """Index the full blocks of the first n tokens of seq by their prefixes."""
        if seq not in self.tables:
            return "enoent"
        if seq in self.on_host or n > self.lens[seq] or n < 0:
            return "einval"
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        for i in range(n // bs):
            key = tuple(tokens[:(i + 1) * bs])
            if key in self.cache:
                continue
            b = self.tables[seq][i]
            if b in self.cached_as:
                break
            self.cache[key] = b
            self.cached_as[b] = key
            self._take(b)
        return "ok"

    def cache_evict(self, max_blocks: int):
        k = 0
        while k < max_blocks and self.lru:
            b = self.lru.pop(0)
            del self.cache[self.cached_as.pop(b)]
            self._drop(b)
            k += 1
        return "ok", k

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
            if s in self.on_host:
                return "einval", None, None
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
            if s in self.on_host:
                return "einval", None
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
        hcounts = [0] * len(self.host_ref)
        for seq, t in self.tables.items():
            assert len(t) == self._blocks_for(self.lens[seq]), "table length != ceil(len/bs)"
            assert len(t) * self.block_size - self.lens[seq] < self.block_size, "tail waste"
            for b in t:
                if seq in self.on_host:
                    hcounts[b] += 1
                else:
                    counts[b] += 1
        for b in self.cached_as:
            counts[b] += 1                       # the cache's reference
        assert counts == self.ref, "refcount != table entries + cache"
        assert hcounts == self.host_ref, "host refcount != host table entries"
        assert set(self.lru) == {b for b in self.cached_as if self.ref[b] == 1}, "evictable set"
        assert len(self.lru) == len(set(self.lru))
        assert set(self.host_free) == {c for c, r in enumerate(self.host_ref) if r == 0}
        free = set(self.free)
        assert len(free) == len(self.free), "duplicate free block"
        for b in range(self.num_blocks):
            assert (b in free) == (self.ref[b] == 0), "free iff unreferenced"
        assert sum(1 for r in self.ref if r > 0) + len(self.free) == self.num_blocks
