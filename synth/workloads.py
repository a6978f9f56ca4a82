"""Workload descriptions: the five decode configurations and small variants.

A workload is a recipe, not a result.  It lists

* the shapes and dtypes of one decode batch,
* the allocator's initial free-list order (a seeded permutation of the pool),
* an op script for the block allocator (allocate / fork / free / append) with
  the K/V writes interleaved, and
* generators for the raw q, K and V values (N(0,1), rounded to the stored
  dtype).

Both the oracle and the HIP path replay the same script with their own
allocator and write code; tests check that the two replays agree.

Op script entries:
  ("allocate", seq, n_tokens)   reserve room for n_tokens (prefill) and mark them filled
  ("fork", parent, child)       child shares every block of parent
  ("free", seq)                 release seq
  ("append", seq)               reserve the slot of the next token (may copy-on-write)
  ("write", seq, start, count)  write K/V of token positions [start, start+count) of seq
                                through that seq's slots; the values are keyed by
                                (content owner, position), see `kv_rows`.
The decode batch is `decode_seqs`; ops after the marker ("step",) form the
measured decode step (C5).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import normal, permutation, randint, stream_key, uniform01

NP_DTYPE = {"f32": np.float32, "f16": np.float16}
SEED_BASE = 387 * 1000


@dataclass
class Workload:
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str            # 'f32' | 'f16'
    src_dtype: str          # dtype of new K/V handed to the cache write: 'f32' | 'f16'
    cache_dtype: str        # 'f32' | 'f16' | 'i8' | 'e4m3'
    out_dtype: str          # 'f32' | 'f16'
    scale: float
    num_blocks: int
    free_order: np.ndarray
    ops: list
    decode_seqs: list
    max_blocks_per_seq: int
    seed: int
    block_size: int = 16
    partition_size: int = 0           # 0: library default
    content_owner: dict = field(default_factory=dict)  # seq -> list of (pos_lo, pos_hi, owner)
    description: str = ""
    memo: dict | None = None          # set to {} to keep generated K/V rows for reuse
    q_lens: list | None = None        # multi-token queries: query tokens per decode sequence
    value_profile: str = "normal"     # K/V value distribution, see PROFILES
    q_scale: float = 1.0              # queries are N(0, q_scale^2): large logits for q_scale >> 1

    @property
    def num_seqs(self) -> int:
        return len(self.decode_seqs)

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    def query(self) -> np.ndarray:
        """q for the decode batch, [num_seqs, num_heads, head_dim]."""
        key = stream_key(self.seed, "q")
        rows = self.num_seqs if self.q_lens is None else int(sum(self.q_lens))
        n = rows * self.num_heads * self.head_dim
        q = normal(key, 0, n).reshape(rows, self.num_heads, self.head_dim) * self.q_scale
        return q.astype(NP_DTYPE[self.q_dtype])

    def q_offsets(self) -> np.ndarray:
        """Multi-token queries: first query row of each decode sequence, and the total."""
        assert self.q_lens is not None
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    def kv_rows(self, which: str, owner: int, start: int, count: int) -> np.ndarray:
        """K ('k') or V ('v') values of positions [start, start+count) owned by `owner`,
        [count, num_kv_heads, head_dim] in the source dtype."""
        mk = (which, owner, start, count)
        if self.memo is not None and mk in self.memo:
            return self.memo[mk]
        key = stream_key(self.seed, "kv", which, owner)
        row = self.num_kv_heads * self.head_dim
        x = normal(key, start * row, count * row).reshape(count, self.num_kv_heads, self.head_dim)
        if self.value_profile != "normal":
            x = _apply_profile(x, self, which, owner, start)
        x = x.astype(NP_DTYPE[self.src_dtype])
        if self.memo is not None:
            self.memo[mk] = x
        return x

    def writes(self):
        """(seq, start, count) of every write in the script, in order."""
        return [(op[1], op[2], op[3]) for op in self.ops if op[0] == "write"]

    def owner_of(self, seq: int, pos: int) -> int:
        """Which seq's stream holds the content of token `pos` of `seq`."""
        for lo, hi, owner in self.content_owner.get(seq, ()):
            if lo <= pos < hi:
                return owner
        return seq


# Value profiles of K/V (the pages name outliers as the weak point of int8 and
# FP8 KV caches: single tokens, or particular positions of some KV heads, with
# a far larger spread than the rest -- "KVcache-learning", s09).  Every draw is
# keyed by (seed, which, owner, position, kv head), so a row's values do not
# depend on how the rows are requested.
#   normal            N(0, 1)
#   row_outliers      about one (token, kv head) row in 24 is scaled by 2^e,
#                     e uniform in [3, 16]; every 97th such row (and the row
#                     of position 5 of every owner, kv head 0) is scaled so
#                     that its largest magnitude is exactly the source
#                     format's limit (65504 for fp16)
#   channel_outliers  in each kv head, 2 dims (chosen per kv head) have
#                     standard deviation 2^e, e uniform in [6, 12]
# Values are clipped to the source format's finite range (fp16: +-65504,
# fp32 sources: +-ROW_MAX_F32).
PROFILES = ("normal", "row_outliers", "channel_outliers")
ROW_MAX_F32 = 4.0e6          # fp32-source limit: its int8 scale 4e6/127 is a finite fp16


def _apply_profile(x: np.ndarray, w: "Workload", which: str, owner: int, start: int):
    count, hkv, d = x.shape
    limit = 65504.0 if w.src_dtype == "f16" else ROW_MAX_F32
    if w.value_profile == "row_outliers":
        key = stream_key(w.seed, "outlier_rows", which, owner)
        u = uniform01(key, 2 * start * hkv, 2 * count * hkv).reshape(count, hkv, 2)
        pos = np.arange(start, start + count)[:, None]
        hit = u[:, :, 0] < 1.0 / 24.0
        e = 3.0 + 13.0 * u[:, :, 1]
        f = np.where(hit, 2.0 ** e, 1.0)
        amax = np.abs(x).max(axis=2)
        full = (hit & ((np.floor(u[:, :, 1] * 1e6).astype(np.int64) % 97) == 0)) | \
            ((pos == 5) & (np.arange(hkv)[None, :] == 0))
        f = np.where(full, limit / np.maximum(amax, 1e-300), f)
        x = x * f[:, :, None]
    elif w.value_profile == "channel_outliers":
        key = stream_key(w.seed, "outlier_channels", which)
        u = uniform01(key, 0, 3 * hkv).reshape(hkv, 3)
        dims = np.stack([np.floor(u[:, 0] * d), np.floor(u[:, 1] * d)], 1).astype(np.int64)
        sd = 2.0 ** (6.0 + 6.0 * u[:, 2])
        x = x.copy()
        for h in range(hkv):
            x[:, h, dims[h]] *= sd[h]
    else:
        raise ValueError(f"unknown value profile {w.value_profile!r}")
    return np.clip(x, -limit, limit)


def with_values(w: "Workload", profile: str = "normal", q_scale: float = 1.0) -> "Workload":
    """The same workload (same script, shapes and seeds) with K/V drawn from
    `profile` and queries scaled by q_scale."""
    import copy
    if profile not in PROFILES:
        raise ValueError(profile)
    w2 = copy.copy(w)
    w2.value_profile = profile
    w2.q_scale = float(q_scale)
    w2.memo = None
    w2.name = f"{w.name}_{profile}_q{q_scale:g}"
    return w2


def _cfg_seed(i: int) -> int:
    return SEED_BASE + i


def _simple(name, seed, lens, H, Hkv, D, q_dt, src_dt, cache_dt, out_dt, num_blocks,
            max_blocks=None, partition_size=0, description=""):
    """Independent sequences 0..S-1: allocate each to its length and write its context."""
    lens = [int(x) for x in lens]
    if max_blocks is None:
        max_blocks = max(1, max(-(-L // 16) for L in lens))
    ops = []
    for s, L in enumerate(lens):
        ops.append(("allocate", s, L))
        if L:
            ops.append(("write", s, 0, L))
    return Workload(
        name=name, num_heads=H, num_kv_heads=Hkv, head_dim=D, q_dtype=q_dt,
        src_dtype=src_dt, cache_dtype=cache_dt, out_dtype=out_dt,
        scale=1.0 / math.sqrt(D), num_blocks=num_blocks,
        free_order=permutation(stream_key(seed, "free_order"), num_blocks),
        ops=ops, decode_seqs=list(range(len(lens))), max_blocks_per_seq=max_blocks,
        seed=seed, partition_size=partition_size, description=description)


def c1_tiny() -> Workload:
    """Tiny fp32 decode: lens {1,17,33,100}, 8/2 heads, d 64, 64-block pool, scale 1/8."""
    w = _simple("c1_tiny", _cfg_seed(1), [1, 17, 33, 100], 8, 2, 64, "f32", "f32", "f32",
                "f32", 64, description="tiny fp32 decode")
    return w


def c2_qwen3_32b_layer(seed_offset: int = 0, num_seqs: int = 32) -> Workload:
    """Qwen3-32B-shaped layer: 32 seqs, lens U[512,768], 64/8 heads, d 128, fp16, 12480 blocks."""
    seed = _cfg_seed(2) + 100 * seed_offset
    lens = randint(stream_key(seed, "lens"), 0, num_seqs, 512, 768)
    return _simple("c2_qwen3_32b_layer", seed, lens, 64, 8, 128, "f16", "f16", "f16", "f16",
                   12480, max_blocks=48, description="Qwen3-32B-shaped single layer decode")


def c3_long_context(num_seqs: int = 8, seq_len: int = 32768) -> Workload:
    """Long context: 8 x 32768 tokens, 64/8 heads, d 128, fp16, 512-token partitions."""
    seed = _cfg_seed(3)
    nb = -(-seq_len // 16)
    return _simple("c3_long_context", seed, [seq_len] * num_seqs, 64, 8, 128, "f16", "f16",
                   "f16", "f16", max(20480, int(num_seqs * nb * 1.25)), max_blocks=nb,
                   partition_size=512, description="long-context split-K decode")


def c4_quantized(cache_dtype: str = "i8", num_seqs: int = 64) -> Workload:
    """Quantized KV: 64 seqs, lognormal lens (median 1500, sigma 1) clamped [16, 8192]."""
    seed = _cfg_seed(4)
    z = normal(stream_key(seed, "lens"), 0, num_seqs)
    lens = np.clip(np.rint(np.exp(math.log(1500.0) + 1.0 * z)), 16, 8192).astype(np.int64)
    nblk = int(sum(-(-int(L) // 16) for L in lens))
    return _simple(f"c4_quantized_{cache_dtype}", seed, lens, 64, 8, 128, "f16", "f16",
                   cache_dtype, "f16", int(math.ceil(nblk * 1.25)), max_blocks=512,
                   description=f"quantized ({cache_dtype}) KV decode")


def c5_shared_prefix(num_seqs: int = 64, prefix: int = 8192, suffix_lo: int = 256,
                     suffix_hi: int = 1024, cow_pairs: bool = False, H: int = 64,
                     Hkv: int = 8, D: int = 128, num_blocks: int = 8192) -> Workload:
    """Shared prefix + copy-on-write decode step.

    The prefix is written once under seq 0, forked to every child and seq 0 is freed.
    Each child then gets its own suffix.  With cow_pairs, half of the children are
    forked once more after their suffix (the pair shares every block, including the
    partly filled tail), so the first writer of a pair copies the tail block.
    The measured step appends one token to every decode seq and writes it.
    """
    seed = _cfg_seed(5) + (1 if cow_pairs else 0)
    n_own = num_seqs // 2 if cow_pairs else num_seqs
    suf = randint(stream_key(seed, "suffix"), 0, n_own, suffix_lo, suffix_hi)
    ops = [("allocate", 0, prefix), ("write", 0, 0, prefix)]
    children = list(range(1, n_own + 1))
    for c in children:
        ops.append(("fork", 0, c))
    ops.append(("free", 0))
    owner = {}
    for c, L in zip(children, suf):
        L = int(L)
        ops.append(("allocate", c, prefix + L))
        ops.append(("write", c, prefix, L))
        owner[c] = [(0, prefix, 0)]
    decode = list(children)
    if cow_pairs:
        for c in children:
            twin = c + n_own
            ops.append(("fork", c, twin))
            owner[twin] = [(0, prefix, 0), (prefix, prefix + int(suf[c - 1]), c)]
            decode.append(twin)
    ops.append(("step",))
    lens_now = {c: prefix + int(suf[c - 1]) for c in children}
    if cow_pairs:
        for c in children:
            lens_now[c + n_own] = lens_now[c]
    for s in decode:
        ops.append(("append", s))
    for s in decode:
        ops.append(("write", s, lens_now[s], 1))
    max_len = prefix + suffix_hi + 1
    return Workload(
        name="c5_shared_prefix_cow" if cow_pairs else "c5_shared_prefix",
        num_heads=H, num_kv_heads=Hkv, head_dim=D, q_dtype="f16", src_dtype="f16",
        cache_dtype="f16", out_dtype="f16", scale=1.0 / math.sqrt(D), num_blocks=num_blocks,
        free_order=permutation(stream_key(seed, "free_order"), num_blocks), ops=ops,
        decode_seqs=decode, max_blocks_per_seq=-(-max_len // 16), seed=seed,
        content_owner=owner, description="shared-prefix copy-on-write decode step")


def forked_groups(name: str, groups, singles=(), suffix_lo: int = 1, suffix_hi: int = 40,
                  H: int = 16, Hkv: int = 2, D: int = 128, cache_dtype: str = "f16",
                  keep_parents: bool = False, seed: int = 11) -> Workload:
    """Several shared prefixes plus independent sequences.

    For each (prefix, n_children) of `groups` a parent is allocated and written
    (prefix tokens), forked to n_children children and, unless keep_parents,
    freed; each child then gets a suffix of U[suffix_lo, suffix_hi] tokens of
    its own (0 allowed).  Kept parents decode too (their length is the
    prefix).  Each length of `singles` is an unrelated sequence.  The decode
    batch lists all of them in a seeded shuffled order.
    """
    seed = _cfg_seed(950) + seed
    ops, owner, decode, lens = [], {}, [], {}
    nid = 1
    for gi, (prefix, nchild) in enumerate(groups):
        parent = nid
        kids = list(range(nid + 1, nid + 1 + nchild))
        nid += 1 + nchild
        ops += [("allocate", parent, prefix), ("write", parent, 0, prefix)]
        ops += [("fork", parent, c) for c in kids]
        if keep_parents:
            decode.append(parent)
            lens[parent] = prefix
        else:
            ops.append(("free", parent))
        suf = randint(stream_key(seed, "suffix", gi), 0, nchild, suffix_lo, suffix_hi)
        for c, L in zip(kids, suf):
            L = int(L)
            if L:
                ops += [("allocate", c, prefix + L), ("write", c, prefix, L)]
            owner[c] = [(0, prefix, parent)]
            lens[c] = prefix + L
            decode.append(c)
    for L in singles:
        ops += [("allocate", nid, int(L)), ("write", nid, 0, int(L))]
        decode.append(nid)
        lens[nid] = int(L)
        nid += 1
    order = permutation(stream_key(seed, "decode_order"), len(decode))
    decode = [decode[int(i)] for i in order]
    need = sum(-(-L // 16) + 1 for L in lens.values())
    num_blocks = need + 16
    max_len = max(lens.values()) + 1
    q_dtype = "f32" if cache_dtype == "f32" else "f16"
    return Workload(
        name=name, num_heads=H, num_kv_heads=Hkv, head_dim=D, q_dtype=q_dtype,
        src_dtype=q_dtype, cache_dtype=cache_dtype,
        out_dtype="f32" if cache_dtype == "f32" else "f16", scale=1.0 / math.sqrt(D),
        num_blocks=num_blocks, free_order=permutation(stream_key(seed, "free_order"), num_blocks),
        ops=ops, decode_seqs=decode, max_blocks_per_seq=-(-max_len // 16), seed=seed,
        content_owner=owner, description="forked shared prefixes and independent sequences")


def chunked_prefill(name: str = "chunked_prefill", contexts=(1536,) * 8, chunks=(512,) * 8,
                    H: int = 64, Hkv: int = 8, D: int = 128, cache_dtype: str = "f16",
                    seed: int = 31) -> Workload:
    """Multi-token queries over the paged cache: sequence i holds contexts[i]
    cached tokens followed by a chunk of chunks[i] new tokens, all written to
    the cache; the chunk's tokens are the queries (chunks[i] = contexts[i] +
    chunks[i] is a whole prefill, chunks[i] = 1 a decode step)."""
    seed = _cfg_seed(960) + seed
    ops, decode, lens = [], [], []
    for i, (c, n) in enumerate(zip(contexts, chunks)):
        L = int(c) + int(n)
        ops += [("allocate", i + 1, L), ("write", i + 1, 0, L)]
        decode.append(i + 1)
        lens.append(L)
    num_blocks = sum(-(-L // 16) for L in lens) + 16
    q_dtype = "f32" if cache_dtype == "f32" else "f16"
    return Workload(
        name=name, num_heads=H, num_kv_heads=Hkv, head_dim=D, q_dtype=q_dtype,
        src_dtype=q_dtype, cache_dtype=cache_dtype,
        out_dtype="f32" if cache_dtype == "f32" else "f16", scale=1.0 / math.sqrt(D),
        num_blocks=num_blocks, free_order=permutation(stream_key(seed, "free_order"), num_blocks),
        ops=ops, decode_seqs=decode, max_blocks_per_seq=-(-max(lens) // 16), seed=seed,
        q_lens=[int(n) for n in chunks], description="chunked prefill over the paged cache")


def custom(name: str, lens, H: int, Hkv: int, D: int, cache_dtype: str = "f16",
           q_dtype: str | None = None, out_dtype: str = "f16", num_blocks: int | None = None,
           max_blocks: int | None = None, partition_size: int = 0, seed: int = 7,
           src_dtype: str | None = None) -> Workload:
    """A small independent-sequence workload for tests and edge cases."""
    if q_dtype is None:
        q_dtype = "f32" if cache_dtype == "f32" else "f16"
    if src_dtype is None:
        src_dtype = "f32" if cache_dtype == "f32" else "f16"
    need = sum(-(-int(L) // 16) for L in lens)
    if num_blocks is None:
        num_blocks = max(4, int(need * 1.5) + 3)
    return _simple(name, _cfg_seed(900) + seed, lens, H, Hkv, D, q_dtype, src_dtype,
                   cache_dtype, out_dtype, num_blocks, max_blocks=max_blocks,
                   partition_size=partition_size)


def with_block_size(w: Workload, block_size: int) -> Workload:
    """The same workload (same token script, same values) on blocks of
    `block_size` tokens: the pool keeps its token capacity and gets a free
    order of its own; table rows hold the same number of tokens."""
    import copy
    w2 = copy.copy(w)
    tokens = w.max_blocks_per_seq * w.block_size
    w2.block_size = block_size
    w2.max_blocks_per_seq = -(-tokens // block_size)
    w2.num_blocks = -(-w.num_blocks * w.block_size // block_size)
    w2.free_order = permutation(stream_key(w.seed, "free_order", block_size), w2.num_blocks)
    w2.name = f"{w.name}_bs{block_size}"
    w2.memo = None
    return w2


def with_decode_step(w: Workload) -> Workload:
    """The same workload followed by one decode step: every decode sequence
    appends one token (position = its current length) and writes it."""
    import copy
    lens = {}
    for op in w.ops:
        if op[0] == "step":
            raise ValueError("workload already has a step")
        if op[0] == "allocate":
            lens[op[1]] = max(lens.get(op[1], 0), op[2])
        elif op[0] == "fork":
            lens[op[2]] = lens.get(op[1], 0)
        elif op[0] == "append":
            lens[op[1]] = lens.get(op[1], 0) + 1
    w2 = copy.copy(w)
    w2.ops = list(w.ops) + [("step",)] + [("append", s) for s in w.decode_seqs] + \
        [("write", s, lens.get(s, 0), 1) for s in w.decode_seqs]
    w2.max_blocks_per_seq = max(w.max_blocks_per_seq,
                                max(-(-(lens.get(s, 0) + 1) // w.block_size)
                                    for s in w.decode_seqs))
    w2.name = w.name + "_step"
    w2.memo = None
    return w2


def step_rows(w: Workload):
    """K and V rows [S, Hkv, D] of the tokens the step of `w` writes, in
    decode-sequence order (the step's write ops)."""
    after = w.ops[w.ops.index(("step",)) + 1:]
    writes = {op[1]: op[2] for op in after if op[0] == "write"}
    ks, vs = [], []
    for s in w.decode_seqs:
        pos = writes[s]
        owner = w.owner_of(s, pos)
        ks.append(w.kv_rows("k", owner, pos, 1)[0])
        vs.append(w.kv_rows("v", owner, pos, 1)[0])
    return np.stack(ks), np.stack(vs)


CONFIGS = {
    "c1": c1_tiny,
    "c2": c2_qwen3_32b_layer,
    "c3": c3_long_context,
    "c4_i8": lambda: c4_quantized("i8"),
    "c4_e4m3": lambda: c4_quantized("e4m3"),
    "c5": c5_shared_prefix,
    "c5_cow": lambda: c5_shared_prefix(cow_pairs=True),
}
