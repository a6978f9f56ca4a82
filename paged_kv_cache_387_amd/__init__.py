"""Python binding of libpkv (paged KV cache + PagedAttention decode for MI355X).

Argument marshalling only: every step of the hot path runs in the HIP kernels
of libpkv.so.  PyTorch provides device memory and streams.  The binding checks
tensor sizes, dtypes and devices against the shapes it passes, because the C
ABI only sees raw pointers.  It never falls back to another implementation:
if libpkv.so is missing or fails to load, importing the device entry points
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

OK, EINVAL, ENOMEM, ENOENT, EEXIST, EDEVICE, ENOTSUP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 48 << 20   # PKV_NOALLOC_SCRATCH_BYTES
WALK_SPLIT, WALK_RUNS, WALK_STREAM = 0, 1, 2   # PKV_WALK_*
F32, F16, I8, E4M3 = 0, 1, 3, 4
DTYPE = {"f32": F32, "f16": F16, "i8": I8, "e4m3": E4M3}
ELEM_BYTES = {F32: 4, F16: 2, I8: 1, E4M3: 1}
BLOCK_SIZE = 16

# every symbol include/pkv.h declares
EXPORTS = [
    "pkv_strerror", "pkv_version",
    "pkv_alloc_create", "pkv_alloc_destroy", "pkv_alloc_num_free", "pkv_alloc_free_list",
    "pkv_block_refcount", "pkv_seq_allocate", "pkv_seq_append_slot", "pkv_seq_append_slots",
    "pkv_seq_step",
    "pkv_seq_fork", "pkv_seq_free", "pkv_seq_len", "pkv_seq_slots", "pkv_export_tables",
    "pkv_export_shared_tables",
    "pkv_alloc_set_host_blocks", "pkv_alloc_num_free_host", "pkv_alloc_free_list_host",
    "pkv_host_block_refcount", "pkv_seq_on_host", "pkv_seq_swap_out", "pkv_seq_swap_in",
    "pkv_seq_allocate_cached", "pkv_seq_cache_blocks", "pkv_prefix_cache_evict",
    "pkv_prefix_cache_size", "pkv_prefix_cache_evictable", "paged_swap_blocks",
    "paged_kv_write", "paged_copy_blocks", "paged_attention_partition_size",
    "paged_attention_decode_walk",
    "paged_attention_workspace_bytes", "paged_attention_decode",
    "paged_attention_decode_noalloc", "paged_decode_step",
    "paged_attention_shared_workspace_bytes", "paged_attention_decode_shared",
    "paged_attention_prefill_workspace_bytes", "paged_attention_prefill",
]


class PrefixGroupsC(ctypes.Structure):
    """struct pkv_prefix_groups of pkv.h (host struct of device pointers)."""
    _fields_ = [("num_groups", ctypes.c_int32), ("num_members", ctypes.c_int32),
                ("max_group_size", ctypes.c_int32), ("max_prefix_blocks", ctypes.c_int32),
                ("offsets", ctypes.c_void_p), ("members", ctypes.c_void_p),
                ("tables", ctypes.c_void_p), ("prefix_lens", ctypes.c_void_p),
                ("seq_group", ctypes.c_void_p)]


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpkv.so (built by `paged_kv_cache_387_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m paged_kv_cache_387_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_float, ctypes.c_size_t)
        sig = {
            "pkv_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "pkv_version": ([], ctypes.c_int),
            "pkv_alloc_create": ([i32, i32, P, P], ctypes.c_int),
            "pkv_alloc_destroy": ([P], None),
            "pkv_alloc_num_free": ([P], i32),
            "pkv_alloc_free_list": ([P, P, i32], i32),
            "pkv_block_refcount": ([P, i32], i32),
            "pkv_seq_allocate": ([P, i64, i32, P, P], ctypes.c_int),
            "pkv_seq_append_slot": ([P, i64, P, P, P], ctypes.c_int),
            "pkv_seq_append_slots": ([P, P, i32, P, P, P, P, P], ctypes.c_int),
            "pkv_seq_step": ([P, P, i32, i32, P, P, P, P], ctypes.c_int),
            "pkv_seq_fork": ([P, i64, i64], ctypes.c_int),
            "pkv_seq_free": ([P, i64], ctypes.c_int),
            "pkv_seq_len": ([P, i64, P], ctypes.c_int),
            "pkv_seq_slots": ([P, i64, i32, i32, P], ctypes.c_int),
            "pkv_export_tables": ([P, P, i32, i32, P, P], ctypes.c_int),
            "pkv_export_shared_tables": ([P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P],
                                         ctypes.c_int),
            "pkv_alloc_set_host_blocks": ([P, i32], ctypes.c_int),
            "pkv_alloc_num_free_host": ([P], i32),
            "pkv_alloc_free_list_host": ([P, P, i32], i32),
            "pkv_host_block_refcount": ([P, i32], i32),
            "pkv_seq_on_host": ([P, i64, P], ctypes.c_int),
            "pkv_seq_swap_out": ([P, P, i32, P, i32, P], ctypes.c_int),
            "pkv_seq_swap_in": ([P, P, i32, P, i32, P], ctypes.c_int),
            "pkv_seq_allocate_cached": ([P, i64, P, i32, P], ctypes.c_int),
            "pkv_seq_cache_blocks": ([P, i64, P, i32], ctypes.c_int),
            "pkv_prefix_cache_evict": ([P, i32, P], ctypes.c_int),
            "pkv_prefix_cache_size": ([P], i32),
            "pkv_prefix_cache_evictable": ([P, P, i32], i32),
            "paged_swap_blocks": ([P, P, P, P, P, P, P, P, i32, i32, i32, P, i32, i32, i32, i32,
                                   i32, P], ctypes.c_int),
            "paged_kv_write": ([P, P, i32, i64, i64, P, i32, P, P, P, P, i32, i32, i32, i32,
                                i32, P], ctypes.c_int),
            "paged_copy_blocks": ([P, P, P, P, i32, i32, P, i32, i32, i32, i32, P],
                                  ctypes.c_int),
            "paged_attention_partition_size": ([i32, i32, i32, i32, i32], i32),
            "paged_attention_decode_walk": ([i32, i32, i32, i32, i32, i32, i32], i32),
            "paged_attention_workspace_bytes": ([i32, i32, i32, i32, i32, i32, i32], sz),
            "paged_attention_decode": ([P, i32, P, i32, P, P, P, P, i32, i32, P, i32, P, i32,
                                        i32, i32, i32, i32, f32, i32, P, sz, P], ctypes.c_int),
            "paged_attention_decode_noalloc": ([P, i32, P, i32, P, P, P, P, i32, i32, P, i32,
                                                P, i32, i32, i32, i32, i32, f32, i32, P],
                                               ctypes.c_int),
            "paged_decode_step": ([P, i32, P, i32, P, P, i32, P, P, P, P, P, i32, i32, P, i32,
                                   P, i32, i32, i32, i32, i32, f32, i32, P, sz, P],
                                  ctypes.c_int),
            "paged_attention_shared_workspace_bytes": ([i32, i32, i32, i32, i32, i32, i32, P],
                                                       sz),
            "paged_attention_decode_shared": ([P, i32, P, i32, P, P, i32, P, P, P, P, P, i32,
                                               i32, P, i32, P, i32, i32, i32, i32, i32, f32, P,
                                               i32, P, sz, P], ctypes.c_int),
            "paged_attention_prefill_workspace_bytes": ([i32, i32, i32, i32, i32, i32, i32,
                                                         i32, i32], sz),
            "paged_attention_prefill": ([P, i32, P, i32, P, P, P, P, i32, i32, P, i32, P, P, i32,
                                         i32, i32, i32, i32, i32, i32, f32, i32, P, sz, P],
                                        ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().pkv_strerror(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise PkvError(status, what)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# host block allocator
# ---------------------------------------------------------------------------

class BlockAllocator:
    """Host block manager: free list, per-sequence tables, refcounts, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        self._h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        _check(lib().pkv_alloc_create(num_blocks, block_size,
                                      None if order is None else _np_ptr(order),
                                      ctypes.byref(self._h)), "pkv_alloc_create")
        self.num_blocks, self.block_size = num_blocks, block_size

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().pkv_alloc_destroy(self._h)
            self._h = ctypes.c_void_p()

    @property
    def num_free(self) -> int:
        return lib().pkv_alloc_num_free(self._h)

    def free_list(self) -> list:
        n = self.num_free
        out = np.empty(max(n, 1), np.int32)
        lib().pkv_alloc_free_list(self._h, _np_ptr(out), n)
        return out[:n].tolist()

    def refcount(self, block: int) -> int:
        return lib().pkv_block_refcount(self._h, block)

    def allocate(self, seq: int, num_tokens: int):
        """Returns the copy-on-write pair (src, dst) or None; raises PkvError on failure."""
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_seq_allocate(self._h, seq, num_tokens, ctypes.byref(src),
                                      ctypes.byref(dst)), "pkv_seq_allocate")
        return None if src.value < 0 else (src.value, dst.value)

    def try_allocate(self, seq: int, num_tokens: int) -> int:
        return lib().pkv_seq_allocate(self._h, seq, num_tokens, None, None)

    def append_slot(self, seq: int):
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_seq_append_slot(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                         ctypes.byref(dst)), "pkv_seq_append_slot")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_slots(self, seqs, with_src: bool = False):
        """Append one token to each sequence: returns (slots, copy pairs [n, 2])
        and, with with_src, each sequence's copy source block (-1: none)."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(ids)
        slots = np.empty(max(n, 1), np.int64)
        pairs = np.empty((max(n, 1), 2), np.int32)
        src = np.empty(max(n, 1), np.int32)
        ncow, done = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_seq_append_slots(self._h, _np_ptr(ids), n, _np_ptr(slots),
                                          _np_ptr(pairs), ctypes.byref(ncow), _np_ptr(src),
                                          ctypes.byref(done)), "pkv_seq_append_slots")
        if with_src:
            return slots[:n], pairs[:ncow.value], src[:n]
        return slots[:n], pairs[:ncow.value]

    def step(self, seqs, max_blocks: int, out=None):
        """One decode step: append a token to each sequence (all or nothing)
        and export the tables, lengths, copy sources and slots of the batch.
        `out` (optional) is a dict of preallocated host arrays (tables, lens,
        cow_src, slots) that is filled and returned."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(ids)
        if out is None:
            out = {"tables": np.empty((max(n, 1), max_blocks), np.int32),
                   "lens": np.empty(max(n, 1), np.int32),
                   "cow_src": np.empty(max(n, 1), np.int32),
                   "slots": np.empty(max(n, 1), np.int64)}
        _check(lib().pkv_seq_step(self._h, _np_ptr(ids), n, max_blocks, _np_ptr(out["slots"]),
                                  _np_ptr(out["cow_src"]), _np_ptr(out["tables"]),
                                  _np_ptr(out["lens"])), "pkv_seq_step")
        return out

    def fork(self, parent: int, child: int):
        _check(lib().pkv_seq_fork(self._h, parent, child), "pkv_seq_fork")

    def free(self, seq: int):
        _check(lib().pkv_seq_free(self._h, seq), "pkv_seq_free")

    def seq_len(self, seq: int) -> int:
        n = ctypes.c_int32()
        _check(lib().pkv_seq_len(self._h, seq, ctypes.byref(n)), "pkv_seq_len")
        return n.value

    def slots(self, seq: int, start: int, count: int) -> np.ndarray:
        out = np.empty(max(count, 1), np.int64)
        _check(lib().pkv_seq_slots(self._h, seq, start, count, _np_ptr(out)), "pkv_seq_slots")
        return out[:count]

    def export_tables(self, seqs, max_blocks: int):
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(ids)
        tables = np.empty((max(n, 1), max_blocks), np.int32)
        lens = np.empty(max(n, 1), np.int32)
        _check(lib().pkv_export_tables(self._h, _np_ptr(ids), n, max_blocks, _np_ptr(tables),
                                       _np_ptr(lens)), "pkv_export_tables")
        return tables[:n], lens[:n]

    # ---- host pool and swapping ------------------------------------------------
    def set_host_blocks(self, n: int):
        _check(lib().pkv_alloc_set_host_blocks(self._h, n), "pkv_alloc_set_host_blocks")
        self._num_host = n

    @property
    def num_free_host(self) -> int:
        return lib().pkv_alloc_num_free_host(self._h)

    def free_list_host(self) -> list:
        n = self.num_free_host
        out = np.empty(max(n, 1), np.int32)
        lib().pkv_alloc_free_list_host(self._h, _np_ptr(out), n)
        return out[:n].tolist()

    def host_refcount(self, block: int) -> int:
        return lib().pkv_host_block_refcount(self._h, block)

    def on_host(self, seq: int) -> bool:
        f = ctypes.c_int32(0)
        _check(lib().pkv_seq_on_host(self._h, seq, ctypes.byref(f)), "pkv_seq_on_host")
        return bool(f.value)

    def _swap(self, fn, seqs, what):
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        # distinct blocks of a swap never exceed either pool
        cap = 1 + self.num_blocks + self.num_free_host + sum(self._host_held())
        pairs = np.empty((cap, 2), np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, _np_ptr(ids), len(ids), _np_ptr(pairs), cap, ctypes.byref(n)), what)
        return pairs[:n.value].copy()

    def _host_held(self):
        # host blocks in use (the pool size minus the free ones)
        return [self._num_host - self.num_free_host] if hasattr(self, "_num_host") else [0]

    def swap_out(self, seqs) -> np.ndarray:
        """[device, host] block pairs to copy (paged_swap_blocks, to_host=True)."""
        return self._swap(lib().pkv_seq_swap_out, seqs, "pkv_seq_swap_out")

    def swap_in(self, seqs) -> np.ndarray:
        """[host, device] block pairs to copy (paged_swap_blocks, to_host=False)."""
        return self._swap(lib().pkv_seq_swap_in, seqs, "pkv_seq_swap_in")

    # ---- automatic prefix caching ---------------------------------------------
    def allocate_cached(self, seq: int, tokens) -> int:
        """New sequence for a prompt; returns how many leading tokens were found
        in the prefix cache (their K/V are there already)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        got = ctypes.c_int32(0)
        _check(lib().pkv_seq_allocate_cached(self._h, seq, _np_ptr(t), len(t), ctypes.byref(got)),
               "pkv_seq_allocate_cached")
        return got.value

    def cache_blocks(self, seq: int, tokens, n: int | None = None):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib().pkv_seq_cache_blocks(self._h, seq, _np_ptr(t), len(t) if n is None else n),
               "pkv_seq_cache_blocks")

    def cache_evict(self, max_blocks: int) -> int:
        k = ctypes.c_int32(0)
        _check(lib().pkv_prefix_cache_evict(self._h, max_blocks, ctypes.byref(k)),
               "pkv_prefix_cache_evict")
        return k.value

    @property
    def cache_size(self) -> int:
        return lib().pkv_prefix_cache_size(self._h)

    def cache_evictable(self) -> list:
        n = lib().pkv_prefix_cache_evictable(self._h, None, 0)
        out = np.empty(max(n, 1), np.int32)
        lib().pkv_prefix_cache_evictable(self._h, _np_ptr(out), n)
        return out[:n].tolist()

    def export_shared(self, seqs, max_prefix_blocks: int, max_suffix_blocks: int,
                      min_prefix_tokens: int = 0) -> dict:
        """Tables split into shared prefixes and private suffixes (host numpy
        arrays, trimmed to their used lengths): suffix_tables, suffix_lens,
        seq_group, group_offsets, group_members, group_tables,
        group_prefix_lens, num_groups, max_group_size, max_prefix_blocks."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(ids)
        m = max(n, 1)
        st = np.empty((m, max_suffix_blocks), np.int32)
        sl = np.empty(m, np.int32)
        sg = np.empty(m, np.int32)
        go = np.empty(m + 1, np.int32)
        gm = np.empty(m, np.int32)
        gt = np.empty((m, max_prefix_blocks), np.int32)
        gp = np.empty(m, np.int32)
        ng, mg = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pkv_export_shared_tables(
            self._h, _np_ptr(ids), n, min_prefix_tokens, max_prefix_blocks, max_suffix_blocks,
            _np_ptr(st), _np_ptr(sl), _np_ptr(sg), _np_ptr(go), _np_ptr(gm), _np_ptr(gt),
            _np_ptr(gp), ctypes.byref(ng), ctypes.byref(mg)), "pkv_export_shared_tables")
        g = ng.value
        return dict(suffix_tables=st[:n], suffix_lens=sl[:n], seq_group=sg[:n],
                    group_offsets=go[:g + 1], group_members=gm[:go[g]],
                    group_tables=gt[:g], group_prefix_lens=gp[:g], num_groups=g,
                    max_group_size=mg.value, max_prefix_blocks=max_prefix_blocks,
                    block_size=self.block_size)


# ---------------------------------------------------------------------------
# device operations
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, what, dtype=None, numel=None):
    torch = _torch()
    if t is None:
        raise ValueError(f"{what} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def cache_bytes(num_blocks: int, num_kv_heads: int, head_dim: int, cache_dtype: int,
                block_size: int = BLOCK_SIZE) -> int:
    return num_blocks * num_kv_heads * block_size * head_dim * ELEM_BYTES[cache_dtype]


class PagedKVCache:
    """K and V block pools (uint8 device tensors in the ABI layout) and, for
    int8 / E4M3, their fp16 scale arrays."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, cache_dtype="f16",
                 block_size: int = BLOCK_SIZE, device="cuda", fill_byte: int | None = None):
        torch = _torch()
        self.cache_dtype = DTYPE[cache_dtype] if isinstance(cache_dtype, str) else cache_dtype
        self.num_blocks, self.num_kv_heads = num_blocks, num_kv_heads
        self.head_dim, self.block_size = head_dim, block_size
        nbytes = cache_bytes(num_blocks, num_kv_heads, head_dim, self.cache_dtype, block_size)
        mk = (lambda n, dt: torch.empty(n, dtype=dt, device=device)) if fill_byte is None else \
            (lambda n, dt: torch.full((n,), fill_byte, dtype=torch.uint8, device=device).view(dt))
        self.k = mk(nbytes, torch.uint8)
        self.v = mk(nbytes, torch.uint8)
        if self.cache_dtype in (I8, E4M3):
            ns = num_blocks * num_kv_heads * block_size
            self.k_scale = mk(2 * ns, torch.uint8).view(torch.float16) if fill_byte is not None \
                else torch.empty(ns, dtype=torch.float16, device=device)
            self.v_scale = mk(2 * ns, torch.uint8).view(torch.float16) if fill_byte is not None \
                else torch.empty(ns, dtype=torch.float16, device=device)
        else:
            self.k_scale = self.v_scale = None

    @property
    def quantized(self) -> bool:
        return self.k_scale is not None

    def _scales(self):
        if not self.quantized:
            return None, None
        n = self.num_blocks * self.num_kv_heads * self.block_size
        torch = _torch()
        return (_dev(self.k_scale, "k_scale", torch.float16, n),
                _dev(self.v_scale, "v_scale", torch.float16, n))

    def write(self, key, value, slot_mapping, stream=None):
        paged_kv_write(key, value, slot_mapping, self, stream=stream)

    def copy_blocks(self, pairs, stream=None):
        paged_copy_blocks(self, pairs, stream=stream)


class HostKVPool:
    """Host-side block pools for swapped-out sequences: pinned (page-locked,
    device-addressable) uint8 tensors in the device pools' layout, plus fp16
    scale arrays for quantized caches."""

    def __init__(self, num_host_blocks: int, like: PagedKVCache):
        torch = _torch()
        self.num_blocks = num_host_blocks
        self.like = like
        nbytes = cache_bytes(num_host_blocks, like.num_kv_heads, like.head_dim, like.cache_dtype,
                             like.block_size)
        self.k = torch.zeros(max(nbytes, 16), dtype=torch.uint8, pin_memory=True)
        self.v = torch.zeros(max(nbytes, 16), dtype=torch.uint8, pin_memory=True)
        self.k_scale = self.v_scale = None
        if like.quantized:
            n = max(num_host_blocks * like.num_kv_heads * like.block_size, 1)
            self.k_scale = torch.zeros(n, dtype=torch.float16, pin_memory=True)
            self.v_scale = torch.zeros(n, dtype=torch.float16, pin_memory=True)


def paged_swap_blocks(cache: PagedKVCache, host: HostKVPool, pairs, to_host: bool,
                      stream=None):
    """Copy whole blocks between the device pools and the host pools: rows
    [device, host] (to_host) or [host, device] of `pairs` (int32 device [n, 2])."""
    torch = _torch()
    n = 0 if pairs is None else pairs.shape[0]
    if n == 0:
        return
    for t in (host.k, host.v):
        if not t.is_pinned():
            raise ValueError("host pools must be pinned memory")
    ks, vs = cache._scales()
    hks = hvs = None
    if cache.quantized:
        hks = ctypes.c_void_p(host.k_scale.data_ptr())
        hvs = ctypes.c_void_p(host.v_scale.data_ptr())
    _check(lib().paged_swap_blocks(
        _dev(cache.k, "k_cache"), _dev(cache.v, "v_cache"), ks, vs,
        ctypes.c_void_p(host.k.data_ptr()), ctypes.c_void_p(host.v.data_ptr()), hks, hvs,
        cache.cache_dtype, cache.num_blocks, host.num_blocks,
        _dev(pairs, "pairs", torch.int32, 2 * n), n, 1 if to_host else 0, cache.num_kv_heads,
        cache.head_dim, cache.block_size, _stream_ptr(stream)), "paged_swap_blocks")


def paged_kv_write(key, value, slot_mapping, cache: PagedKVCache, stream=None):
    """Write key/value [T, num_kv_heads, head_dim] (f32 or f16) into their slots."""
    torch = _torch()
    T = slot_mapping.shape[0]
    row = cache.num_kv_heads * cache.head_dim
    src = {torch.float32: F32, torch.float16: F16}.get(key.dtype)
    if src is None or value.dtype != key.dtype:
        raise ValueError("key/value must both be float32 or float16")
    if key.shape != (T, cache.num_kv_heads, cache.head_dim) or value.shape != key.shape:
        raise ValueError(f"key/value must be [{T}, {cache.num_kv_heads}, {cache.head_dim}]")
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, cache.head_dim,
                         cache.cache_dtype, cache.block_size)
    ks, vs = cache._scales()
    _check(lib().paged_kv_write(
        _dev(key, "key", numel=T * row), _dev(value, "value", numel=T * row), src, 0, 0,
        _dev(slot_mapping, "slot_mapping", torch.int64, T), T,
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks, cache.num_kv_heads, cache.head_dim,
        cache.block_size, _stream_ptr(stream)), "paged_kv_write")


def paged_copy_blocks(cache: PagedKVCache, pairs, stream=None):
    """Copy whole blocks for pairs (int32 device tensor [n, 2] of src, dst)."""
    torch = _torch()
    n = pairs.shape[0] if pairs.dim() == 2 else pairs.numel() // 2
    if n == 0:
        return
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, cache.head_dim,
                         cache.cache_dtype, cache.block_size)
    ks, vs = cache._scales()
    _check(lib().paged_copy_blocks(
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks, _dev(pairs, "pairs", torch.int32, 2 * n), n,
        cache.num_kv_heads, cache.head_dim, cache.block_size, _stream_ptr(stream)),
        "paged_copy_blocks")


def partition_size(num_seqs: int, num_kv_heads: int, max_blocks_per_seq: int,
                   requested: int = 0, block_size: int = BLOCK_SIZE) -> int:
    v = lib().paged_attention_partition_size(num_seqs, num_kv_heads, max_blocks_per_seq,
                                             block_size, requested)
    _check(min(v, 0), "paged_attention_partition_size")
    return v


def decode_walk(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                max_blocks_per_seq: int, partition_size: int = 0,
                block_size: int = BLOCK_SIZE) -> int:
    """How paged_attention_decode spreads the work for these shapes:
    WALK_SPLIT, WALK_RUNS or WALK_STREAM."""
    v = lib().paged_attention_decode_walk(num_seqs, num_heads, num_kv_heads, head_dim,
                                          max_blocks_per_seq, block_size, partition_size)
    _check(min(v, 0), "paged_attention_decode_walk")
    return v


def workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                    max_blocks_per_seq: int, partition_size: int = 0,
                    block_size: int = BLOCK_SIZE) -> int:
    return lib().paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                 max_blocks_per_seq, block_size, partition_size)


def alloc_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                    partition_size=0, device="cuda", block_size: int = BLOCK_SIZE):
    n = workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                        partition_size, block_size)
    torch = _torch()
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def paged_attention_decode(query, cache: PagedKVCache, block_tables, seq_lens, scale: float,
                           out=None, out_dtype=None, partition_size: int = 0, workspace=None,
                           stream=None):
    """out[s, h] = softmax(scale * q[s, h] . K) V over the sequence's cached tokens."""
    torch = _torch()
    S, H, D = query.shape
    q_dt = {torch.float32: F32, torch.float16: F16}.get(query.dtype)
    if q_dt is None:
        raise ValueError("query must be float32 or float16")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    maxb = block_tables.shape[1]
    if out is None:
        odt = out_dtype if out_dtype is not None else query.dtype
        out = torch.empty((S, H, D), dtype=odt, device=query.device)
    o_dt = {torch.float32: F32, torch.float16: F16}.get(out.dtype)
    if o_dt is None or tuple(out.shape) != (S, H, D):
        raise ValueError("out must be float32/float16 [num_seqs, num_heads, head_dim]")
    if D != cache.head_dim or H % cache.num_kv_heads:
        raise ValueError("query shape does not match the cache")
    need = workspace_bytes(S, H, cache.num_kv_heads, D, maxb, partition_size, cache.block_size)
    if need > 0 and workspace is None:
        workspace = alloc_workspace(S, H, cache.num_kv_heads, D, maxb, partition_size,
                                    device=query.device, block_size=cache.block_size)
    ws_ptr, ws_len = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", numel=need)
        ws_len = workspace.numel() * workspace.element_size()
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, D, cache.cache_dtype,
                         cache.block_size)
    ks, vs = cache._scales()
    _check(lib().paged_attention_decode(
        _dev(out, "out"), o_dt, _dev(query, "query"), q_dt,
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks,
        _dev(block_tables, "block_tables", torch.int32, S * maxb), maxb,
        _dev(seq_lens, "seq_lens", torch.int32, S), S, H, cache.num_kv_heads, D,
        cache.block_size, float(scale), partition_size, ws_ptr, ws_len, _stream_ptr(stream)),
        "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(query, cache: PagedKVCache, block_tables, seq_lens,
                                   scale: float, out, partition_size: int = 0, stream=None):
    """paged_attention_decode with the split-K partials in the library's own
    scratch array (no workspace, nothing allocated by the library; `out` is
    the caller's)."""
    torch = _torch()
    S, H, D = query.shape
    q_dt = {torch.float32: F32, torch.float16: F16}.get(query.dtype)
    o_dt = {torch.float32: F32, torch.float16: F16}.get(out.dtype)
    if q_dt is None or o_dt is None or tuple(out.shape) != (S, H, D):
        raise ValueError("query / out must be float32 or float16 [num_seqs, num_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    maxb = block_tables.shape[1]
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, D, cache.cache_dtype,
                         cache.block_size)
    ks, vs = cache._scales()
    _check(lib().paged_attention_decode_noalloc(
        _dev(out, "out"), o_dt, _dev(query, "query"), q_dt,
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks,
        _dev(block_tables, "block_tables", torch.int32, S * maxb), maxb,
        _dev(seq_lens, "seq_lens", torch.int32, S), S, H, cache.num_kv_heads, D,
        cache.block_size, float(scale), partition_size, _stream_ptr(stream)),
        "paged_attention_decode_noalloc")
    return out


def paged_decode_step(query, key, value, cache: PagedKVCache, block_tables, seq_lens,
                      scale: float, cow_src=None, out=None, out_dtype=None,
                      partition_size: int = 0, workspace=None, stream=None):
    """One fused decode step: copy-on-write of each sequence's tail block from
    cow_src[s] (int32 device [S], -1 none; optional), the new token key[s] /
    value[s] ([S, num_kv_heads, head_dim]) written at position seq_lens[s]-1,
    then paged decode attention over all seq_lens[s] tokens."""
    torch = _torch()
    S, H, D = query.shape
    q_dt = {torch.float32: F32, torch.float16: F16}.get(query.dtype)
    src = {torch.float32: F32, torch.float16: F16}.get(key.dtype)
    if q_dt is None or src is None or value.dtype != key.dtype:
        raise ValueError("query/key/value must be float32 or float16")
    if tuple(key.shape) != (S, cache.num_kv_heads, D) or value.shape != key.shape:
        raise ValueError(f"key/value must be [{S}, {cache.num_kv_heads}, {D}]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    maxb = block_tables.shape[1]
    if out is None:
        odt = out_dtype if out_dtype is not None else query.dtype
        out = torch.empty((S, H, D), dtype=odt, device=query.device)
    o_dt = {torch.float32: F32, torch.float16: F16}.get(out.dtype)
    if o_dt is None or tuple(out.shape) != (S, H, D):
        raise ValueError("out must be float32/float16 [num_seqs, num_heads, head_dim]")
    if D != cache.head_dim or H % cache.num_kv_heads:
        raise ValueError("query shape does not match the cache")
    need = workspace_bytes(S, H, cache.num_kv_heads, D, maxb, partition_size, cache.block_size)
    if need > 0 and workspace is None:
        workspace = alloc_workspace(S, H, cache.num_kv_heads, D, maxb, partition_size,
                                    device=query.device, block_size=cache.block_size)
    ws_ptr, ws_len = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", numel=need)
        ws_len = workspace.numel() * workspace.element_size()
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, D, cache.cache_dtype,
                         cache.block_size)
    ks, vs = cache._scales()
    row = S * cache.num_kv_heads * D
    _check(lib().paged_decode_step(
        _dev(out, "out"), o_dt, _dev(query, "query"), q_dt,
        _dev(key, "key", numel=row), _dev(value, "value", numel=row), src,
        None if cow_src is None else _dev(cow_src, "cow_src", torch.int32, S),
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks,
        _dev(block_tables, "block_tables", torch.int32, S * maxb), maxb,
        _dev(seq_lens, "seq_lens", torch.int32, S), S, H, cache.num_kv_heads, D,
        cache.block_size, float(scale), partition_size, ws_ptr, ws_len, _stream_ptr(stream)),
        "paged_decode_step")
    return out


class PrefixGroups:
    """Device copy of the group arrays of BlockAllocator.export_shared and the
    pkv_prefix_groups struct that points at them."""

    def __init__(self, shared: dict, device="cuda"):
        torch = _torch()

        def up(a):
            a = np.ascontiguousarray(a, dtype=np.int32).reshape(-1)
            return torch.from_numpy(a if a.size else np.zeros(1, np.int32)).to(device)

        self.num_groups = int(shared["num_groups"])
        self.max_group_size = max(int(shared["max_group_size"]), 1)
        # the prefix tables cut to the longest prefix (the prefix pass plans
        # its partitions over this width)
        plens = np.asarray(shared["group_prefix_lens"], np.int64)
        width = int(shared["max_prefix_blocks"])
        if self.num_groups > 0:
            bs = int(shared.get("block_size", 0)) or None
            longest = int(plens.max())
            if bs:
                width = max(1, min(width, -(-longest // bs)))
            shared = dict(shared, group_tables=np.ascontiguousarray(
                np.asarray(shared["group_tables"], np.int32)[:, :width]))
        self.max_prefix_blocks = width
        self.num_members = int(len(shared["group_members"]))
        self.offsets = up(shared["group_offsets"])
        self.members = up(shared["group_members"])
        self.tables = up(shared["group_tables"])
        self.prefix_lens = up(shared["group_prefix_lens"])
        self.seq_group = up(shared["seq_group"])
        self.num_seqs = int(len(shared["seq_group"]))
        if self.num_groups > 0:
            need = self.num_groups * self.max_prefix_blocks
            if self.tables.numel() < need or self.offsets.numel() < self.num_groups + 1:
                raise ValueError("group arrays are shorter than num_groups needs")
        self.c = PrefixGroupsC(self.num_groups, self.num_members, self.max_group_size,
                               self.max_prefix_blocks, self.offsets.data_ptr(),
                               self.members.data_ptr(), self.tables.data_ptr(),
                               self.prefix_lens.data_ptr(), self.seq_group.data_ptr())


def shared_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                           max_blocks_per_seq: int, groups: PrefixGroups,
                           partition_size: int = 0, block_size: int = BLOCK_SIZE) -> int:
    return lib().paged_attention_shared_workspace_bytes(
        num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
        partition_size, ctypes.byref(groups.c))


def paged_attention_decode_shared(query, cache: PagedKVCache, block_tables, seq_lens,
                                  scale: float, groups: PrefixGroups, key=None, value=None,
                                  cow_src=None, out=None, out_dtype=None,
                                  partition_size: int = 0, workspace=None, stream=None):
    """Decode (or, with key / value, the fused decode step) of sequences whose
    tables are split into a shared prefix (groups) and a private suffix
    (block_tables / seq_lens): each prefix block is read once per (group, kv
    head) for all the group's queries."""
    torch = _torch()
    S, H, D = query.shape
    q_dt = {torch.float32: F32, torch.float16: F16}.get(query.dtype)
    if q_dt is None:
        raise ValueError("query must be float32 or float16")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if groups.num_groups > 0 and groups.num_seqs != S:
        raise ValueError("groups describe a different number of sequences")
    maxb = block_tables.shape[1]
    if out is None:
        odt = out_dtype if out_dtype is not None else query.dtype
        out = torch.empty((S, H, D), dtype=odt, device=query.device)
    o_dt = {torch.float32: F32, torch.float16: F16}.get(out.dtype)
    if o_dt is None or tuple(out.shape) != (S, H, D):
        raise ValueError("out must be float32/float16 [num_seqs, num_heads, head_dim]")
    if D != cache.head_dim or H % cache.num_kv_heads:
        raise ValueError("query shape does not match the cache")
    kp = vp = cp = None
    src = F16
    if key is not None or value is not None:
        src = {torch.float32: F32, torch.float16: F16}.get(key.dtype)
        if src is None or value is None or value.dtype != key.dtype:
            raise ValueError("key/value must both be float32 or float16")
        if tuple(key.shape) != (S, cache.num_kv_heads, D) or value.shape != key.shape:
            raise ValueError(f"key/value must be [{S}, {cache.num_kv_heads}, {D}]")
        row = S * cache.num_kv_heads * D
        kp, vp = _dev(key, "key", numel=row), _dev(value, "value", numel=row)
        cp = None if cow_src is None else _dev(cow_src, "cow_src", torch.int32, S)
    need = shared_workspace_bytes(S, H, cache.num_kv_heads, D, maxb, groups, partition_size,
                                  cache.block_size)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr, ws_len = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", numel=need)
        ws_len = workspace.numel() * workspace.element_size()
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, D, cache.cache_dtype,
                         cache.block_size)
    ks, vs = cache._scales()
    _check(lib().paged_attention_decode_shared(
        _dev(out, "out"), o_dt, _dev(query, "query"), q_dt, kp, vp, src, cp,
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks,
        _dev(block_tables, "block_tables", torch.int32, S * maxb), maxb,
        _dev(seq_lens, "seq_lens", torch.int32, S), S, H, cache.num_kv_heads, D,
        cache.block_size, float(scale), ctypes.byref(groups.c), partition_size, ws_ptr, ws_len,
        _stream_ptr(stream)), "paged_attention_decode_shared")
    return out


def prefill_workspace_bytes(num_seqs: int, num_query_tokens: int, max_query_len: int,
                            num_heads: int, num_kv_heads: int, head_dim: int,
                            max_blocks_per_seq: int, partition_size: int = 0,
                            block_size: int = BLOCK_SIZE) -> int:
    return lib().paged_attention_prefill_workspace_bytes(
        num_seqs, num_query_tokens, max_query_len, num_heads, num_kv_heads, head_dim,
        max_blocks_per_seq, block_size, partition_size)


def paged_attention_prefill(query, cache: PagedKVCache, block_tables, seq_lens, query_offsets,
                            scale: float, max_query_len: int, out=None, out_dtype=None,
                            partition_size: int = 0, workspace=None, stream=None):
    """Multi-token queries (prefill / chunked prefill): query rows
    query_offsets[s] .. query_offsets[s+1]-1 are the last tokens of sequence
    s (already in the cache) and attend causally over its cached tokens."""
    torch = _torch()
    T, H, D = query.shape
    if query.dtype != torch.float16:
        raise ValueError("query must be float16")
    S = block_tables.shape[0]
    if block_tables.dim() != 2 or seq_lens.numel() < S or query_offsets.numel() < S + 1:
        raise ValueError("block_tables [S, max_blocks], seq_lens [S], query_offsets [S+1]")
    maxb = block_tables.shape[1]
    if out is None:
        odt = out_dtype if out_dtype is not None else torch.float16
        out = torch.empty((T, H, D), dtype=odt, device=query.device)
    o_dt = {torch.float32: F32, torch.float16: F16}.get(out.dtype)
    if o_dt is None or tuple(out.shape) != (T, H, D):
        raise ValueError("out must be float32/float16 [num_query_tokens, num_heads, head_dim]")
    if D != cache.head_dim or H % cache.num_kv_heads:
        raise ValueError("query shape does not match the cache")
    need = prefill_workspace_bytes(S, T, max_query_len, H, cache.num_kv_heads, D, maxb,
                                   partition_size, cache.block_size)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr, ws_len = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", numel=need)
        ws_len = workspace.numel() * workspace.element_size()
    nbytes = cache_bytes(cache.num_blocks, cache.num_kv_heads, D, cache.cache_dtype,
                         cache.block_size)
    ks, vs = cache._scales()
    _check(lib().paged_attention_prefill(
        _dev(out, "out"), o_dt, _dev(query, "query"), F16,
        _dev(cache.k, "k_cache", numel=nbytes), _dev(cache.v, "v_cache", numel=nbytes), ks, vs,
        cache.cache_dtype, cache.num_blocks,
        _dev(block_tables, "block_tables", torch.int32, S * maxb), maxb,
        _dev(seq_lens, "seq_lens", torch.int32, S),
        _dev(query_offsets, "query_offsets", torch.int32, S + 1), S, T, int(max_query_len), H,
        cache.num_kv_heads, D, cache.block_size, float(scale), partition_size, ws_ptr, ws_len,
        _stream_ptr(stream)), "paged_attention_prefill")
    return out
