"""CPU oracle for paged attention decode -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  It shares no code with the HIP library
(`paged_kv_cache_387_amd`) and never imports it.

The arithmetic lives in `oracle.c` (fp64, plain loops); this module builds it
with gcc, loads it with ctypes and marshals numpy arrays.  The block
allocator model is in `allocator_model.py` and the replay of a workload script
in `replay.py`.  Every function states the page passage it follows in the C
source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
KIND = {"f32": 0, "f16": 1, "i8": 2, "e4m3": 3}
ELEM_BYTES = {"f32": 4, "f16": 2, "i8": 1, "e4m3": 1}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O3 for x86-64-v3 (AVX2; the built
    library may run on another host than the one that built it), OpenMP, IEEE
    arithmetic: no fast-math, no contraction into FMAs, so the results are the
    same at every optimization level)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v3", "-std=c11", "-fPIC",
                               "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_decode.argtypes = [P, P, P, P, P, P, i32, P, i32, P, i32, i32, i32, i32, i32,
                                 dbl, i32]
        L.orc_decode.restype = i32
        L.orc_write.argtypes = [P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32]
        L.orc_write.restype = i32
        L.orc_copy_blocks.argtypes = [P, P, P, P, i32, P, i32, i32, i32, i32, i32]
        L.orc_copy_blocks.restype = i32
        for name in ("orc_f16_to_f64_n", "orc_f32_to_f16_n", "orc_e4m3_to_f64_n",
                     "orc_f32_to_e4m3_n", "orc_f32_to_i8_n"):
            getattr(L, name).argtypes = [P, P, i64]
            getattr(L, name).restype = None
        L.orc_quantize_rows.argtypes = [P, i64, i32, i32, P, P]
        L.orc_quantize_rows.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- number formats ------------------------------------------------------

def f16_bits_to_f64(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().orc_f16_to_f64_n(_p(bits), _p(out), bits.size)
    return out


def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_p(x), _p(out), x.size)
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    lib().orc_e4m3_to_f64_n(_p(codes), _p(out), codes.size)
    return out


def f32_to_e4m3(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_f32_to_e4m3_n(_p(y), _p(out), y.size)
    return out


def f32_to_i8(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.int8)
    lib().orc_f32_to_i8_n(_p(y), _p(out), y.size)
    return out


def quantize_rows(x, kind: str):
    """Quantize each last-axis row of x (float32): returns (codes uint8, scale bits uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[-1]
    rows = x.size // n
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1], np.uint16)
    lib().orc_quantize_rows(_p(x), rows, n, KIND[kind], _p(codes), _p(scales))
    return codes, scales


# ---- pools ---------------------------------------------------------------

class Pools:
    """Host K/V block pools in the documented byte layout, plus fp16 scales."""

    SENTINEL = 0xFF  # every unwritten byte; 0xFFFF is a NaN in fp16, 0xFFFFFFFF in fp32

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, cache_dtype: str,
                 block_size: int = 16, sentinel: int | None = SENTINEL):
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        self.cache_dtype, self.block_size = cache_dtype, block_size
        nbytes = num_blocks * num_kv_heads * block_size * head_dim * ELEM_BYTES[cache_dtype]
        fill = 0 if sentinel is None else sentinel
        self.k = np.full(nbytes, fill, np.uint8)
        self.v = np.full(nbytes, fill, np.uint8)
        quant = cache_dtype in ("i8", "e4m3")
        ns = num_blocks * num_kv_heads * block_size if quant else 1
        self.k_scale = np.full(ns, 0xFFFF if sentinel is not None else 0, np.uint16)
        self.v_scale = np.full(ns, 0xFFFF if sentinel is not None else 0, np.uint16)


def write(pools: Pools, key, value, slot_mapping) -> int:
    """Cache write of tokens [T, Hkv, D] into their slots (slot < 0: skipped)."""
    key = np.ascontiguousarray(key, dtype=np.float32)       # fp16 -> fp32 is exact
    value = np.ascontiguousarray(value, dtype=np.float32)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = slots.shape[0]
    assert key.shape == value.shape == (T, pools.num_kv_heads, pools.head_dim)
    return lib().orc_write(_p(key), _p(value), _p(slots), T, _p(pools.k), _p(pools.v),
                           _p(pools.k_scale), _p(pools.v_scale), KIND[pools.cache_dtype],
                           pools.num_blocks, pools.num_kv_heads, pools.head_dim,
                           pools.block_size)


def copy_blocks(pools: Pools, pairs) -> int:
    """Copy-on-write: pairs [n][2] of (src, dst) physical blocks."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    return lib().orc_copy_blocks(_p(pools.k), _p(pools.v), _p(pools.k_scale),
                                 _p(pools.v_scale), KIND[pools.cache_dtype], _p(pairs),
                                 pairs.shape[0], pools.num_blocks, pools.num_kv_heads,
                                 pools.head_dim, pools.block_size)


def decode(pools: Pools, q, block_tables, seq_lens, scale: float, num_threads: int = 0):
    """fp64 paged decode attention.  q [S, H, D] (any float dtype, widened exactly);
    returns (out float64 [S, H, D], threads used)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S, H, D = q.shape
    assert D == pools.head_dim and bt.shape[0] == S and lens.shape == (S,)
    out = np.zeros((S, H, D), np.float64)
    used = lib().orc_decode(_p(out), _p(q), _p(pools.k), _p(pools.v), _p(pools.k_scale),
                            _p(pools.v_scale), KIND[pools.cache_dtype], _p(bt), bt.shape[1],
                            _p(lens), S, H, pools.num_kv_heads, D, pools.block_size,
                            float(scale), num_threads)
    if used < 0:
        raise ValueError("oracle decode: invalid shape")
    return out, used


def prefill(pools: Pools, q, block_tables, seq_lens, q_offsets, scale: float,
            num_threads: int = 0):
    """fp64 attention of multi-token queries over the paged cache (prefill and
    chunked prefill: the new tokens' K/V are in the cache already).  Sequence
    s has the q_offsets[s+1] - q_offsets[s] query rows q_offsets[s] ..; they
    are the last of its seq_lens[s] tokens, so query i sits at position
    P = seq_lens[s] - q_len + i.  It attends over tokens 0 .. P: the cached
    context and the new tokens up to itself (causal within the new tokens,
    "KVcache-learning", s01 and s04; the paged layout does not change the
    math, jsqmd.com section 9).  Each query row is therefore one decode row
    over the first P + 1 tokens of its sequence's table.  q [T, H, D];
    returns (out float64 [T, H, D], threads used)."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.asarray(seq_lens, np.int64)
    offs = np.asarray(q_offsets, np.int64)
    S = len(lens)
    assert offs.shape == (S + 1,) and bt.shape[0] == S
    T = int(offs[-1])
    rows = np.empty((T, bt.shape[1]), np.int32)
    rlen = np.empty(T, np.int32)
    for s in range(S):
        n = int(offs[s + 1] - offs[s])
        assert 0 <= n <= lens[s]
        for i in range(n):
            rows[offs[s] + i] = bt[s]
            rlen[offs[s] + i] = lens[s] - n + i + 1
    return decode(pools, q, rows, rlen, scale, num_threads)
