"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers and lays out the structure of the workloads
(shapes, sequence lengths, free-list orders, allocator op scripts and the raw
K/V/q values).  It holds none of the attention, quantization, layout or
allocation arithmetic: each side turns these inputs into pools, tables and
outputs with its own code.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used as a counter-based
generator: draw i of a stream with key k is mix64(k + (i + 1) * GOLDEN).
Normals use the Box-Muller transform (Box and Muller, 1958).
"""
from __future__ import annotations

import zlib

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, *labels) -> np.uint64:
    """Key of an independent stream, derived from the seed and string/int labels."""
    k = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for lab in labels:
            h = zlib.crc32(str(lab).encode()) & 0xFFFFFFFF
            k = _mix64(np.array([k ^ np.uint64(h) ^ (np.uint64(h) << np.uint64(32))],
                                dtype=np.uint64))[0]
    return k


def u64(key: np.uint64, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of stream `key` as uint64."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + idx * GOLDEN)


def uniform01(key, start: int, count: int) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (u64(key, start, count) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def _normal_pairs(key, p0: int, npairs: int) -> np.ndarray:
    """Box-Muller pairs p0 .. p0+npairs-1: pair p uses draws 2p, 2p+1 and yields
    normals 2p (cosine branch) and 2p+1 (sine branch)."""
    raw = u64(key, 2 * p0, 2 * npairs).reshape(npairs, 2)
    u1 = ((raw[:, 0] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53  # (0, 1]
    ang = (raw[:, 1] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53 * 2.0 * np.pi)
    rad = np.sqrt(-2.0 * np.log(u1))
    out = np.empty((npairs, 2), np.float64)
    np.multiply(rad, np.cos(ang), out=out[:, 0])
    np.multiply(rad, np.sin(ang), out=out[:, 1])
    return out.reshape(-1)


_CHUNK_PAIRS = 1 << 21


def normal(key, start: int, count: int) -> np.ndarray:
    """Standard normals start .. start+count-1 of stream `key`."""
    if count <= 0:
        return np.empty(0, np.float64)
    p0, p1 = start // 2, (start + count + 1) // 2
    npairs = p1 - p0
    if npairs <= _CHUNK_PAIRS:
        z = _normal_pairs(key, p0, npairs)
    else:  # independent chunks of a counter-based stream: same values, several threads
        from concurrent.futures import ThreadPoolExecutor
        bounds = list(range(p0, p1, _CHUNK_PAIRS)) + [p1]
        with ThreadPoolExecutor(max_workers=8) as ex:
            parts = list(ex.map(lambda ab: _normal_pairs(key, ab[0], ab[1] - ab[0]),
                                zip(bounds[:-1], bounds[1:])))
        z = np.concatenate(parts)
    off = start - 2 * p0
    return z[off:off + count]


def randint(key, start: int, count: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi] (inclusive)."""
    u = uniform01(key, start, count)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


def permutation(key, n: int) -> np.ndarray:
    """A uniformly random permutation of 0..n-1 (sort by random 64-bit keys)."""
    return np.argsort(u64(key, 0, n), kind="stable").astype(np.int32)
