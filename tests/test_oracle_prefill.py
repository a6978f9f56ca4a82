"""Pins of the oracle's multi-token-query attention (prefill / chunked prefill)
over the paged cache (CPU only).

* A dense causal attention computed as one masked matrix product per head
  (numpy, over contiguous K/V that never went through a pool): query i of a
  chunk of n new tokens at the end of an L-token sequence sees tokens
  0 .. L - n + i ("KVcache-learning", s01 attention formula and s04: a new
  token attends to the cached context and to the earlier new tokens).
* One query token per sequence is exactly the decode.
* The first token of a whole prefill sees only itself: its output is its V.
"""
import numpy as np
import pytest
import scipy.special

import oracle

BS = 16


def _pools_for(rng, lens, Hkv, D, dtype, num_blocks):
    """Contiguous K/V per sequence written through random block tables."""
    perm = rng.permutation(num_blocks)
    tables, KV, used = [], [], 0
    maxb = max(-(-L // BS) for L in lens)
    pools = oracle.Pools(num_blocks, Hkv, D, dtype)
    for L in lens:
        K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        if dtype == "f16":
            K, V = K.astype(np.float16).astype(np.float32), V.astype(np.float16).astype(np.float32)
        nb = -(-L // BS)
        t = np.asarray(perm[used:used + nb], np.int32)
        used += nb
        slots = np.array([t[i // BS] * BS + i % BS for i in range(L)], np.int64)
        oracle.write(pools, K, V, slots)
        tables.append(np.concatenate([t, -np.ones(maxb - nb, np.int32)]))
        KV.append((K, V))
    return pools, np.stack(tables), KV


def _dense_causal(q, K, V, n, scale):
    """softmax(Q K^T * scale + causal mask) V for the n last positions of a
    sequence; q [n, H, D], K/V [L, Hkv, D] -> [n, H, D] (fp64)."""
    L, Hkv, D = K.shape
    H = q.shape[1]
    G = H // Hkv
    pos = np.arange(L - n, L)
    mask = np.where(np.arange(L)[None, :] <= pos[:, None], 0.0, -np.inf)   # [n, L]
    out = np.zeros((n, H, D))
    for h in range(H):
        k = K[:, h // G, :].astype(np.float64)
        v = V[:, h // G, :].astype(np.float64)
        s = scale * (q[:, h, :].astype(np.float64) @ k.T) + mask
        out[:, h, :] = scipy.special.softmax(s, axis=1) @ v
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("lens,chunks", [([35, 40, 101], [5, 40, 1]), ([64, 17], [64, 9])])
def test_equals_dense_causal_attention(dtype, lens, chunks):
    rng = np.random.default_rng(7)
    H, Hkv, D = 8, 2, 32
    pools, tables, KV = _pools_for(rng, lens, Hkv, D, dtype, 32)
    offs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(offs[-1]), H, D)).astype(np.float32)
    scale = 0.17
    out, _ = oracle.prefill(pools, q, tables, np.array(lens, np.int32), offs, scale)
    for s, (K, V) in enumerate(KV):
        ref = _dense_causal(q[offs[s]:offs[s + 1]], K, V, chunks[s], scale)
        np.testing.assert_allclose(out[offs[s]:offs[s + 1]], ref, rtol=1e-11, atol=1e-12)


def test_one_query_token_is_the_decode():
    rng = np.random.default_rng(8)
    lens = [1, 33, 70]
    pools, tables, _ = _pools_for(rng, lens, 2, 16, "f32", 16)
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    a, _ = oracle.prefill(pools, q, tables, np.array(lens, np.int32),
                          np.arange(4, dtype=np.int32), 0.3)
    b, _ = oracle.decode(pools, q, tables, np.array(lens, np.int32), 0.3)
    assert np.array_equal(a, b)


def test_first_token_of_a_prefill_returns_its_v():
    rng = np.random.default_rng(9)
    L = 20
    pools, tables, KV = _pools_for(rng, [L], 1, 16, "f16", 4)
    q = rng.standard_normal((L, 2, 16)).astype(np.float32)
    out, _ = oracle.prefill(pools, q, tables, np.array([L], np.int32),
                            np.array([0, L], np.int32), 0.25)
    V = KV[0][1]
    assert np.array_equal(out[0, 0], V[0, 0].astype(np.float64))
    assert np.array_equal(out[0, 1], V[0, 0].astype(np.float64))
