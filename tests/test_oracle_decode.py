"""Pins of the oracle's paged decode, cache write and block copy (CPU only).

Each test pins the oracle to something other than itself:
* library routines on contiguous K/V that never went through a pool
  (scipy's softmax + numpy matmul, PyTorch's scaled_dot_product_attention),
* closed forms (one token, two tokens, identical keys, q = 0),
* invariances the pages fix: paging is storage only, so any permutation of
  physical block ids gives the bit-identical result ("vLLM PagedAttention deep
  dive", jsqmd.com, section 9; the block-table indirection of
  "KV Cache and PagedAttention (vllm-musa)", 7yue.com, section 5),
* GQA as MHA with K/V replicated per group (KVcache-learning s11: num_kv_heads
  may be smaller than num_attention_heads),
* brute force in 50-digit arithmetic on tiny inputs,
* the byte layout documented for the library (hand-worked offsets).
"""
import json
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle

BS = 16


def _scatter(rng, L, Hkv, D, num_blocks, dtype="f32", perm=None):
    """Contiguous K, V (float32) of one sequence written into oracle pools
    through a block table drawn from `perm`."""
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    if dtype == "f16":
        K = K.astype(np.float16).astype(np.float32)
        V = V.astype(np.float16).astype(np.float32)
    nb = -(-L // BS)
    if perm is None:
        perm = rng.permutation(num_blocks)
    table = np.asarray(perm[:nb], np.int32)
    slots = np.array([table[t // BS] * BS + t % BS for t in range(L)], np.int64)
    pools = oracle.Pools(num_blocks, Hkv, D, dtype)
    oracle.write(pools, K, V, slots)
    return K, V, table, pools


def _contiguous_reference(q, K, V, scale):
    """softmax(q K^T * scale) V with scipy/numpy, per head group; q [H, D], K/V [L, Hkv, D]."""
    H, D = q.shape
    Hkv = K.shape[1]
    G = H // Hkv
    out = np.zeros((H, D))
    for h in range(H):
        k = K[:, h // G, :].astype(np.float64)
        v = V[:, h // G, :].astype(np.float64)
        w = scipy.special.softmax(scale * (k @ q[h].astype(np.float64)))
        out[h] = w @ v
    return out


@pytest.mark.parametrize("L,H,Hkv,D,dtype", [(1, 4, 2, 64, "f32"), (17, 8, 2, 64, "f32"),
                                              (100, 8, 1, 128, "f16"), (48, 4, 4, 64, "f16"),
                                              (333, 16, 2, 128, "f32")])
def test_equals_contiguous_attention(L, H, Hkv, D, dtype):
    rng = np.random.default_rng(L * 7 + H)
    K, V, table, pools = _scatter(rng, L, Hkv, D, 64, dtype)
    q = rng.standard_normal((1, H, D))
    scale = 1 / np.sqrt(D)
    out, _ = oracle.decode(pools, q, table[None, :], np.array([L]), scale)
    ref = _contiguous_reference(q[0], K, V, scale)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_equals_torch_sdpa_gqa():
    rng = np.random.default_rng(11)
    S, H, Hkv, D = 3, 8, 2, 64
    lens = [5, 40, 77]
    tables, outs_ref = [], []
    pools = oracle.Pools(40, Hkv, D, "f32")
    perm = rng.permutation(40)
    used = 0
    qs = rng.standard_normal((S, H, D))
    for s, L in enumerate(lens):
        nb = -(-L // BS)
        table = perm[used:used + nb]
        used += nb
        K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        slots = np.array([table[t // BS] * BS + t % BS for t in range(L)], np.int64)
        oracle.write(pools, K, V, slots)
        tables.append(np.concatenate([table, -np.ones(7 - nb, int)]))
        qt = torch.from_numpy(qs[s]).view(1, H, 1, D)
        kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        kt = kt.repeat_interleave(H // Hkv, dim=1).contiguous()
        vt = vt.repeat_interleave(H // Hkv, dim=1).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.125)
        outs_ref.append(o.view(H, D).numpy())
    out, _ = oracle.decode(pools, qs, np.array(tables, np.int32), np.array(lens), 0.125)
    np.testing.assert_allclose(out, np.stack(outs_ref), rtol=1e-12, atol=1e-12)


def test_block_permutation_invariance_bit_identical():
    rng = np.random.default_rng(5)
    L, Hkv, D = 150, 2, 64
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, 8, D))
    outs = []
    for seed in range(4):
        perm = np.random.default_rng(100 + seed).permutation(32)
        table = perm[:10].astype(np.int32)
        slots = np.array([table[t // BS] * BS + t % BS for t in range(L)], np.int64)
        pools = oracle.Pools(32, Hkv, D, "f32")
        oracle.write(pools, K, V, slots)
        outs.append(oracle.decode(pools, q, table[None], np.array([L]), 0.125)[0])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("dtype", ["f32", "f16", "i8", "e4m3"])
def test_single_token_returns_v_exactly(dtype):
    rng = np.random.default_rng(9)
    Hkv, D = 2, 128
    K = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    pools = oracle.Pools(8, Hkv, D, dtype)
    oracle.write(pools, K, V, np.array([5 * BS + 0], np.int64))
    q = rng.standard_normal((1, 8, D)) * 10
    out, _ = oracle.decode(pools, q, np.array([[5]], np.int32), np.array([1]), 0.3)
    if dtype == "f32":
        vv = V.astype(np.float64)
    elif dtype == "f16":
        vv = V.astype(np.float16).astype(np.float64)
    else:
        codes, s = oracle.quantize_rows(V, dtype)
        dec = codes.view(np.int8).astype(np.float64) if dtype == "i8" else oracle.e4m3_to_f64(codes)
        vv = dec * s.view(np.float16).astype(np.float64)[..., None]
    for h in range(8):
        assert np.array_equal(out[0, h], vv[0, h // 4])


def test_identical_keys_give_mean_of_v_and_q_zero_too():
    rng = np.random.default_rng(12)
    L, Hkv, D = 45, 1, 64
    k = rng.standard_normal(D).astype(np.float32)
    K = np.broadcast_to(k, (L, Hkv, D)).copy()
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    pools = oracle.Pools(4, Hkv, D, "f32")
    table = np.array([2, 0, 3], np.int32)
    oracle.write(pools, K, V, np.array([table[t // BS] * BS + t % BS for t in range(L)]))
    q = rng.standard_normal((1, 2, D))
    q[0, 1] = 0.0
    out, _ = oracle.decode(pools, q, table[None], np.array([L]), 1.0)
    mean = V[:, 0, :].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, 1], mean, rtol=0, atol=1e-14)


def test_two_token_closed_form():
    rng = np.random.default_rng(13)
    D = 64
    K = rng.standard_normal((2, 1, D)).astype(np.float32)
    V = rng.standard_normal((2, 1, D)).astype(np.float32)
    pools = oracle.Pools(3, 1, D, "f32")
    oracle.write(pools, K, V, np.array([2 * BS + 0, 2 * BS + 1]))
    q = rng.standard_normal((1, 1, D))
    out, _ = oracle.decode(pools, q, np.array([[2]], np.int32), np.array([2]), 0.125)
    x0 = 0.125 * float(q[0, 0] @ K[0, 0].astype(np.float64))
    x1 = 0.125 * float(q[0, 0] @ K[1, 0].astype(np.float64))
    sig = lambda z: 1 / (1 + np.exp(-z))
    ref = sig(x1 - x0) * V[1, 0].astype(np.float64) + sig(x0 - x1) * V[0, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-13, atol=1e-14)


def test_gqa_equals_mha_with_replicated_kv():
    rng = np.random.default_rng(14)
    L, H, Hkv, D, G = 70, 8, 2, 64, 4
    K, V, table, pools = _scatter(rng, L, Hkv, D, 16)
    q = rng.standard_normal((1, H, D))
    gqa, _ = oracle.decode(pools, q, table[None], np.array([L]), 0.125)
    Kr = np.repeat(K, G, axis=1)
    Vr = np.repeat(V, G, axis=1)
    pm = oracle.Pools(16, H, D, "f32")
    oracle.write(pm, Kr, Vr, np.array([table[t // BS] * BS + t % BS for t in range(L)]))
    mha, _ = oracle.decode(pm, q, table[None], np.array([L]), 0.125)
    assert np.array_equal(gqa, mha)


def test_brute_force_50_digits():
    rng = np.random.default_rng(15)
    L, H, Hkv, D = 19, 2, 1, 64
    K, V, table, pools = _scatter(rng, L, Hkv, D, 4)
    q = rng.standard_normal((1, H, D))
    out, _ = oracle.decode(pools, q, table[None], np.array([L]), 0.125)
    mpmath.mp.dps = 50
    for h in range(H):
        xs = [mpmath.mpf(0.125) * mpmath.fsum(mpmath.mpf(float(q[0, h, d])) * mpmath.mpf(float(K[t, 0, d]))
                                            for d in range(D)) for t in range(L)]
        ws = [mpmath.exp(x) for x in xs]
        Z = mpmath.fsum(ws)
        for d in range(0, D, 7):
            exact = mpmath.fsum(w * mpmath.mpf(float(V[t, 0, d])) for t, w in enumerate(ws)) / Z
            assert abs(out[0, h, d] - float(exact)) <= 1e-13


def test_saturated_softmax_no_overflow():
    rng = np.random.default_rng(16)
    L, Hkv, D = 64, 1, 64
    K, V, table, pools = _scatter(rng, L, Hkv, D, 8)
    q = rng.standard_normal((1, 1, D)) * 1000
    out, _ = oracle.decode(pools, q, table[None], np.array([L]), 1.0)
    assert np.all(np.isfinite(out))
    top = np.argmax(K[:, 0, :].astype(np.float64) @ q[0, 0])
    np.testing.assert_allclose(out[0, 0], V[top, 0], rtol=0, atol=1e-12)


def test_zero_length_gives_zeros_and_reads_nothing():
    pools = oracle.Pools(2, 1, 64, "f16")           # every byte is the NaN sentinel
    q = np.ones((2, 4, 64))
    bt = np.array([[-1, -1], [-1, -1]], np.int32)
    out, _ = oracle.decode(pools, q, bt, np.array([0, 0]), 0.125)
    assert np.array_equal(out, np.zeros_like(out))


def test_quantized_pool_equals_contiguous_on_dequantized_values():
    rng = np.random.default_rng(17)
    L, H, Hkv, D = 90, 8, 2, 128
    for kind in ("i8", "e4m3"):
        K = rng.standard_normal((L, Hkv, D)).astype(np.float16).astype(np.float32)
        V = rng.standard_normal((L, Hkv, D)).astype(np.float16).astype(np.float32)
        table = rng.permutation(12)[:6].astype(np.int32)
        pools = oracle.Pools(12, Hkv, D, kind)
        oracle.write(pools, K, V, np.array([table[t // BS] * BS + t % BS for t in range(L)]))
        deq = []
        for X in (K, V):
            c, s = oracle.quantize_rows(X, kind)
            dec = c.view(np.int8).astype(np.float64) if kind == "i8" else oracle.e4m3_to_f64(c)
            deq.append(dec * s.view(np.float16).astype(np.float64)[..., None])
        q = rng.standard_normal((1, H, D))
        out, _ = oracle.decode(pools, q, table[None], np.array([L]), 1 / np.sqrt(D))
        ref = _contiguous_reference(q[0], deq[0], deq[1], 1 / np.sqrt(D))
        np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_layout_offsets_golden(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "layout_offsets.json")))["cases"]
    for c in cases:
        Hkv, D, dt = c["Hkv"], c["D"], c["dtype"]
        bs = c.get("block_size", BS)
        nb = c["slot"] // bs + 2
        pools = oracle.Pools(nb, Hkv, D, dt, block_size=bs, sentinel=None)   # all zero
        K = np.zeros((1, Hkv, D), np.float32)
        V = np.zeros((1, Hkv, D), np.float32)
        # values whose every byte is nonzero in f32 and f16 (1.2345678: 0x3F9E0651 / 0x3CF0)
        K[0, c["kvh"], c["d"]] = 1.2345678
        V[0, c["kvh"], c["d"]] = -2.7182817
        oracle.write(pools, K, V, np.array([c["slot"]], np.int64))
        for arr, pos, val in ((pools.k, c["k_bytes"], 1.2345678), (pools.v, c["v_bytes"], -2.7182817)):
            nz = np.nonzero(arr)[0].tolist()
            assert nz == pos, (c, nz)
            raw = arr[pos].tobytes()
            if dt == "f32":
                assert np.frombuffer(raw, np.float32)[0] == np.float32(val)
            elif dt == "f16":
                assert np.frombuffer(raw, np.float16)[0] == np.float16(val)
            elif dt == "i8":
                assert np.frombuffer(raw, np.int8)[0] == np.sign(val) * 127
            else:   # the amax element maps to +-448: E4M3 code 0x7E with the sign bit
                assert raw[0] == (0x7E | (0x80 if val < 0 else 0))
        if "scale_index" in c:
            assert np.nonzero(pools.k_scale)[0].tolist() == [c["scale_index"]]


def test_copy_blocks_copies_whole_block_all_heads():
    rng = np.random.default_rng(18)
    Hkv, D = 2, 64
    for kind in ("f16", "i8"):
        pools = oracle.Pools(6, Hkv, D, kind)
        K = rng.standard_normal((16, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((16, Hkv, D)).astype(np.float32)
        oracle.write(pools, K, V, np.arange(3 * BS, 4 * BS))
        before = pools.k.copy()
        n = oracle.copy_blocks(pools, [[3, 1], [7, 0]])          # second pair out of range
        assert n == 1
        blk = len(pools.k) // 6
        assert np.array_equal(pools.k[blk:2 * blk], pools.k[3 * blk:4 * blk])
        assert np.array_equal(pools.v[blk:2 * blk], pools.v[3 * blk:4 * blk])
        assert np.array_equal(pools.k[:blk], before[:blk])
        if kind == "i8":
            sb = len(pools.k_scale) // 6
            assert np.array_equal(pools.k_scale[sb:2 * sb], pools.k_scale[3 * sb:4 * sb])


def test_write_skips_negative_and_out_of_range_slots():
    pools = oracle.Pools(2, 1, 64, "f16")
    K = np.ones((3, 1, 64), np.float32)
    n = oracle.write(pools, K, K, np.array([-1, 2 * BS, 5], np.int64))
    assert n == 1
    assert np.count_nonzero(pools.k != 0xFF) == 64 * 2
