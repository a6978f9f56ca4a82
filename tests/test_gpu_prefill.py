"""GPU parity of multi-token queries over the paged cache
(paged_attention_prefill: prefill and chunked prefill, causal within the new
tokens) against the oracle, over ragged contexts and chunk lengths, GQA
ratios, dtypes, head sizes, block sizes and partitionings, and at the
benchmark's size on sampled query rows."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle.replay import oracle_prefill_output, replay as oracle_replay  # noqa: E402
from synth import workloads as W  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402


def _cp(name, contexts, chunks, **kw):
    return lambda: W.chunked_prefill(name, contexts, chunks, **kw)


CASES = {
    # ragged: a decode-like query, a whole prefill, partial tiles, long chunks
    "ragged": _cp("ragged", [100, 0, 37, 300, 5], [28, 64, 1, 77, 3], H=16, Hkv=2, D=128),
    "prefill_only": _cp("prefill_only", [0, 0], [129, 40], H=16, Hkv=2, D=128),
    "g16": _cp("g16", [60, 200], [30, 17], H=32, Hkv=2, D=128),
    "mha": _cp("mha", [90, 33], [70, 5], H=4, Hkv=4, D=128),
    "d64": _cp("d64", [64, 130], [50, 9], H=8, Hkv=2, D=64),
    "i8": _cp("i8", [100, 0, 250], [28, 64, 33], H=16, Hkv=2, D=128, cache_dtype="i8"),
    "e4m3": _cp("e4m3", [100, 0, 250], [28, 64, 33], H=16, Hkv=2, D=128, cache_dtype="e4m3"),
    "e4m3_d64": _cp("e4m3_d64", [70, 10], [20, 40], H=8, Hkv=2, D=64, cache_dtype="e4m3"),
    "i8_d64": _cp("i8_d64", [70, 10], [20, 40], H=8, Hkv=2, D=64, cache_dtype="i8"),
    "bs8": lambda: W.with_block_size(W.chunked_prefill("bs8", [100, 7], [28, 50], H=16, Hkv=2),
                                     8),
    "bs32": lambda: W.with_block_size(W.chunked_prefill("bs32", [100, 7], [28, 50], H=16,
                                                        Hkv=2), 32),
    "bs32_e4m3": lambda: W.with_block_size(W.chunked_prefill("bs32_e4m3", [90, 3], [33, 60],
                                                             H=16, Hkv=2, cache_dtype="e4m3"),
                                           32),
}


def _run(name, part, out_dtype=None):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = CASES[name]()
    w.memo = {}
    if part == "min":
        part = max(32, w.block_size)
    say(f"prefill {name} partition={part}: S={w.num_seqs} T={sum(w.q_lens)} H={w.num_heads}/"
        f"{w.num_kv_heads} D={w.head_dim} {w.cache_dtype} bs={w.block_size}")
    ro = oracle_replay(w)
    rg = driver.replay(w)
    torch.cuda.synchronize()
    check_pools_equal(rg.cache, ro.pools, f"{name} pools")
    out = driver.prefill(rg, w, partition_size=part, out_dtype=out_dtype)
    torch.cuda.synchronize()
    check_close(out, oracle_prefill_output(ro, w), w.cache_dtype, f"{name} partition={part}")


@pytest.mark.parametrize("part", [0, "min", 64])
@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name, part):
    _run(name, part)


def test_prefill_f32_output():
    _run("ragged", 0, out_dtype=torch.float32)


@pytest.mark.parametrize("scale", [-0.07, 0.0])
@pytest.mark.parametrize("name", ["ragged", "i8"])
def test_prefill_scale_sign(name, scale):
    """A negative scale (the fp16 pass folds its sign into q) and a zero scale
    (uniform weights over each query's causal prefix)."""
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = CASES[name]()
    w.scale = scale
    w.memo = {}
    say(f"prefill {name} scale={scale}")
    ro = oracle_replay(w)
    rg = driver.replay(w)
    out = driver.prefill(rg, w, partition_size=0)
    torch.cuda.synchronize()
    check_close(out, oracle_prefill_output(ro, w), w.cache_dtype, f"{name} scale={scale}")


def test_prefill_one_token_is_the_decode():
    """One query token per sequence gives paged_attention_decode's output."""
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    w = W.chunked_prefill("decode_like", [1, 63, 200, 511], [1, 1, 1, 1], H=16, Hkv=2, D=128)
    rg = driver.replay(w)
    a = driver.prefill(rg, w)
    b = pkv.paged_attention_decode(rg.query, rg.cache, rg.block_tables, rg.seq_lens,
                                   float(np.float32(w.scale)))
    torch.cuda.synchronize()
    check_close(a, b.double().cpu().numpy(), "f16", "prefill(q_len=1) vs decode")


@pytest.mark.parametrize("cache_dtype", ["f16", "i8", "e4m3"])
def test_prefill_full_size_sampled(cache_dtype):
    """8 sequences of 1536 cached + 512 new tokens (64/8 heads, d 128): the
    benchmark's shape, over each cache dtype it times; 64 query rows checked
    against the oracle."""
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = W.chunked_prefill(cache_dtype=cache_dtype)
    ro = oracle_replay(w)
    rg = driver.replay(w)
    out = driver.prefill(rg, w)
    torch.cuda.synchronize()
    T = sum(w.q_lens)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(T, 64, replace=False))
    offs = w.q_offsets()
    seq_of = np.searchsorted(offs, rows, side="right") - 1
    tables = ro.block_tables[seq_of]
    lens = np.array([ro.seq_lens[s] - w.q_lens[s] + (r - offs[s]) + 1
                     for r, s in zip(rows, seq_of)], np.int32)
    ref, _ = oracle.decode(ro.pools, ro.q[rows], tables, lens, np.float32(w.scale))
    check_close(out[torch.from_numpy(rows).cuda()], ref, cache_dtype,
                f"chunked prefill sampled rows, {cache_dtype} cache")
