"""GPU test of the allocation-free decode entry point
(paged_attention_decode_noalloc), called through the C ABI: on two calls in
a row, the second with a smaller input, its output must equal
paged_attention_decode's (same kernels, same partials) bit for bit, and the
oracle's within the stated tolerance; a call whose partials exceed the fixed
scratch returns PKV_ESCRATCH and enqueues nothing.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads as W  # noqa: E402

from gpu_helpers import check_close, say  # noqa: E402

CALLS = [
    # (name, lens, H, Hkv, cache dtype, partition): split-K with runs, then a
    # smaller ragged batch with other partitions, then the library's choice
    # (equal shares of the batch's tiles, per-unit records in the scratch)
    ("big", [4096] * 8, 64, 8, "f16", 512),
    ("small", [100, 1500, 2999], 16, 2, "f16", 256),
    ("shares", [3000, 17, 0, 1200, 500], 32, 4, "f16", 0),
]


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_noalloc_matches_decode_on_consecutive_calls(dt):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    for name, lens, H, Hkv, _, part in CALLS:
        w = W.custom(f"noalloc_{name}_{dt}", lens, H, Hkv, 128, dt, seed=13,
                     partition_size=part)
        w.memo = {}
        say(f"noalloc {w.name}: S={w.num_seqs} H={H}/{Hkv} partition={part}")
        maxb = w.max_blocks_per_seq
        need = pkv.workspace_bytes(w.num_seqs, H, Hkv, 128, maxb, part, w.block_size)
        assert 0 < need <= pkv.NOALLOC_SCRATCH_BYTES
        ro = oracle_replay(w)
        rg = driver.replay(w)
        ref_gpu = driver.decode(rg, w, partition_size=part)
        out = torch.full_like(ref_gpu, float("nan"))
        pkv.paged_attention_decode_noalloc(rg.query, rg.cache, rg.block_tables, rg.seq_lens,
                                           float(np.float32(w.scale)), out,
                                           partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_gpu), f"{w.name}: differs from paged_attention_decode"
        w.memo = None
        check_close(out, oracle_output(ro, w), dt, f"{w.name} noalloc")


def test_noalloc_rejects_more_than_its_scratch():
    import paged_kv_cache_387_amd as pkv
    pkv.lib()
    # 64 sequences of up to 32K tokens in 16-token partitions: far beyond 32 MiB
    S, H, Hkv, D, maxb = 64, 64, 8, 128, 2048
    assert pkv.workspace_bytes(S, H, Hkv, D, maxb, 16, 16) > pkv.NOALLOC_SCRATCH_BYTES
    cache = pkv.PagedKVCache(64, Hkv, D, "f16")
    q = torch.zeros((S, H, D), dtype=torch.float16, device="cuda")
    out = torch.zeros_like(q)
    tables = torch.zeros((S, maxb), dtype=torch.int32, device="cuda")
    lens = torch.zeros(S, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_noalloc(q, cache, tables, lens, 0.1, out, partition_size=16)
    assert e.value.status == pkv.ESCRATCH
