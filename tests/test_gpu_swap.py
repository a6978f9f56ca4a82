"""GPU check of block swapping (pkv_seq_swap_out / swap_in and
paged_swap_blocks): sequences moved to a pinned host pool and back -- with the
device blocks they freed overwritten in between -- hold the same bytes in
their new blocks and decode to the oracle's output for the original state."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads as W  # noqa: E402

from gpu_helpers import check_close, say  # noqa: E402


def _block_view(t, num_blocks):
    return t.view(num_blocks, -1)


@pytest.mark.parametrize("dtype", ["f16", "i8", "e4m3"])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_swap_round_trip(dtype, bs):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = W.forked_groups("swap", [(96, 3), (250, 4)], singles=[1, 17, 300], keep_parents=True,
                        cache_dtype=dtype)
    if bs != 16:
        w = W.with_block_size(w, bs)
    say(f"swap round trip {dtype} bs={bs}: S={w.num_seqs}")
    ro = oracle_replay(w)
    ref = oracle_output(ro, w)
    rg = driver.replay(w)
    torch.cuda.synchronize()
    cache, alloc = rg.cache, rg.alloc
    alloc.set_host_blocks(w.num_blocks)
    host = pkv.HostKVPool(w.num_blocks, cache)
    seqs = list(w.decode_seqs)
    before_k = cache.k.clone()
    tables0, _ = alloc.export_tables(seqs, w.max_blocks_per_seq)
    # out: every decode sequence (shared blocks move once)
    pairs_out = alloc.swap_out(seqs)
    assert all(alloc.on_host(s) for s in seqs)
    pkv.paged_swap_blocks(cache, host, torch.from_numpy(pairs_out).cuda(), to_host=True)
    torch.cuda.synchronize()
    # the device blocks are free now: overwrite them
    freed = torch.from_numpy(pairs_out[:, 0].astype(np.int64)).cuda()
    for t in (cache.k, cache.v):
        _block_view(t, cache.num_blocks)[freed] = 0xAB
    if cache.quantized:
        for t in (cache.k_scale, cache.v_scale):
            t.view(cache.num_blocks, -1)[freed] = float("nan")
    # in again, in another order: the blocks come from the free list
    pairs_in = alloc.swap_in(list(reversed(seqs)))
    pkv.paged_swap_blocks(cache, host, torch.from_numpy(pairs_in).cuda(), to_host=False)
    torch.cuda.synchronize()
    assert len(pairs_in) == len(pairs_out)
    # block bytes moved unchanged: old device block -> host block -> new block
    to_host = {int(b): int(c) for b, c in pairs_out}
    to_dev = {int(c): int(b) for c, b in pairs_in}
    bk_before = _block_view(before_k, cache.num_blocks)
    bk_after = _block_view(cache.k, cache.num_blocks)
    for b_old, c in to_host.items():
        assert torch.equal(bk_after[to_dev[c]], bk_before[b_old]), (b_old, c, to_dev[c])
    tables1, lens1 = alloc.export_tables(seqs, w.max_blocks_per_seq)
    mapped = np.where(tables0 >= 0, np.vectorize(lambda b: to_dev.get(to_host.get(b, -1), -1))(
        tables0), -1)
    assert np.array_equal(tables1, mapped)
    out = pkv.paged_attention_decode(rg.query, cache, torch.from_numpy(tables1).cuda(),
                                     torch.from_numpy(lens1).cuda(), float(np.float32(w.scale)),
                                     out_dtype=torch.float16)
    torch.cuda.synchronize()
    check_close(out, ref, dtype, f"decode after swap round trip {dtype} bs={bs}")
