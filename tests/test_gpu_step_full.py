"""Full-size parity of the fused decode step (paged_decode_step), the call the
benchmark times: copy-on-write, the new token's write and the paged decode
in one launch ("KVcache-learning", s02: append the new token's K/V, then
attend; s05: copy-on-write).

* The Qwen3-32B-shaped layer as the benchmark builds it: eight batches of 32
  sequences (lengths U[512, 768]) replayed into one 12480-block pool, then
  steps in rotation over the batches (two rounds: every batch steps twice).
  Each step's slots, copy pairs, tables and output are checked against the
  oracle, which replays the same batches into one pool of its own; the pools
  must be equal byte for byte after the last step.
* The 8 x 32K-token configuration with its 512-token partitions (runs of
  partitions plus the merge) and with the library's own partitions.
* The quantized configuration (64 lognormal lengths) over int8 and E4M3
  caches.
"""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle.allocator_model import BlockManagerModel  # noqa: E402
from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads as W  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402

OFF = 1 << 24      # sequence-id offset of batch r (as the benchmark uses)


def test_c2_fused_step_rotating_batches():
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    R, rounds = 8, 2
    ws = [W.c2_qwen3_32b_layer(seed_offset=r) for r in range(R)]
    w0 = ws[0]
    pool, bs = 12480, w0.block_size
    maxb = -(-(768 + rounds + 1) // bs)
    t0 = time.time()
    say(f"c2 fused step, {R} batches in one pool of {pool} blocks, {rounds} rounds")
    alloc = pkv.BlockAllocator(pool, bs, w0.free_order)
    cache = pkv.PagedKVCache(pool, w0.num_kv_heads, w0.head_dim, w0.cache_dtype, block_size=bs,
                             fill_byte=0xFF)
    mgr = BlockManagerModel(pool, bs, w0.free_order)
    pools = oracle.Pools(pool, w0.num_kv_heads, w0.head_dim, w0.cache_dtype, bs)
    for r, w in enumerate(ws):
        w.memo = {}
        driver.replay(w, alloc=alloc, cache=cache, seq_offset=r * OFF)
        oracle_replay(w, model=mgr, pools=pools, seq_offset=r * OFF)
        w.memo = None
    torch.cuda.synchronize()
    say(f"  replayed {time.time() - t0:.1f}s")
    ws_bytes = pkv.workspace_bytes(w0.num_seqs, w0.num_heads, w0.num_kv_heads, w0.head_dim,
                                   maxb, 0, bs)
    assert ws_bytes == 0   # one pass per (sequence, kv head), as timed
    scale = float(np.float32(w0.scale))
    for step in range(R * rounds):
        r = step % R
        w = ws[r]
        seqs = [s + r * OFF for s in w.decode_seqs]
        # the library: allocator, then one fused launch
        slots, pairs, src = alloc.append_slots(seqs, with_src=True)
        tables, lens = alloc.export_tables(seqs, maxb)
        pos = lens - 1     # position of each sequence's new token
        k = np.stack([w.kv_rows("k", s, int(p), 1)[0] for s, p in zip(w.decode_seqs, pos)])
        v = np.stack([w.kv_rows("v", s, int(p), 1)[0] for s, p in zip(w.decode_seqs, pos)])
        q = torch.from_numpy(w.query()).cuda()
        out = pkv.paged_decode_step(q, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                    cache, torch.from_numpy(tables).cuda(),
                                    torch.from_numpy(lens).cuda(), scale,
                                    cow_src=torch.from_numpy(src.astype(np.int32)).cuda())
        # the oracle: the model's appends, its copies and writes, then decode
        oslots, opairs = [], []
        for s in seqs:
            st, slot, pair = mgr.append(s)
            assert st == "ok"
            oslots.append(slot)
            if pair is not None:
                opairs.append(pair)
                oracle.copy_blocks(pools, [pair])
        oracle.write(pools, k, v, np.asarray(oslots, np.int64))
        st, rows, olens = mgr.export(seqs, maxb)
        assert st == "ok"
        torch.cuda.synchronize()
        assert np.array_equal(slots, np.asarray(oslots, np.int64)), f"step {step}: slots"
        assert np.array_equal(pairs.reshape(-1, 2), np.asarray(opairs, np.int32).reshape(-1, 2))
        assert np.array_equal(tables, np.asarray(rows, np.int32)), f"step {step}: tables"
        assert np.array_equal(lens, np.asarray(olens, np.int32))
        ref, _ = oracle.decode(pools, w.query(), np.asarray(rows, np.int32),
                               np.asarray(olens, np.int32), np.float32(w.scale))
        check_close(out, ref, w.cache_dtype, f"c2 step {step} (batch {r})")
    check_pools_equal(cache, pools, "c2 pools after the steps")
    say(f"  done {time.time() - t0:.1f}s")


def _full_step(w, parts):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = W.with_decode_step(w)
    w.memo = {}
    t0 = time.time()
    say(f"fused step full size {w.name}: S={w.num_seqs} {w.cache_dtype} pool={w.num_blocks}")
    ro = oracle_replay(w)
    say(f"  oracle replay {time.time() - t0:.1f}s")
    ref = oracle_output(ro, w)
    say(f"  oracle decode {time.time() - t0:.1f}s")
    for ps in parts:
        rg = driver.replay(w, stop_at_step=True)   # the K/V rows drawn once (memo)
        out, slots, pairs, tables, lens = driver.fused_step(rg, w, partition_size=ps)
        torch.cuda.synchronize()
        assert np.array_equal(slots, ro.step_slots)
        assert np.array_equal(pairs, ro.step_pairs)
        assert np.array_equal(tables, ro.block_tables)
        assert np.array_equal(lens, ro.seq_lens)
        check_pools_equal(rg.cache, ro.pools, f"{w.name} pools after the step")
        check_close(out, ref, w.cache_dtype, f"{w.name} fused step partition={ps}")
        del rg, out
        torch.cuda.empty_cache()
    w.memo = None
    say(f"  done {time.time() - t0:.1f}s")


def test_c3_fused_step_full_size():
    _full_step(W.c3_long_context(), [512, 0])


@pytest.mark.parametrize("dt", ["i8", "e4m3"])
def test_c4_fused_step_full_size(dt):
    _full_step(W.c4_quantized(dt), [0])
