"""GPU parity of the stream walk, the library's choice for tables of several
partitions: the batch's 16-token tiles, in (sequence, kv head, tile) order,
dealt to the GPU's waves in equal shares of whole blocks; the pieces of a
(sequence, kv head) split between shares merged by the log-sum-exp reduction
("partial accumulate, then merge", "vLLM PagedAttention deep dive", jsqmd.com,
section 4.1); a wave's outputs other than its last staged in LDS.

The cases stress the share arithmetic: empty sequences at the start, in the
middle and at the end (no wave visits them, the merge writes their zero
rows); lengths just past tile and block boundaries; 8- and 32-token blocks (a
32-token block whose second tile lies past the length still counts two tiles,
so shares end on block boundaries); groups of 1, 8 and 16 query heads; fp32,
fp16, int8 and E4M3 caches; batches of few units (one workgroup per compute
unit) and of many (two); the fused step with copy-on-write; a batch of only
empty sequences.  Each call is checked to take the stream walk.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads as W  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402

# empty sequences first, between and last; lengths around tile / block edges;
# long ones, so that the table spans several automatic partitions
LENS = [0, 0, 3, 1500, 0, 17, 2049, 33, 0, 900, 4000, 1, 16, 31, 32, 48, 0]


def _lib():
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    return pkv, driver


def _check_stream(w, pkv):
    walk = pkv.decode_walk(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                           w.max_blocks_per_seq, 0, w.block_size)
    assert walk == pkv.WALK_STREAM, f"{w.name}: walk {walk}"


def _decode_case(w):
    pkv, driver = _lib()
    _check_stream(w, pkv)
    w.memo = {}
    say(f"stream walk {w.name}: S={w.num_seqs} H={w.num_heads}/{w.num_kv_heads} "
        f"D={w.head_dim} {w.cache_dtype} bs={w.block_size}")
    ro = oracle_replay(w)
    rg = driver.replay(w)
    torch.cuda.synchronize()
    check_pools_equal(rg.cache, ro.pools, f"{w.name} pools")
    ref = oracle_output(ro, w)
    for rep in range(2):   # a second call over the same workspace
        out = driver.decode(rg, w, partition_size=0)
        torch.cuda.synchronize()
        check_close(out, ref, w.cache_dtype, f"{w.name} call {rep}")
    w.memo = None


@pytest.mark.parametrize("dt", ["f16", "i8", "e4m3"])
@pytest.mark.parametrize("H,Hkv", [(16, 2), (8, 8), (32, 2)])
def test_stream_walk_ragged(dt, H, Hkv):
    _decode_case(W.custom(f"stream_{dt}_{H}_{Hkv}", LENS, H, Hkv, 128, dt, seed=21))


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_stream_walk_block_sizes(bs, dt):
    w = W.with_block_size(W.custom(f"stream_bs_{dt}", LENS, 16, 2, 128, dt, seed=22), bs)
    _decode_case(w)


def test_stream_walk_fp32_head_dim_64():
    w = W.custom("stream_f32_d64", LENS, 8, 2, 64, "f32", out_dtype="f32", seed=23)
    _decode_case(w)


def test_stream_walk_many_units():
    # 48 sequences x 8 kv heads = 384 units: the grid of two workgroups per
    # compute unit
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 2200, 48)
    lens[[0, 7, 47]] = 0
    lens[3] = 2300
    _decode_case(W.custom("stream_many_units", lens.tolist(), 64, 8, 128, "i8", seed=24))


def test_stream_walk_all_empty():
    pkv, driver = _lib()
    w = W.custom("stream_all_empty", [0, 0, 0, 0], 16, 2, 128, "f16", max_blocks=100, seed=25)
    _check_stream(w, pkv)
    ro = oracle_replay(w)
    rg = driver.replay(w)
    out = driver.decode(rg, w, partition_size=0)
    torch.cuda.synchronize()
    assert not bool(out.abs().sum()), "empty sequences: zero rows"
    check_close(out, oracle_output(ro, w), "f16", "all empty")


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_stream_walk_fused_step_copy_on_write(dt):
    """The fused step on a stream batch: forked sequences whose tail block is
    shared copy it first; the new token is written at its slot; pools and
    outputs match the oracle's."""
    pkv, driver = _lib()
    # three children of a 1100-token prefix with no suffix of their own share
    # its partly filled tail block: the step's appends copy it
    w = W.with_decode_step(W.forked_groups(f"stream_step_{dt}", [(1100, 3)],
                                           singles=[1500, 5, 0, 700], suffix_lo=0, suffix_hi=0,
                                           cache_dtype=dt))
    _check_stream(w, pkv)
    w.memo = {}
    say(f"stream walk fused step {w.name}")
    ro = oracle_replay(w)
    rg = driver.replay(w, stop_at_step=True)
    out, slots, pairs, tables, lens = driver.fused_step(rg, w, partition_size=0)
    torch.cuda.synchronize()
    assert np.array_equal(slots, ro.step_slots) and np.array_equal(pairs, ro.step_pairs)
    assert np.array_equal(tables, ro.block_tables) and np.array_equal(lens, ro.seq_lens)
    assert len(pairs) > 0, "the case should copy at least one shared tail block"
    check_pools_equal(rg.cache, ro.pools, f"{w.name} pools after the step")
    check_close(out, oracle_output(ro, w), dt, f"{w.name} fused step")
    w.memo = None
