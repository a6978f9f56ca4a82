"""GPU parity of the shared-prefix decode (paged_attention_decode_shared):
sequences grouped by the blocks they share read each prefix block once per
(group, kv head), and their outputs must equal the oracle's plain attention
over the full tables -- decode only and fused with the step (copy-on-write and
new-token write, pools bit for bit), over several groups, group sizes, GQA
ratios, dtypes, head sizes, block sizes and partitionings, empty suffixes,
and the full-size shared-prefix configurations."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402

W = workloads


def _fg(name, groups, **kw):
    return lambda: W.forked_groups(name, groups, **kw)


CASES = {
    # one group, G = 8, suffixes 1..40
    "one_group": _fg("one_group", [(160, 6)]),
    # three groups (one not block-aligned), kept parents (empty suffixes when
    # decoding only) and unrelated sequences, shuffled
    "mixed": _fg("mixed", [(96, 3), (250, 5), (48, 2)], singles=[1, 17, 300],
                 keep_parents=True),
    # 20 members x 8 heads = 160 query columns: several column blocks
    "big_group": _fg("big_group", [(512, 20)], suffix_lo=0, suffix_hi=70),
    # group of 16 query heads per kv head, and MHA (one head per kv head)
    "g16": _fg("g16", [(128, 5)], H=32, Hkv=2),
    "mha": _fg("mha", [(128, 9)], H=4, Hkv=4),
    # a long prefix over few units: many prefix partitions
    "long_prefix": _fg("long_prefix", [(4096, 4)], H=8, Hkv=1, suffix_hi=300),
    "d64": _fg("d64", [(208, 7)], D=64, H=8, Hkv=2),
    "i8": _fg("i8", [(160, 6), (64, 3)], singles=[40], cache_dtype="i8"),
    "e4m3": _fg("e4m3", [(160, 6), (64, 3)], singles=[40], cache_dtype="e4m3"),
    "e4m3_d64": _fg("e4m3_d64", [(96, 5)], D=64, H=8, Hkv=2, cache_dtype="e4m3"),
    "f32_d64": _fg("f32_d64", [(112, 5), (32, 2)], D=64, H=8, Hkv=2, cache_dtype="f32"),
    "f32_d128": _fg("f32_d128", [(64, 3)], cache_dtype="f32"),
    "bs8": lambda: W.with_block_size(W.forked_groups("bs8", [(168, 5), (40, 2)],
                                                     singles=[9]), 8),
    "bs32": lambda: W.with_block_size(W.forked_groups("bs32", [(200, 5), (64, 3)],
                                                      singles=[70]), 32),
    "bs32_i8": lambda: W.with_block_size(W.forked_groups("bs32_i8", [(256, 4)],
                                                         cache_dtype="i8"), 32),
    "c5_small": lambda: W.c5_shared_prefix(num_seqs=6, prefix=160, suffix_lo=5, suffix_hi=40,
                                           H=16, Hkv=2, D=128, num_blocks=96),
    "c5_cow_small": lambda: W.c5_shared_prefix(num_seqs=8, prefix=96, suffix_lo=1,
                                               suffix_hi=30, cow_pairs=True, H=16, Hkv=2,
                                               D=128, num_blocks=96),
}


def _run(name, step, part, min_prefix=0, scale=None):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = CASES[name]()
    if step and not any(op[0] == "step" for op in w.ops):
        w = W.with_decode_step(w)
    if scale is not None:
        w.scale = scale
    w.memo = {}
    if part == "min":   # the smallest partition: one tile, or one block if larger
        part = max(16, w.block_size)
    say(f"shared {name} step={step} partition={part}: S={w.num_seqs} H={w.num_heads}/"
        f"{w.num_kv_heads} D={w.head_dim} {w.cache_dtype} bs={w.block_size}")
    ro = oracle_replay(w)
    rg = driver.replay(w, stop_at_step=step)
    out, slots, pairs, sh, tables, lens = driver.shared(rg, w, step, partition_size=part,
                                                        min_prefix_tokens=min_prefix)
    torch.cuda.synchronize()
    assert np.array_equal(tables, ro.block_tables)
    assert np.array_equal(lens, ro.seq_lens)
    if step:
        assert np.array_equal(slots, ro.step_slots)
        assert np.array_equal(pairs, ro.step_pairs)
    check_pools_equal(rg.cache, ro.pools, f"{name} pools")
    check_close(out, oracle_output(ro, w), w.cache_dtype,
                f"{name} step={step} partition={part} groups={sh['num_groups']}")
    return sh


# 64 tokens = 4 tiles: suffix decodes walk runs of partitions
@pytest.mark.parametrize("part", [0, "min", 64])
@pytest.mark.parametrize("step", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_shared_matches_oracle(name, step, part):
    sh = _run(name, step, part)
    assert sh["num_groups"] >= 1


@pytest.mark.parametrize("scale", [-0.07, 0.0])
@pytest.mark.parametrize("name", ["big_group", "i8"])
def test_shared_scale_sign(name, scale):
    """A negative scale (the fp16 prefix pass folds its sign into q) and a
    zero scale (uniform weights), through the suffix, prefix and merge."""
    sh = _run(name, False, 0, scale=scale)
    assert sh["num_groups"] >= 1


def test_no_groups_runs_the_plain_path():
    sh = _run("mixed", True, 0, min_prefix=1 << 20)
    assert sh["num_groups"] == 0


def test_empty_suffixes():
    # kept parents decode only: their whole table is the prefix
    sh = _run("mixed", False, 0)
    assert (sh["suffix_lens"] == 0).any()


@pytest.mark.parametrize("name", ["c5", "c5_cow"])
def test_shared_full_size(name):
    """The shared-prefix configurations at full size (64 sequences forked from
    an 8192-token prefix), fused step, every output against the oracle."""
    import time
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = W.CONFIGS[name]()
    w.memo = {}
    t0 = time.time()
    say(f"shared full size {name}: S={w.num_seqs}")
    ro = oracle_replay(w)
    rg = driver.replay(w, stop_at_step=True)
    out, slots, pairs, sh, tables, lens = driver.shared(rg, w, True)
    torch.cuda.synchronize()
    say(f"  gpu done {time.time() - t0:.1f}s groups={sh['num_groups']} "
        f"prefix={sh['group_prefix_lens'].tolist()}")
    assert sh["num_groups"] == 1 and sh["group_prefix_lens"].tolist() == [8192]
    assert np.array_equal(tables, ro.block_tables) and np.array_equal(lens, ro.seq_lens)
    assert np.array_equal(slots, ro.step_slots) and np.array_equal(pairs, ro.step_pairs)
    check_pools_equal(rg.cache, ro.pools, f"{name} pools")
    w.memo = None
    check_close(out, oracle_output(ro, w), w.cache_dtype, f"{name} shared")
