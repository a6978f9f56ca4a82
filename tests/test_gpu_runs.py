"""GPU parity of decode over runs of partitions.

With an explicit partition size of whole wave rounds (a multiple of 4 tiles),
one workgroup walks several consecutive partitions of a (sequence, kv head)
and emits one partial per partition; the merge then folds them.  Outputs must
match the oracle for sequences that end at every position relative to the
partition and run boundaries: inside a run's first partition, exactly on a
partition end, one tile into the next, with the run's last partition holding
fewer tiles than there are waves, and across several runs.  Partition sizes
of 4, 8, 12, 20 and 32 tiles give runs of up to 8 partitions (the LDS stage
limit for 8 query heads per kv head), 4 (16 heads per kv head), and longer
ones capped by the sequence's partition count (one head per kv head).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402

LENS = (1, 63, 64, 65, 80, 127, 128, 145, 531, 1024, 1025, 1607, 2075)
PARTS = [64, 128, 192, 320, 512]

CASES = {
    # name: (cache dtype, head_dim, heads, kv heads, block size)
    "f16_d128_g8": ("f16", 128, 16, 2, 16),
    "i8_d128_g8": ("i8", 128, 16, 2, 16),
    "e4m3_d128_g8": ("e4m3", 128, 16, 2, 16),
    "f32_d64_g8": ("f32", 64, 16, 2, 16),
    "f16_d64_g4": ("f16", 64, 8, 2, 16),
    "f16_d128_g16": ("f16", 128, 32, 2, 16),
    "f16_mha": ("f16", 128, 4, 4, 16),
    "f16_bs8": ("f16", 128, 16, 2, 8),
    "i8_bs32": ("i8", 128, 16, 2, 32),
}


def _workload(name, lens=LENS, step=False):
    dt, D, H, Hkv, bs = CASES[name]
    w = workloads.custom(f"runs_{name}", list(lens), H, Hkv, D, dt, seed=11,
                         out_dtype="f32" if dt == "f32" else "f16")
    if bs != 16:
        w = workloads.with_block_size(w, bs)
    if step:
        w = workloads.with_decode_step(w)
    return w


@pytest.mark.parametrize("name", list(CASES))
def test_decode_runs(name):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = _workload(name)
    w.memo = {}
    say(f"runs {name}: S={w.num_seqs} H={w.num_heads}/{w.num_kv_heads} D={w.head_dim} "
        f"{w.cache_dtype} bs={w.block_size}")
    ro = oracle_replay(w)
    rg = driver.replay(w)
    torch.cuda.synchronize()
    assert np.array_equal(rg.tables_host, ro.block_tables)
    check_pools_equal(rg.cache, ro.pools, name)
    ref = oracle_output(ro, w)
    for ps in PARTS:
        if ps % max(16, w.block_size):
            continue
        out = driver.decode(rg, w, partition_size=ps)
        torch.cuda.synchronize()
        check_close(out, ref, w.cache_dtype, f"{name} partition={ps}")


@pytest.mark.parametrize("name", ["f16_d128_g8", "i8_d128_g8", "e4m3_d128_g8", "f16_bs8"])
def test_fused_step_runs(name):
    """The fused step's write-behind token and copy-on-write with the tail tile
    in the last partition of a run."""
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = _workload(name, lens=(1025, 1607, 2075, 64, 65, 127, 531), step=True)
    w.memo = {}
    ro = oracle_replay(w)
    say(f"fused step runs {name}")
    for ps in [64, 192, 512]:
        rg = driver.replay(w, stop_at_step=True)
        out, slots, pairs, tables, lens = driver.fused_step(rg, w, partition_size=ps)
        torch.cuda.synchronize()
        assert np.array_equal(slots, ro.step_slots)
        assert np.array_equal(tables, ro.block_tables)
        check_pools_equal(rg.cache, ro.pools, f"{name} partition={ps} pools")
        check_close(out, oracle_output(ro, w), w.cache_dtype, f"{name} partition={ps}")
