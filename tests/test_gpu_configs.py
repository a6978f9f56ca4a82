"""GPU parity at the five workload configurations' full sizes.

Each configuration is replayed by both sides (allocator, copy-on-write, cache
writes); block tables and pool bytes must be identical and every decode output
is compared with the oracle's (which computes all of them: the largest case
takes a few seconds on the host cores).  The decode runs in the launch
configuration the benchmark times (the workload's partition size) and with the
library's automatic choice.
"""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402

CONFIGS = ["c1", "c2", "c3", "c4_i8", "c4_e4m3", "c5", "c5_cow"]


@pytest.mark.parametrize("name", CONFIGS)
def test_config_full_size(name):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = workloads.CONFIGS[name]()
    w.memo = {}
    t0 = time.time()
    say(f"config {name}: S={w.num_seqs} H={w.num_heads}/{w.num_kv_heads} D={w.head_dim} "
        f"{w.cache_dtype} pool={w.num_blocks}")
    ro = oracle_replay(w)
    say(f"  oracle replay {time.time() - t0:.1f}s")
    rg = driver.replay(w)
    torch.cuda.synchronize()
    say(f"  gpu replay {time.time() - t0:.1f}s  tokens={int(ro.seq_lens.sum())} "
        f"cow_pairs={len(ro.step_pairs)}")
    assert np.array_equal(rg.tables_host, ro.block_tables)
    assert np.array_equal(rg.lens_host, ro.seq_lens)
    assert np.array_equal(rg.step_slots, ro.step_slots)
    assert np.array_equal(rg.step_pairs, ro.step_pairs)
    check_pools_equal(rg.cache, ro.pools, name)
    w.memo = None
    ref = oracle_output(ro, w)
    say(f"  oracle decode done {time.time() - t0:.1f}s")
    for ps in sorted({w.partition_size, 0}):
        out = driver.decode(rg, w, partition_size=ps)
        torch.cuda.synchronize()
        check_close(out, ref, w.cache_dtype, f"{name} partition={ps}")
    if name == "c5_cow":
        assert len(ro.step_pairs) > 0
