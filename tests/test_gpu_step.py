"""GPU parity of the fused decode step (paged_decode_step): copy-on-write of
the tail block, the new token's write and the decode in one launch must give
the oracle's pools bit for bit and its outputs within tolerance -- the same
results as the separate copy, write and decode entry points."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle.replay import oracle_output, replay as oracle_replay  # noqa: E402
from synth import workloads  # noqa: E402

from gpu_helpers import check_close, check_pools_equal, say  # noqa: E402


def _ragged(cache_dt, D=128, H=16, Hkv=2, lens=(1, 15, 16, 17, 31, 33, 100, 255, 256, 257),
            seed=3):
    return lambda: workloads.with_decode_step(
        workloads.custom(f"step_{cache_dt}_{D}_{H}_{Hkv}", list(lens), H, Hkv, D, cache_dt,
                         seed=seed, out_dtype="f32" if cache_dt == "f32" else "f16"))


STEP_CASES = {
    "f16_d128_g8": _ragged("f16"),
    "f32_d64_g4": _ragged("f32", D=64, H=8, Hkv=2),
    "i8_d128_g8": _ragged("i8"),
    "e4m3_d128_g8": _ragged("e4m3"),
    "e4m3_d64_g4": _ragged("e4m3", D=64, H=8, Hkv=2),
    "mha_f16": _ragged("f16", H=4, Hkv=4),
    "long_f16": _ragged("f16", lens=(1500, 2047, 2048), H=8, Hkv=1),
    # the new token lands on every row of its 16-token tile
    "rows_f16": _ragged("f16", lens=tuple(range(16, 32)) + (100,)),
    "rows_i8": _ragged("i8", lens=tuple(range(16, 32)) + (100,)),
    "rows_f32": _ragged("f32", D=64, H=8, Hkv=2, lens=tuple(range(16, 32))),
    "c5_small": lambda: workloads.c5_shared_prefix(num_seqs=6, prefix=160, suffix_lo=5,
                                                   suffix_hi=40, H=16, Hkv=2, D=128,
                                                   num_blocks=96),
    "c5_cow_small": lambda: workloads.c5_shared_prefix(num_seqs=8, prefix=96, suffix_lo=1,
                                                       suffix_hi=30, cow_pairs=True, H=16,
                                                       Hkv=2, D=128, num_blocks=96),
    "c5_cow_i8": lambda: _c5_quant("i8"),
}


def _c5_quant(dt):
    w = workloads.c5_shared_prefix(num_seqs=8, prefix=96, suffix_lo=1, suffix_hi=30,
                                   cow_pairs=True, H=16, Hkv=2, D=128, num_blocks=96)
    w.cache_dtype = dt
    w.name += "_" + dt
    return w


@pytest.mark.parametrize("part", [0, 16, 64])
@pytest.mark.parametrize("name", list(STEP_CASES))
def test_fused_step_matches_oracle(name, part):
    import paged_kv_cache_387_amd as pkv
    import hip_replay as driver
    pkv.lib()
    w = STEP_CASES[name]()
    w.memo = {}
    say(f"fused step {name} partition={part}: S={w.num_seqs} H={w.num_heads}/"
        f"{w.num_kv_heads} D={w.head_dim} {w.cache_dtype}")
    ro = oracle_replay(w)
    rg = driver.replay(w, stop_at_step=True)
    out, slots, pairs, tables, lens = driver.fused_step(rg, w, partition_size=part)
    torch.cuda.synchronize()
    assert np.array_equal(slots, ro.step_slots)
    assert np.array_equal(pairs, ro.step_pairs)
    assert np.array_equal(tables, ro.block_tables)
    assert np.array_equal(lens, ro.seq_lens)
    check_pools_equal(rg.cache, ro.pools, f"{name} pools after the step")
    check_close(out, oracle_output(ro, w), w.cache_dtype, f"{name} partition={part}")
    if name.startswith("c5_cow"):
        assert len(pairs) > 0
