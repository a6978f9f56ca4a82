"""The oracle's replay of workload scripts, pinned to contiguous attention
computed straight from the generated K/V (which never went through a pool or
an allocator).  CPU only; small sizes."""
import numpy as np
import pytest
import scipy.special

import oracle
from oracle.replay import oracle_output, replay
from synth import workloads


def _contiguous(w, seq, L):
    """Context of `seq` reassembled from the generator, following content ownership."""
    ks, vs = [], []
    pos = 0
    while pos < L:
        owner = w.owner_of(seq, pos)
        end = pos + 1
        while end < L and w.owner_of(seq, end) == owner:
            end += 1
        ks.append(w.kv_rows("k", owner, pos, end - pos))
        vs.append(w.kv_rows("v", owner, pos, end - pos))
        pos = end
    return np.concatenate(ks).astype(np.float64), np.concatenate(vs).astype(np.float64)


def _reference(w, lens):
    q = w.query().astype(np.float64)
    G = w.group
    out = np.zeros(q.shape)
    for i, seq in enumerate(w.decode_seqs):
        if lens[i] == 0:
            continue
        K, V = _contiguous(w, seq, lens[i])
        for h in range(w.num_heads):
            x = np.float64(np.float32(w.scale)) * (K[:, h // G, :] @ q[i, h])
            out[i, h] = scipy.special.softmax(x) @ V[:, h // G, :]
    return out


@pytest.mark.parametrize("make", [
    workloads.c1_tiny,
    lambda: workloads.custom("ragged", [0, 1, 15, 16, 17, 40], 4, 2, 64, "f16", seed=3),
    lambda: workloads.c5_shared_prefix(num_seqs=4, prefix=64, suffix_lo=3, suffix_hi=20,
                                       H=4, Hkv=2, D=64, num_blocks=64),
    lambda: workloads.c5_shared_prefix(num_seqs=6, prefix=40, suffix_lo=1, suffix_hi=9,
                                       cow_pairs=True, H=4, Hkv=1, D=64, num_blocks=64),
])
def test_replay_matches_contiguous_attention(make):
    w = make()
    r = replay(w)
    r.model.check_invariants()
    out = oracle_output(r, w)
    ref = _reference(w, r.seq_lens.tolist())
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_cow_pairs_workload_copies_shared_tails():
    w = workloads.c5_shared_prefix(num_seqs=6, prefix=40, suffix_lo=1, suffix_hi=9,
                                   cow_pairs=True, H=4, Hkv=1, D=64, num_blocks=64)
    r = replay(w)
    n_own = 3
    tails_partial = [(40 + L) % 16 != 0 for L in
                     [r.seq_lens[i] - 1 - 40 for i in range(n_own)]]
    assert len(r.step_pairs) == sum(tails_partial)
    # after the step, no block is shared between a pair's tails
    for i in range(n_own):
        a, b = r.block_tables[i], r.block_tables[i + n_own]
        nb = -(-int(r.seq_lens[i]) // 16)
        assert a[nb - 1] != b[nb - 1]
