"""Replay a workload script through the oracle -- TEST INFRASTRUCTURE ONLY.

Runs the allocator op script of a `synth.workloads.Workload` with the
allocator model, applies copy-on-write copies and K/V writes to oracle pools,
and returns everything the oracle's decode needs, plus a log of every
allocator result so tests can compare it with the library's allocator.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import Pools, copy_blocks, decode, prefill, write
from .allocator_model import BlockManagerModel

# positions of sequence ids in each op
_SEQ_FIELDS = {"allocate": (1,), "fork": (1, 2), "free": (1,), "append": (1,), "write": (1,)}


@dataclass
class OracleReplay:
    pools: Pools
    model: BlockManagerModel
    block_tables: np.ndarray      # int32 [S, max_blocks], -1 padding
    seq_lens: np.ndarray          # int32 [S]
    q: np.ndarray
    step_slots: np.ndarray        # int64 slots of the measured step's appends
    step_pairs: np.ndarray        # int32 [n, 2] copy-on-write pairs of the step
    log: list = field(default_factory=list)


def replay(w, sentinel=Pools.SENTINEL, model: BlockManagerModel | None = None,
           pools: Pools | None = None, seq_offset: int = 0,
           stop_at_step: bool = False) -> OracleReplay:
    """Run the script of workload `w`.  `model` / `pools` may be shared between
    several replays (sequence ids are then shifted by `seq_offset`); with
    `stop_at_step` the ops after the ("step",) marker are left out."""
    mgr = model if model is not None else BlockManagerModel(w.num_blocks, w.block_size,
                                                            w.free_order)
    if pools is None:
        pools = Pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype, w.block_size,
                      sentinel=sentinel)
    log, step_slots, step_pairs = [], [], []
    in_step = False
    for op0 in w.ops:
        kind = op0[0]
        if kind == "step":
            if stop_at_step:
                break
            in_step = True
            continue
        # sequence ids shifted; the content owner is looked up unshifted
        op = (kind,) + tuple(x + seq_offset if k in _SEQ_FIELDS.get(kind, ()) else x
                             for k, x in enumerate(op0[1:], start=1))
        if kind == "allocate":
            st, pair = mgr.allocate(op[1], op[2])
            log.append((op, st, pair))
            assert st == "ok", (op, st)
            if pair is not None:
                copy_blocks(pools, [pair])
        elif kind == "fork":
            st = mgr.fork(op[1], op[2])
            log.append((op, st, None))
            assert st == "ok", (op, st)
        elif kind == "free":
            st = mgr.release(op[1])
            log.append((op, st, None))
            assert st == "ok", (op, st)
        elif kind == "append":
            st, slot, pair = mgr.append(op[1])
            log.append((op, st, (slot, pair)))
            assert st == "ok", (op, st)
            if in_step:
                step_slots.append(slot)
                if pair is not None:
                    step_pairs.append(pair)
            if pair is not None:
                copy_blocks(pools, [pair])
        elif kind == "write":
            seq, start, count = op[1], op[2], op[3]
            st, slots = mgr.slots(seq, start, count)
            assert st == "ok", (op, st)
            owner = w.owner_of(seq - seq_offset, start)
            assert owner == w.owner_of(seq - seq_offset, start + count - 1)
            k = w.kv_rows("k", owner, start, count)
            v = w.kv_rows("v", owner, start, count)
            write(pools, k, v, np.asarray(slots, np.int64))
        else:
            raise ValueError(op)
    st, rows, lens = mgr.export([s + seq_offset for s in w.decode_seqs], w.max_blocks_per_seq)
    assert st == "ok"
    return OracleReplay(
        pools=pools, model=mgr, block_tables=np.asarray(rows, np.int32).reshape(
            len(w.decode_seqs), w.max_blocks_per_seq),
        seq_lens=np.asarray(lens, np.int32), q=w.query(),
        step_slots=np.asarray(step_slots, np.int64),
        step_pairs=np.asarray(step_pairs, np.int32).reshape(-1, 2), log=log)


def oracle_output(r: OracleReplay, w, num_threads: int = 0):
    out, used = decode(r.pools, r.q, r.block_tables, r.seq_lens, np.float32(w.scale),
                       num_threads=num_threads)
    return out


def oracle_prefill_output(r: OracleReplay, w, num_threads: int = 0):
    """Multi-token queries of workload w (w.q_lens set) over the replayed cache."""
    out, used = prefill(r.pools, r.q, r.block_tables, r.seq_lens, w.q_offsets(),
                        np.float32(w.scale), num_threads=num_threads)
    return out
