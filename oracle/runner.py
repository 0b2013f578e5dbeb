"""Replay a workload's pool-operation script on the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The script (new / append / fork / release, then one attention call) is plain
data drawn by the input generators.  This runner executes it with the oracle
allocator and the oracle cache writes, in op order: for every append, the
copy-on-write copies first, then the new tokens' writes -- the order the
copy-on-write description of "19.2 KV Cache 系统化管理" §19.2.2 implies (the new
block receives the old content, then the diverging token).  Unused slots
start as NaN so that any read of them shows up in the outputs.

The workload object is read by attribute only; nothing from the GPU package
is imported.
"""

from __future__ import annotations

import numpy as np

from .allocator import OracleBlockPool
from .kvcache import copy_blocks, kv_write
from .attention import paged_attention, split_partials


def _nan_pool(w):
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    if w.dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, 0x7FC0, dtype=np.uint16)


def replay(w, with_pools: bool = True):
    """Run the script; returns a dict with the pools, tables and the op log."""
    pool = OracleBlockPool(w.num_blocks, w.block_size, initial_free=w.free_order)
    k_pool = _nan_pool(w) if with_pools else None
    v_pool = _nan_pool(w) if with_pools else None
    handles = {}
    row = 0
    log = []  # (script seq, slots, cow pairs) per append
    for op in w.ops:
        kind = op[0]
        if kind == "new":
            handles[op[1]] = pool.new_seq()
        elif kind == "append":
            s, n = op[1], op[2]
            slots, cow = pool.append(handles[s], n)
            if with_pools:
                if cow:
                    copy_blocks(k_pool, v_pool, cow)
                kv_write(k_pool, v_pool, w.k_tokens[row:row + n], w.v_tokens[row:row + n],
                         slots, w.block_size)
            row += n
            log.append((s, slots, cow))
        elif kind == "fork":
            handles[op[2]] = pool.fork(handles[op[1]])
        elif kind == "release":
            pool.release(handles.pop(op[1]))
        else:
            raise ValueError(f"unknown op {kind!r}")
    seqs = [handles[s] for s in w.decode_seqs]
    seq_lens = np.array([pool.seq_len(s) for s in seqs], dtype=np.int32)
    tables = np.array(pool.block_tables(seqs, w.max_blocks, fill=-1), dtype=np.int32)
    return {"pool": pool, "handles": handles, "k_pool": k_pool, "v_pool": v_pool,
            "seq_lens": seq_lens, "block_tables": tables, "log": log}


def attention(w, state, tokens=None):
    """Oracle attention output (float64) of the workload's queries."""
    return paged_attention(w.q, state["k_pool"], state["v_pool"], state["block_tables"],
                           state["seq_lens"], w.scale, w.block_size,
                           cu_q_lens=w.cu_q_lens, tokens=tokens)


def partials(w, state, tokens=None):
    """Oracle split-partition summaries ``(o, lse, nparts)``."""
    return split_partials(w.q, state["k_pool"], state["v_pool"], state["block_tables"],
                          state["seq_lens"], w.scale, w.block_size, w.partition_size,
                          w.max_partitions, cu_q_lens=w.cu_q_lens, tokens=tokens)
