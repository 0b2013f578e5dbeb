"""Drive a workload's pool-operation script through libpa on the GPU.

The host block pool (C++) turns every append into slots and copy-on-write
pairs; the device work is batched: consecutive appends become one
``pa_kv_write``, and a batch is flushed before any ``pa_copy_blocks`` (the
copied block must hold every earlier token) and before any release (a freed
block may be handed out again).  Copies run before the writes that follow
them on the same stream, the order copy-on-write needs ("19.2 KV Cache
系统化管理" §19.2.2: the new block receives the old content, then the
diverging token).
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array (float32, or uint16 bfloat16 bits) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    bits = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return bits.to(device).view(torch.bfloat16)


def to_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage array (float32, or uint16 bfloat16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def empty_pools(w, device, poison: bool = True):
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    dt = TORCH_DTYPES[w.dtype]
    k = torch.empty(shape, dtype=dt, device=device)
    v = torch.empty(shape, dtype=dt, device=device)
    if poison:
        k.fill_(float("nan"))
        v.fill_(float("nan"))
    return k, v


def replay(w, device, poison: bool = True, tokens_on_device=None):
    """Run the script; returns the pool, device pools, tables and the op log."""
    pool = binding.BlockPool(w.num_blocks, w.block_size, w.free_order)
    k_pool, v_pool = empty_pools(w, device, poison)
    if tokens_on_device is None:
        k_tok = to_device(w.k_tokens, w.dtype, device)
        v_tok = to_device(w.v_tokens, w.dtype, device)
    else:
        k_tok, v_tok = tokens_on_device
    handles = {}
    log = []
    row = 0
    pend_start = 0
    pend_slots = []

    def flush():
        nonlocal pend_start, pend_slots
        if pend_slots:
            slots = torch.from_numpy(np.concatenate(pend_slots)).to(device)
            binding.kv_write(k_pool, v_pool, k_tok[pend_start:row], v_tok[pend_start:row], slots)
        pend_start = row
        pend_slots = []

    for op in w.ops:
        kind = op[0]
        if kind == "new":
            handles[op[1]] = pool.new_seq()
        elif kind == "append":
            s, n = op[1], op[2]
            slots, cow = pool.append(handles[s], n)
            if cow:
                flush()
                pairs = torch.tensor(cow, dtype=torch.int32).to(device)
                binding.copy_blocks(k_pool, v_pool, pairs)
            pend_slots.append(slots)
            row += n
            log.append((s, slots.tolist(), cow))
        elif kind == "fork":
            handles[op[2]] = pool.fork(handles[op[1]])
        elif kind == "release":
            flush()
            pool.release(handles.pop(op[1]))
        else:
            raise ValueError(f"unknown op {kind!r}")
    flush()
    seqs = [handles[s] for s in w.decode_seqs]
    seq_lens = np.array([pool.seq_len(h) for h in seqs], dtype=np.int32)
    tables = pool.block_tables(seqs, w.max_blocks, fill=-1)
    cu = w.cu_q_lens
    return {
        "pool": pool, "handles": handles, "k_pool": k_pool, "v_pool": v_pool,
        "seq_lens_host": seq_lens, "block_tables_host": tables, "log": log,
        "seq_lens": torch.from_numpy(seq_lens).to(device),
        "block_tables": torch.from_numpy(tables).to(device),
        "cu_q_lens": None if cu is None else torch.from_numpy(cu).to(device),
        "q": to_device(w.q, w.dtype, device),
    }


def split_workspace(w, st, partition_size=None):
    """A zeroed split workspace sized for the workload's queries."""
    p = w.partition_size if partition_size is None else partition_size
    maxp = binding.max_partitions_for(w.max_blocks, w.block_size, p, st["cu_q_lens"] is not None)
    q = st["q"]
    return binding.SplitWorkspace(q.shape[0], q.shape[1], q.shape[2], maxp, q.device)


def attention(w, st, partition_size=None, workspace=None, out=None):
    """Split pass + reduce over the workload's queries (device output)."""
    p = w.partition_size if partition_size is None else partition_size
    return binding.paged_attention(st["q"], st["k_pool"], st["v_pool"], st["block_tables"],
                                   st["seq_lens"], w.scale, partition_size=p,
                                   cu_q_lens=st["cu_q_lens"], workspace=workspace, out=out)
