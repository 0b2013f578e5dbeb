"""Cache-write and block-copy oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``kv_write`` follows "19.2 KV Cache 系统化管理" §19.2.3, ``write_slot``:
  the key and value of one token are stored at ``pool[block, slot]`` of the
  pools shaped ``[num_blocks, block_size, num_heads, head_dim]``.  Here the
  (block, slot) pair is given flat, ``block * block_size + slot``, and a
  negative slot means "do not write" (a padding token).
* ``copy_blocks`` is the copy step of copy-on-write, §19.2.2 of the same
  page: the new block receives the content of the shared one, keys and
  values alike.

* ``swap_blocks`` is the swap of a preempted request ("LLM 推理引擎的内存管理与
  调度" §9; "19.2 KV Cache 系统化管理" §19.2.6): its blocks move between the
  device pools and pools in CPU memory, ``dst[d] = src[s]`` for each pair.

All are bit copies: they work on arrays of any dtype (bf16 pools are held
as their uint16 bit patterns), so results can be compared bit for bit.
Pins: closed form (a copy), checked elementwise in the tests, plus the
structural guarantee that the allocator never hands out overlapping pairs.
"""

from __future__ import annotations

import numpy as np


def kv_write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
             v_new: np.ndarray, slot_mapping, block_size: int) -> None:
    """In place: ``pool[s // bs, s % bs] = new[t]`` for every token with s >= 0."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if k_new.shape[0] != slots.shape[0] or v_new.shape[0] != slots.shape[0]:
        raise ValueError("one slot per new token")
    for t, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        block, offset = divmod(s, block_size)
        k_pool[block, offset] = k_new[t]
        v_pool[block, offset] = v_new[t]


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs) -> None:
    """In place: ``pool[dst] = pool[src]`` for every ``(src, dst)`` pair."""
    pairs = [(int(s), int(d)) for s, d in pairs]
    dsts = [d for _, d in pairs]
    srcs = {s for s, _ in pairs}
    if len(set(dsts)) != len(dsts) or srcs.intersection(dsts):
        raise ValueError("copy pairs overlap: a destination is repeated or is also a source")
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray,
                pairs) -> None:
    """In place: ``dst[d] = src[s]`` for every ``(s, d)`` pair (two different pools)."""
    pairs = [(int(s), int(d)) for s, d in pairs]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("swap destinations must be distinct")
    for src, dst in pairs:
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]
