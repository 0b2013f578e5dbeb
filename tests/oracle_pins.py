"""Independent reference computations used to pin the oracle (CPU only).

Nothing here imports the oracle or the GPU package.  Each helper reaches the
expected value by a route other than the oracle's own:

* ``sequence_rows``: which token rows of a workload belong to each sequence,
  read straight off the op script (bookkeeping, no allocator),
* ``widen``: bfloat16 bit patterns -> float64 through ``torch``'s own dtype,
* ``sdpa``: ``torch.nn.functional.scaled_dot_product_attention`` in float64
  on contiguous (unpaged) keys and values, with an explicit mask,
* ``online_blocks``: the block-by-block running max / running sum loop of
  "19.2 KV Cache 系统化管理" §19.2.3, restated in NumPy float64.
"""

from __future__ import annotations

import numpy as np
import torch


def widen(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
        return t.double().numpy()
    return a.astype(np.float64)


def sequence_rows(w):
    """Token-row indices of every live script sequence, in token order."""
    rows = {}
    nxt = 0
    for op in w.ops:
        if op[0] == "new":
            rows[op[1]] = []
        elif op[0] == "append":
            rows[op[1]] += list(range(nxt, nxt + op[2]))
            nxt += op[2]
        elif op[0] == "fork":
            rows[op[2]] = list(rows[op[1]])
        elif op[0] == "release":
            rows.pop(op[1])
    return rows


def contiguous_kv(w):
    """Per decode sequence: (K, V) float64 ``[len, Hkv, D]`` in token order."""
    rows = sequence_rows(w)
    k = widen(w.k_tokens)
    v = widen(w.v_tokens)
    return [(k[rows[s]], v[rows[s]]) for s in w.decode_seqs]


def sdpa(q, k, v, scale, causal_offset=None):
    """Library attention on contiguous K/V.

    ``q``: [nq, Hq, D]; ``k``, ``v``: [n, Hkv, D] (float64).  Query ``i`` sees
    keys ``0 .. causal_offset + i`` when ``causal_offset`` is given (bottom
    right aligned), else every key.
    """
    qt = torch.from_numpy(np.ascontiguousarray(q)).permute(1, 0, 2)  # [Hq, nq, D]
    kt = torch.from_numpy(np.ascontiguousarray(k)).permute(1, 0, 2)
    vt = torch.from_numpy(np.ascontiguousarray(v)).permute(1, 0, 2)
    g = qt.shape[0] // kt.shape[0]
    kt = kt.repeat_interleave(g, dim=0).contiguous()
    vt = vt.repeat_interleave(g, dim=0).contiguous()
    mask = None
    if causal_offset is not None:
        nq, n = qt.shape[1], kt.shape[1]
        qi = torch.arange(nq)[:, None]
        kj = torch.arange(n)[None, :]
        mask = kj <= (causal_offset + qi)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt.unsqueeze(0), kt.unsqueeze(0), vt.unsqueeze(0), attn_mask=mask, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def online_blocks(q, k, v, scale, block_size):
    """The pages' online-softmax loop over blocks of contiguous K/V (one query).

    ``q`` [H, D], ``k``/``v`` [n, H, D] with equal head counts (MHA, as on the
    page).  Returns [H, D].
    """
    h, d = q.shape
    running_max = np.full(h, -np.inf)
    running_sum = np.zeros(h)
    acc = np.zeros((h, d))
    n = k.shape[0]
    for start in range(0, n, block_size):
        kb = k[start:start + block_size]
        vb = v[start:start + block_size]
        s = np.einsum("hd,thd->ht", q, kb) * scale
        new_max = np.maximum(running_max, s.max(axis=1))
        rescale = np.exp(running_max - new_max)
        weights = np.exp(s - new_max[:, None])
        running_sum = running_sum * rescale + weights.sum(axis=1)
        acc = acc * rescale[:, None] + np.einsum("ht,thd->hd", weights, vb)
        running_max = new_max
    return acc / running_sum[:, None]
