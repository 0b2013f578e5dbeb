"""Independent reference computations used to pin the oracle (CPU only).

Nothing here imports the oracle or the GPU package.  Each helper reaches the
expected value by a route other than the oracle's own:

* ``sequence_rows``: which token rows of a workload belong to each sequence,
  read straight off the op script (bookkeeping, no allocator),
* ``widen``: bfloat16 bit patterns -> float64 through ``torch``'s own dtype,
* ``sdpa``: ``torch.nn.functional.scaled_dot_product_attention`` in float64
  on contiguous (unpaged) keys and values, with an explicit mask,
* ``chunked_lse_merge``: softmax attention assembled from key chunks cut at
  arbitrary positions and combined with the log-sum-exp identity -- the
  property the running max / running sum of "19.2 KV Cache 系统化管理"
  §19.2.3 rests on, checked without following that loop.
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


def chunked_lse_merge(q, k, v, scale, cuts):
    """Softmax attention of one query, assembled from key chunks.

    ``q`` [H, D], ``k``/``v`` [n, H, D] (equal head counts).  The keys are cut
    at the sorted positions ``cuts`` (any positions, not block boundaries);
    each chunk c is summarised on its own by its log-sum-exp
    ``L_c = log sum_t exp(s_t)`` and its normalised weighted sum ``o_c``, and
    the chunks are combined with the identity
    ``softmax(s) . V = sum_c exp(L_c - L) o_c`` with ``L = log sum_c exp(L_c)``
    (scipy's logsumexp).  Returns [H, D].
    """
    import scipy.special

    n = k.shape[0]
    edges = [0] + sorted(int(c) for c in cuts if 0 < c < n) + [n]
    lse, outs = [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        if lo == hi:
            continue
        s = np.einsum("hd,thd->ht", q, k[lo:hi]) * scale
        lc = scipy.special.logsumexp(s, axis=1)
        lse.append(lc)
        outs.append(np.einsum("ht,thd->hd", np.exp(s - lc[:, None]), v[lo:hi]))
    lse = np.stack(lse)            # [chunks, H]
    total = scipy.special.logsumexp(lse, axis=0)
    w = np.exp(lse - total[None])  # [chunks, H]
    return np.einsum("ch,chd->hd", w, np.stack(outs))
