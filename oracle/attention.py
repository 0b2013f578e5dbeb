"""Attention oracle: softmax attention over the keys a block table names.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method ("19.2 KV Cache 系统化管理" §19.2.3, ``paged_attention``) walks the
request's blocks in logical order, takes the first ``min(block_size,
remaining)`` rows of each physical block, and folds the scores into a running
maximum, a running sum of exponentials and a running weighted sum of values;
at the end the weighted sum is divided by the sum.  The page's own check,
``verify_paged_attention`` in the same section, compares that loop with
standard attention over the stacked keys and values, ``softmax(q K^T *
scale) V``.  Up to rounding order the two are the same number, so this
oracle is that plain definition written out in float64: gather the keys and
values through the block table, then one softmax and one weighted sum.

Where the pages are silent, these readings are taken (listed in the design doc):

* Grouped-query attention: query head ``h`` reads KV head ``h // G`` with
  ``G = num_q_heads // num_kv_heads`` (the pages only show one head count).
* ``scale`` is an argument (the pages fix it to ``1/sqrt(head_dim)``; every
  workload here passes that value).
* ``seq_lens[b]`` counts the tokens in the cache *including* this step's new
  tokens: the page appends the token, then attends.
* Several query tokens of one sequence (a chunked-prefill chunk, "LLM 推理引擎
  的内存管理与调度" §8) are its last ``q_len`` tokens; query ``i`` sits at
  position ``len - q_len + i`` and sees keys ``0 .. position``.
* A query that sees no key returns zeros.
* Split-sequence partitions (not on the pages) apply the same running
  max/sum recurrence with one partition as the unit: for a sequence with one
  query token (a decode step), partition ``p`` covers keys
  ``[p*P, min((p+1)*P, key_end))``; every query of a prefill chunk (a
  sequence with several query tokens) has two partitions, keys ``[0, h)``
  and ``[h, key_end)``, split at ``h = 32 * floor(ceil(ctx / 32) / 2)``
  with ``ctx = len - q_len`` the context cached before the chunk, or one
  partition with all its keys when ``h`` is 0.  A partition is summarised by its normalised output and its
  natural-log log-sum-exp of scaled scores; merging the summaries with
  weights ``exp(lse_p - L)``, ``L = log(sum exp(lse_p))``, gives back the
  full softmax.

Storage convention: pools, queries and new tokens are either float arrays or
``uint16`` arrays holding bfloat16 bit patterns; the gathered rows are
widened exactly to float64 before any arithmetic.

Pins (tests/test_oracle_attention.py): agreement with contiguous attention
via ``torch.nn.functional.scaled_dot_product_attention`` on the CPU, with the
pages' block-by-block online loop, closed forms (one key -> that value;
equal keys -> mean of the values; a dominating key -> its value; query
orthogonal to all keys -> mean), the pages' worked example (8 heads, head
dim 32, block size 4, 10 tokens in 3 blocks, error below 1e-5), and for the
partials, ``scipy.special.logsumexp`` and the merge identity.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round values to the nearest bfloat16, ties to even, in one step from
    float64 (bit patterns).  A bfloat16 has 8 significant bits and the float32
    exponent range: a value of binary exponent e is a multiple of
    2^max(e - 7, -133) after rounding (2^-133 is the subnormal step), so it is
    scaled by that power of two, rounded to an integer half-to-even, and
    scaled back; magnitudes that round past the largest finite value
    (3.3895e38) become infinite."""
    v = np.asarray(x, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    finite = np.isfinite(v)
    _, e = np.frexp(np.where(finite, v, 1.0))  # v = m * 2^e, 0.5 <= |m| < 1
    quantum = np.maximum(e - 8, -133)
    r = np.ldexp(np.round(np.ldexp(np.where(finite, v, 0.0), -quantum)), quantum)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact: r is a bfloat16 value (or overflows to inf)
    f = np.where(finite, f, v.astype(np.float32))
    out = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(v)] = np.uint16(0x7FC0)
    return out


def _widen(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def query_positions(seq_lens, cu_q_lens=None):
    """Map every query token to ``(sequence, position)``.

    With ``cu_q_lens`` None every sequence has exactly one query token, its
    last one.  Otherwise sequence ``b`` owns query tokens
    ``cu_q_lens[b] .. cu_q_lens[b+1]-1``, which are its last tokens.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if cu_q_lens is None:
        return [(b, int(seq_lens[b]) - 1) for b in range(seq_lens.shape[0])]
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    out = []
    for b in range(seq_lens.shape[0]):
        q_len = int(cu[b + 1] - cu[b])
        if q_len > int(seq_lens[b]):
            raise ValueError("a sequence has more query tokens than tokens")
        for i in range(q_len):
            out.append((b, int(seq_lens[b]) - q_len + i))
    return out


def gather_kv(k_pool, v_pool, table_row, num_keys: int, block_size: int):
    """Keys and values ``0 .. num_keys-1`` of one request, through its table.

    Returns float64 arrays ``[num_keys, num_kv_heads, head_dim]``.  This is
    the block-table address computation of "LLM 推理引擎的内存管理与调度" §3:
    logical block ``t // block_size`` -> physical block -> in-block offset
    ``t % block_size``.
    """
    t = np.arange(num_keys, dtype=np.int64)
    row = np.asarray(table_row, dtype=np.int64)
    phys = row[t // block_size]
    off = t % block_size
    return _widen(np.asarray(k_pool)[phys, off]), _widen(np.asarray(v_pool)[phys, off])


def _scores(q_j, keys, scale, num_kv_heads):
    """Scaled dot products ``[Hq, num_keys]`` of each query head with its KV head."""
    hq = q_j.shape[0]
    group = hq // num_kv_heads
    kv_of_head = np.arange(hq) // group
    # keys[t, kvh, d]; pick the KV head of every query head -> [Hq, t, d]
    k_for_head = np.transpose(keys[:, kv_of_head, :], (1, 0, 2))
    return scale * np.einsum("hd,htd->ht", q_j, k_for_head), kv_of_head


def paged_attention_query(q_j, k_pool, v_pool, table_row, key_end: int,
                          block_size: int, scale: float):
    """Attention output ``[Hq, D]`` (float64) of one query token over keys ``< key_end``."""
    q_j = _widen(q_j)
    hq, d = q_j.shape
    if key_end <= 0:
        return np.zeros((hq, d), dtype=np.float64)
    keys, vals = gather_kv(k_pool, v_pool, table_row, key_end, block_size)
    num_kv_heads = keys.shape[1]
    s, kv_of_head = _scores(q_j, keys, scale, num_kv_heads)
    s_max = s.max(axis=1, keepdims=True)
    e = np.exp(s - s_max)
    p = e / e.sum(axis=1, keepdims=True)
    v_for_head = np.transpose(vals[:, kv_of_head, :], (1, 0, 2))  # [Hq, t, d]
    return np.einsum("ht,htd->hd", p, v_for_head)


def paged_attention(q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                    block_size: int, cu_q_lens=None, tokens=None):
    """Attention output ``[num_q_tokens, Hq, D]`` (float64) for every query token.

    ``tokens`` optionally restricts the work to a list of query-token indices
    (the other rows are left as NaN), for sampled checks of large cases.
    """
    q = np.asarray(q)
    positions = query_positions(seq_lens, cu_q_lens)
    if len(positions) != q.shape[0]:
        raise ValueError("q has one row per query token")
    out = np.full(q.shape, np.nan, dtype=np.float64)
    tables = np.asarray(block_tables)
    which = range(len(positions)) if tokens is None else tokens
    for j in which:
        b, pos = positions[j]
        out[j] = paged_attention_query(q[j], k_pool, v_pool, tables[b], pos + 1,
                                       block_size, scale)
    return out


def prefill_split(seq_len: int, q_len: int) -> int:
    """Where the keys of a prefill chunk's queries are split: half of the context
    cached before the chunk, in whole 32-key tiles (0: no split)."""
    ctx = seq_len - q_len
    return 32 * (((ctx + 31) // 32) // 2)


def partition_bounds(key_end: int, partition_size: int, seq_len: int = 0, q_len: int = 1):
    """Key ranges ``[(lo, hi), ...]`` of the partitions of a query that sees keys
    ``0 .. key_end - 1``: ``[p*P, min((p+1)*P, key_end))`` for a decode query;
    ``[0, h)`` and ``[h, key_end)`` for a query of a prefill chunk
    (``q_len > 1``, ``h = prefill_split``), or ``[0, key_end)`` when ``h`` is 0."""
    if key_end <= 0:
        return []
    if q_len > 1:
        h = prefill_split(seq_len, q_len)
        return [(0, h), (h, key_end)] if h > 0 else [(0, key_end)]
    return [(lo, min(lo + partition_size, key_end)) for lo in range(0, key_end, partition_size)]


def num_partitions(key_end: int, partition_size: int, seq_len: int = 0, q_len: int = 1) -> int:
    return len(partition_bounds(key_end, partition_size, seq_len, q_len))


def split_partials(q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                   block_size: int, partition_size: int, max_partitions: int,
                   cu_q_lens=None, tokens=None):
    """Per-partition summaries of every query token.

    Returns ``(o, lse, nparts)``: ``o[j, h, p]`` is the softmax-weighted mean
    of the values of partition ``p`` alone, ``lse[j, h, p]`` is
    ``log(sum_t exp(s_t))`` over that partition's scaled scores (natural log),
    ``nparts[j]`` is how many partitions query ``j`` has.  Entries of absent
    partitions are NaN.
    """
    q = np.asarray(q)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    positions = query_positions(seq_lens, cu_q_lens)
    if cu_q_lens is None:
        q_lens = np.ones(len(seq_lens), dtype=np.int64)
    else:
        q_lens = np.diff(np.asarray(cu_q_lens, dtype=np.int64))
    nq, hq, d = q.shape
    o = np.full((nq, hq, max_partitions, d), np.nan)
    lse = np.full((nq, hq, max_partitions), np.nan)
    nparts = np.zeros(nq, dtype=np.int64)
    tables = np.asarray(block_tables)
    which = range(nq) if tokens is None else tokens
    for j in which:
        b, pos = positions[j]
        key_end = pos + 1
        bounds = partition_bounds(key_end, partition_size, int(seq_lens[b]), int(q_lens[b]))
        n = len(bounds)
        if n > max_partitions:
            raise ValueError("max_partitions too small")
        nparts[j] = n
        if n == 0:
            continue
        q_j = _widen(q[j])
        keys, vals = gather_kv(k_pool, v_pool, tables[b], key_end, block_size)
        s, kv_of_head = _scores(q_j, keys, scale, keys.shape[1])
        v_for_head = np.transpose(vals[:, kv_of_head, :], (1, 0, 2))
        for p, (lo, hi) in enumerate(bounds):
            sp = s[:, lo:hi]
            m = sp.max(axis=1, keepdims=True)
            e = np.exp(sp - m)
            tot = e.sum(axis=1)
            lse[j, :, p] = m[:, 0] + np.log(tot)
            o[j, :, p] = np.einsum("ht,htd->hd", e / tot[:, None], v_for_head[:, lo:hi])
    return o, lse, nparts


def merge_partials(o, lse, nparts):
    """Log-sum-exp merge of per-partition summaries -> ``(out, lse_total)``."""
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    nq, hq, _, d = o.shape
    out = np.zeros((nq, hq, d))
    total = np.full((nq, hq), -np.inf)
    for j in range(nq):
        n = int(nparts[j])
        if n == 0:
            continue
        l_j = lse[j, :, :n]
        m = l_j.max(axis=1, keepdims=True)
        w = np.exp(l_j - m)
        tot = w.sum(axis=1)
        total[j] = m[:, 0] + np.log(tot)
        out[j] = np.einsum("hp,hpd->hd", w / tot[:, None], o[j, :, :n])
    return out, total
