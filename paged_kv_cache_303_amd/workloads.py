"""Seeded synthetic inputs for the paged-KV decode workloads.

This module only draws inputs: pool free-list orders, sequence lengths, the
script of pool operations (new / append / fork / release) and the token
values.  It holds none of the attention, allocator or cache arithmetic, so
the GPU path and the CPU oracle can both be fed from it without sharing any
of the method's code.

Workloads (shapes follow the pages' settings: one decode token per running
request, chunked prefill, parallel sampling from a shared prompt, lengths
that vary from request to request):

* ``worked_example``: the pages' own check ("19.2 KV Cache 系统化管理"
  §19.2.3): 16 blocks of 4 tokens, 8 heads, head dim 32, fp32, 10 tokens
  (3 blocks), one query, scale 1/sqrt(32).  ``table="pages"`` keeps the
  page's ascending free list (blocks 15, 14, 13); ``table="random"`` uses a
  seeded permutation, so the three blocks are random distinct ids.
* ``mha_decode``: batch 32, 40 heads (MHA), head dim 128, block size 16,
  lengths uniform in [128, 2048], 4096-block pool with a shuffled free list.
* ``gqa_decode``: batch 256, 32 query / 8 KV heads, head dim 128, block size
  16, lognormal lengths (median 1024, sigma 1.0, rounded, clipped to
  [16, 8192]), 65536-block pool with a permuted free list; the context is
  written first, then one new token per sequence.
* ``shared_prefix``: 4 prompts of 1024 tokens plus one shared decoded token,
  each forked into 16 samples (the parent is then released, so every shared
  block has reference count 16), then 1..256 divergent decode tokens per
  sample; 32/8 heads, head dim 128, block size 16, 4096 blocks.
* ``long_context``: 8 decode sequences of 32768 tokens and one chunked
  prefill sequence (4096-token context + a 512-token chunk) in one batch;
  block size 32, 32/8 heads, head dim 128, 16384 blocks, 512-token
  partitions.

Every value is drawn from ``numpy.random.Generator(PCG64)`` streams spawned
from one master seed; floats are N(0, 1) in float32 and, for bfloat16
workloads, rounded to nearest-even bfloat16 by ``torch`` and kept as uint16
bit patterns.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass
class Workload:
    """A pool configuration, a script of pool operations and token values.

    ``ops`` is a list of tuples, run in order:

    * ``("new", s)``: start script sequence ``s`` (an int chosen by the
      script; each runner maps it to its own sequence handle);
    * ``("append", s, n)``: append ``n`` tokens to ``s``; their keys/values
      are the next ``n`` rows of ``k_tokens`` / ``v_tokens``;
    * ``("fork", parent, child)``: ``child`` shares every block of ``parent``;
    * ``("release", s)``: free ``s``.

    After the script, attention runs once for the sequences ``decode_seqs``
    (in that order) whose last ``q_lens[i]`` tokens are query tokens; their
    queries are the rows of ``q``.
    """

    name: str
    dtype: str
    num_blocks: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    free_order: np.ndarray
    ops: list
    k_tokens: np.ndarray
    v_tokens: np.ndarray
    q: np.ndarray
    decode_seqs: list
    q_lens: list
    seq_lens: list
    partition_size: int = 512
    info: dict = field(default_factory=dict)

    @property
    def num_q_tokens(self) -> int:
        return int(sum(self.q_lens))

    @property
    def max_blocks(self) -> int:
        return max(1, max(-(-n // self.block_size) for n in self.seq_lens))

    @property
    def max_partitions(self) -> int:
        """Partition slots per query for the split layout: enough for the longest
        table, and two for workloads with prefill chunks."""
        cap = self.max_blocks * self.block_size
        return max(2 if self.cu_q_lens is not None else 1, -(-cap // self.partition_size))

    @property
    def cu_q_lens(self):
        """Prefix sums of ``q_lens``, or None when every sequence has one query."""
        if all(n == 1 for n in self.q_lens):
            return None
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V one pass over every decode sequence reads."""
        esize = 4 if self.dtype == F32 else 2
        return int(sum(self.seq_lens)) * self.num_kv_heads * self.head_dim * 2 * esize


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def _values(rng, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == F32:
        return x
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def nan_bits(dtype: str):
    """A quiet-NaN element of the storage dtype (used to poison unused slots)."""
    return np.float32(np.nan) if dtype == F32 else np.uint16(0x7FC0)


def storage_dtype(dtype: str):
    return np.float32 if dtype == F32 else np.uint16


def _decode_workload(name, dtype, num_blocks, block_size, hq, hkv, d, lens,
                     rng_free, rng_q, rng_k, rng_v, free_order=None,
                     partition_size=512, info=None) -> Workload:
    """Context of ``len - 1`` tokens per sequence, then one new token each."""
    lens = [int(x) for x in lens]
    b = len(lens)
    if free_order is None:
        free_order = rng_free.permutation(num_blocks).astype(np.int32)
    ops = [("new", i) for i in range(b)]
    ops += [("append", i, lens[i] - 1) for i in range(b)]
    ops += [("append", i, 1) for i in range(b)]
    n_tok = sum(lens)
    # Token rows are consumed in op order: all contexts, then the new tokens.
    k_tokens = _values(rng_k, (n_tok, hkv, d), dtype)
    v_tokens = _values(rng_v, (n_tok, hkv, d), dtype)
    q = _values(rng_q, (b, hq, d), dtype)
    return Workload(name=name, dtype=dtype, num_blocks=num_blocks,
                    block_size=block_size, num_q_heads=hq, num_kv_heads=hkv,
                    head_dim=d, scale=1.0 / math.sqrt(d),
                    free_order=np.asarray(free_order, dtype=np.int32), ops=ops,
                    k_tokens=k_tokens, v_tokens=v_tokens, q=q,
                    decode_seqs=list(range(b)), q_lens=[1] * b, seq_lens=lens,
                    partition_size=partition_size, info=dict(info or {}))


def worked_example(seed: int = 0, table: str = "random", dtype: str = F32) -> Workload:
    """The pages' check: 16 blocks x 4 tokens, 8 heads x 32, 10 tokens, one query."""
    rf, rq, rk, rv = _streams(seed, 4)
    free = None if table == "random" else np.arange(16, dtype=np.int32)
    return _decode_workload("worked_example", dtype, 16, 4, 8, 8, 32, [10],
                            rf, rq, rk, rv, free_order=free, partition_size=16,
                            info={"table": table})


def mha_decode(seed: int = 1, batch: int = 32, min_len: int = 128, max_len: int = 2048,
               num_blocks: int = 4096, heads: int = 40, dtype: str = BF16,
               partition_size: int = 512) -> Workload:
    """MHA decode: ``heads`` query = KV heads, head dim 128, block size 16."""
    rf, rl, rq, rk, rv = _streams(seed, 5)
    lens = rl.integers(min_len, max_len + 1, size=batch)
    return _decode_workload("mha_decode", dtype, num_blocks, 16, heads, heads, 128, lens,
                            rf, rq, rk, rv, partition_size=partition_size,
                            info={"len_dist": f"uniform[{min_len},{max_len}]"})


def lognormal_lens(rng, batch: int, median: float, sigma: float, lo: int, hi: int):
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=batch)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def gqa_decode(seed: int = 2, batch: int = 256, median: float = 1024.0, sigma: float = 1.0,
               lo: int = 16, hi: int = 8192, num_blocks: int = 65536, dtype: str = BF16,
               num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
               block_size: int = 16, partition_size: int = 512) -> Workload:
    """GQA decode, the throughput workload: batch 256, 32/8 heads, lognormal lengths."""
    rf, rl, rq, rk, rv = _streams(seed, 5)
    lens = lognormal_lens(rl, batch, median, sigma, lo, hi)
    return _decode_workload("gqa_decode", dtype, num_blocks, block_size, num_q_heads,
                            num_kv_heads, head_dim, lens, rf, rq, rk, rv,
                            partition_size=partition_size,
                            info={"len_dist": f"lognormal(median={median},sigma={sigma})"
                                              f" clip[{lo},{hi}]"})


def shared_prefix(seed: int = 3, prompts: int = 4, prompt_len: int = 1024, samples: int = 16,
                  max_divergent: int = 256, num_blocks: int = 4096, dtype: str = BF16,
                  num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                  block_size: int = 16, partition_size: int = 512) -> Workload:
    """Parallel sampling: fork each prompt into ``samples`` sequences, then diverge.

    Each prompt gets ``prompt_len`` tokens plus one shared decoded token, so
    its tail block is partly filled when it is forked; the parent is
    released after forking.  Sample ``i`` then appends ``d_i ~ U{1..max}``
    tokens, one per round, round by round across all samples in order.
    """
    rf, rd, rq, rk, rv = _streams(seed, 5)
    free = rf.permutation(num_blocks).astype(np.int32)
    ops = []
    n_tok = 0
    parent_ids = list(range(prompts))
    for p in parent_ids:
        ops.append(("new", p))
        ops.append(("append", p, prompt_len + 1))
        n_tok += prompt_len + 1
    children = []
    nxt = prompts
    for p in parent_ids:
        for _ in range(samples):
            ops.append(("fork", p, nxt))
            children.append(nxt)
            nxt += 1
        ops.append(("release", p))
    div = rd.integers(1, max_divergent + 1, size=len(children))
    for t in range(1, int(div.max()) + 1):
        for i, c in enumerate(children):
            if div[i] >= t:
                ops.append(("append", c, 1))
                n_tok += 1
    lens = [prompt_len + 1 + int(x) for x in div]
    k_tokens = _values(rk, (n_tok, num_kv_heads, head_dim), dtype)
    v_tokens = _values(rv, (n_tok, num_kv_heads, head_dim), dtype)
    q = _values(rq, (len(children), num_q_heads, head_dim), dtype)
    return Workload(name="shared_prefix", dtype=dtype, num_blocks=num_blocks,
                    block_size=block_size, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim,
                    scale=1.0 / math.sqrt(head_dim), free_order=free, ops=ops,
                    k_tokens=k_tokens, v_tokens=v_tokens, q=q, decode_seqs=children,
                    q_lens=[1] * len(children), seq_lens=lens,
                    partition_size=partition_size,
                    info={"prompts": prompts, "samples": samples,
                          "divergent": [int(x) for x in div]})


def long_context(seed: int = 4, n_decode: int = 8, decode_len: int = 32768,
                 prefill_ctx: int = 4096, chunk: int = 512, num_blocks: int = 16384,
                 dtype: str = BF16, num_q_heads: int = 32, num_kv_heads: int = 8,
                 head_dim: int = 128, block_size: int = 32,
                 partition_size: int = 512) -> Workload:
    """Long decodes plus one chunked-prefill chunk, attended in one launch.

    Sequences ``0..n_decode-1`` hold ``decode_len`` tokens (context plus one
    new token); the last sequence holds ``prefill_ctx`` context tokens and
    receives a ``chunk``-token prefill chunk whose queries attend causally.
    """
    rf, rq, rk, rv = _streams(seed, 4)
    free = rf.permutation(num_blocks).astype(np.int32)
    b = n_decode + 1
    pre = n_decode
    ctx = [decode_len - 1] * n_decode + [prefill_ctx]
    new = [1] * n_decode + [chunk]
    ops = [("new", i) for i in range(b)]
    ops += [("append", i, ctx[i]) for i in range(b)]
    ops += [("append", i, new[i]) for i in range(b)]
    n_tok = sum(ctx) + sum(new)
    k_tokens = _values(rk, (n_tok, num_kv_heads, head_dim), dtype)
    v_tokens = _values(rv, (n_tok, num_kv_heads, head_dim), dtype)
    q = _values(rq, (sum(new), num_q_heads, head_dim), dtype)
    lens = [c + n for c, n in zip(ctx, new)]
    return Workload(name="long_context", dtype=dtype, num_blocks=num_blocks,
                    block_size=block_size, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim,
                    scale=1.0 / math.sqrt(head_dim), free_order=free, ops=ops,
                    k_tokens=k_tokens, v_tokens=v_tokens, q=q,
                    decode_seqs=list(range(b)), q_lens=new, seq_lens=lens,
                    partition_size=partition_size,
                    info={"prefill_seq": pre, "chunk": chunk, "prefill_ctx": prefill_ctx})


def custom_decode(seed: int, lens, num_blocks: int, block_size: int, num_q_heads: int,
                  num_kv_heads: int, head_dim: int, dtype: str, q_lens=None,
                  partition_size: int = 512, name: str = "custom") -> Workload:
    """A decode/extend batch with explicit lengths (edge cases in the tests).

    Sequence ``b`` gets ``lens[b] - q_lens[b]`` context tokens and then
    ``q_lens[b]`` new tokens (default one), which are its query tokens.
    """
    rf, rq, rk, rv = _streams(seed, 4)
    lens = [int(x) for x in lens]
    q_lens = [1] * len(lens) if q_lens is None else [int(x) for x in q_lens]
    b = len(lens)
    free = rf.permutation(num_blocks).astype(np.int32)
    ops = [("new", i) for i in range(b)]
    ops += [("append", i, lens[i] - q_lens[i]) for i in range(b)]
    ops += [("append", i, q_lens[i]) for i in range(b)]
    n_tok = sum(lens)
    return Workload(name=name, dtype=dtype, num_blocks=num_blocks, block_size=block_size,
                    num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    scale=1.0 / math.sqrt(head_dim), free_order=free, ops=ops,
                    k_tokens=_values(rk, (n_tok, num_kv_heads, head_dim), dtype),
                    v_tokens=_values(rv, (n_tok, num_kv_heads, head_dim), dtype),
                    q=_values(rq, (sum(q_lens), num_q_heads, head_dim), dtype),
                    decode_seqs=list(range(b)), q_lens=q_lens, seq_lens=lens,
                    partition_size=partition_size)
