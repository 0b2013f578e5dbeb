"""ctypes binding of libpa.so: the C ABI with the same names, torch for memory.

Argument marshalling only -- every step of the attention path runs in the HIP
kernels of ``libpa.so``; there is no CPU fallback.  Device arrays are torch
tensors on the current HIP device (contiguous, of the dtypes the ABI names),
and device calls are enqueued on ``torch.cuda.current_stream()``.  A non-OK
status raises :class:`PagedAttentionError` (``NoFreeBlocks`` for an exhausted
pool) with the library's message, as the pages' allocator raises a
``RuntimeError`` when no block is left ("19.2 KV Cache 系统化管理" §19.2.3).

The library must be loaded after ``torch`` so that it binds to the HIP
runtime torch already loaded (same soname), and therefore to torch's streams.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_NO_FREE_BLOCKS, PA_ERR_HIP, \
    PA_ERR_NOT_FOUND = range(6)
PA_F32, PA_BF16, PA_FP8 = 0, 1, 2


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class NoFreeBlocks(PagedAttentionError):
    pass


class KVLayout(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_f32 = ctypes.c_float
_LAYOUT = ctypes.POINTER(KVLayout)

_SIGNATURES = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
    "pa_kv_write": (_i32, [_LAYOUT, _p, _p, _p, _p, _p, _i32, _p]),
    "pa_copy_blocks": (_i32, [_LAYOUT, _p, _p, _p, _i32, _p]),
    "pa_decode": (_i32, [_LAYOUT, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _f32, _p,
                         ctypes.c_size_t, _p]),
    "pa_decode_workspace_size": (_i32, [_LAYOUT, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "pa_decode_noalloc": (_i32, [_LAYOUT, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _f32, _p]),
    "pa_kv_write_fp8": (_i32, [_LAYOUT, _p, _p, _p, _p, _p, _p, _p, _i32, _p]),
    "pa_decode_fp8": (_i32, [_LAYOUT, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _f32,
                             _p, ctypes.c_size_t, _p]),
    "pa_copy_blocks_fp8": (_i32, [_LAYOUT, _p, _p, _p, _p, _p, _i32, _p]),
    "pa_swap_blocks": (_i32, [_LAYOUT, _p, _p, _p, _p, _i32, _p, _i32, _p]),
    "pa_split_workspace_layout": (_i32, [_i32, _i32, _i32, _i32, ctypes.c_void_p]),
    "pa_split_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "pa_decode_split": (_i32, [_LAYOUT, _p, ctypes.c_size_t, _i32, _i32, _p, _p, _i32, _p, _p,
                               _p, _i32, _p, _i32, _i32, _f32, _p]),
    "pa_decode_split_fp8": (_i32, [_LAYOUT, _p, ctypes.c_size_t, _i32, _i32, _p, _p, _i32, _p,
                                   _p, _p, _p, _p, _i32, _p, _i32, _i32, _f32, _p]),
    "pa_reduce": (_i32, [_p, _i32, _p, _p, ctypes.c_size_t, _i32, _i32, _p, _p, _i32, _i32, _i32,
                         _i32, _p]),
    "pa_pool_create": (_i32, [_i32, _i32, _pi32, ctypes.POINTER(_p)]),
    "pa_pool_destroy": (None, [_p]),
    "pa_pool_num_free": (_i32, [_p]),
    "pa_pool_refcount": (_i32, [_p, _i32]),
    "pa_pool_free_list": (_i32, [_p, _pi32, _i32, _pi32]),
    "pa_seq_new": (_i32, [_p, _pi32]),
    "pa_seq_fork": (_i32, [_p, _i32, _pi32]),
    "pa_seq_blocks_needed": (_i32, [_p, _i32, _i32, _pi32]),
    "pa_seq_append": (_i32, [_p, _i32, _i32, _pi32, _pi32, _i32, _pi32]),
    "pa_seq_release": (_i32, [_p, _i32]),
    "pa_seq_len": (_i32, [_p, _i32, _pi32]),
    "pa_block_tables": (_i32, [_p, _pi32, _i32, _i32, _i32, _pi32]),
    "pa_prefix_hash": (ctypes.c_uint64, [ctypes.c_uint64, _pi32, _i32, ctypes.c_uint64]),
    "pa_seq_match_prefix": (_i32, [_p, _i32, ctypes.POINTER(ctypes.c_uint64), _i32, _pi32]),
    "pa_seq_register_prefix": (_i32, [_p, _i32, ctypes.POINTER(ctypes.c_uint64), _i32]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = _build.library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m paged_kv_cache_303_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def exported_symbols():
    return list(_SIGNATURES)


def version() -> str:
    return lib().pa_version().decode()


def _check(status: int) -> None:
    if status != PA_OK:
        msg = lib().pa_last_error().decode(errors="replace")
        cls = NoFreeBlocks if status == PA_ERR_NO_FREE_BLOCKS else PagedAttentionError
        raise cls(status, msg)


# --- device calls -------------------------------------------------------------

# fp8 pools hold e4m3 codes: uint8 tensors (or torch's float8_e4m3fn, the same bytes)
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8,
           torch.float8_e4m3fn: PA_FP8}


def _dev(t: torch.Tensor, name: str, dtype=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name, dtype=None):
    return ctypes.c_void_p(0) if t is None else _dev(t, name, dtype)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def layout_of(k_pool: torch.Tensor) -> KVLayout:
    if k_pool.dim() != 4:
        raise ValueError("pools are [num_blocks, block_size, num_kv_heads, head_dim]")
    if k_pool.dtype not in _DTYPES:
        raise TypeError(f"unsupported pool dtype {k_pool.dtype}")
    nb, bs, hkv, d = k_pool.shape
    return KVLayout(nb, bs, hkv, d, _DTYPES[k_pool.dtype])


def _pools(k_pool, v_pool):
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool must have the same shape and dtype")
    return layout_of(k_pool), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool")


def kv_write(k_pool, v_pool, k_new, v_new, slot_mapping) -> None:
    """``pa_kv_write``: pool[slot // bs, slot % bs] = new[t] for slot >= 0."""
    lay, kp, vp = _pools(k_pool, v_pool)
    n = int(slot_mapping.shape[0])
    row = (lay.num_kv_heads, lay.head_dim)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (n, *row):
            raise ValueError(f"{name} must be [num_tokens, num_kv_heads, head_dim]")
    _check(lib().pa_kv_write(ctypes.byref(lay), kp, vp, _dev(k_new, "k_new", k_pool.dtype),
                             _dev(v_new, "v_new", k_pool.dtype),
                             _dev(slot_mapping, "slot_mapping", torch.int32), n, _stream()))


def copy_blocks(k_pool, v_pool, pairs) -> None:
    """``pa_copy_blocks``: pool[dst] = pool[src] for every (src, dst) row of ``pairs``."""
    lay, kp, vp = _pools(k_pool, v_pool)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    _check(lib().pa_copy_blocks(ctypes.byref(lay), kp, vp, _dev(pairs, "pairs", torch.int32),
                                int(pairs.shape[0]), _stream()))


def fp8_scale_shape(k_pool) -> tuple:
    """Shape of the scale pools of an e4m3 code pool ``[NB, bs, Hkv, D]``:
    ``[NB, Hkv, bs]`` (one float32 per block, KV head and row; a head's rows
    contiguous)."""
    nb, bs, hkv = (int(x) for x in k_pool.shape[:3])
    return (nb, hkv, bs)


def _fp8_pools(k_pool, v_pool, k_scale, v_scale):
    lay, kp, vp = _pools(k_pool, v_pool)
    if lay.dtype != PA_FP8:
        raise TypeError("fp8 pools are uint8 (e4m3 codes)")
    shape = fp8_scale_shape(k_pool)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be [num_blocks, num_kv_heads, block_size]")
    return lay, kp, vp, _dev(k_scale, "k_scale", torch.float32), \
        _dev(v_scale, "v_scale", torch.float32)


def kv_write_fp8(k_pool, v_pool, k_scale, v_scale, k_new, v_new, slot_mapping) -> None:
    """``pa_kv_write_fp8``: quantize bf16 rows ``new[t]`` into slot ``slot_mapping[t]``."""
    lay, kp, vp, ks, vs = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    n = int(slot_mapping.shape[0])
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (n, lay.num_kv_heads, lay.head_dim):
            raise ValueError(f"{name} must be [num_tokens, num_kv_heads, head_dim]")
    _check(lib().pa_kv_write_fp8(ctypes.byref(lay), kp, vp, ks, vs,
                                 _dev(k_new, "k_new", torch.bfloat16),
                                 _dev(v_new, "v_new", torch.bfloat16),
                                 _dev(slot_mapping, "slot_mapping", torch.int32), n, _stream()))


def _host_or_dev(t: torch.Tensor, name: str) -> ctypes.c_void_p:
    """Device tensor, or pinned host tensor (the GPU reaches it through the same pointer)."""
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or t.is_pinned()):
        raise TypeError(f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs) -> None:
    """``pa_swap_blocks``: ``dst[d] = src[s]`` for every (s, d) row of ``pairs``.

    Pools are ``[num_blocks, ...block shape]`` device or pinned host tensors of one
    dtype and block shape (swap-out: host destinations; swap-in: host sources);
    a pool of any block shape works (fp8 scale pools included).
    """
    if dst_k.shape != dst_v.shape or src_k.shape != src_v.shape:
        raise ValueError("K and V pools must have the same shape")
    if dst_k.shape[1:] != src_k.shape[1:] or dst_k.dtype != src_k.dtype:
        raise ValueError("source and destination pools must share block shape and dtype")
    if pairs.dim() != 2 or pairs.shape[1] != 2 or pairs.dtype != torch.int32:
        raise ValueError("pairs must be int32 [n, 2]")
    per_block = int(np.prod(dst_k.shape[1:])) if dst_k.dim() > 1 else 1
    dt = _DTYPES.get(dst_k.dtype)
    if dt is None:
        raise TypeError(f"unsupported pool dtype {dst_k.dtype}")
    # the block as rows of one element: only its byte size matters to the copy
    lay = KVLayout(int(dst_k.shape[0]), 1, 1, per_block, dt)
    _check(lib().pa_swap_blocks(ctypes.byref(lay), _host_or_dev(dst_k, "dst_k"),
                                _host_or_dev(dst_v, "dst_v"), _host_or_dev(src_k, "src_k"),
                                _host_or_dev(src_v, "src_v"), int(src_k.shape[0]),
                                _host_or_dev(pairs, "pairs"), int(pairs.shape[0]), _stream()))


def copy_blocks_fp8(k_pool, v_pool, k_scale, v_scale, pairs) -> None:
    """``pa_copy_blocks_fp8``: codes and scales of block src copied to dst."""
    lay, kp, vp, ks, vs = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    _check(lib().pa_copy_blocks_fp8(ctypes.byref(lay), kp, vp, ks, vs,
                                    _dev(pairs, "pairs", torch.int32), int(pairs.shape[0]),
                                    _stream()))


def decode_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, scale: float,
               out=None, workspace=None):
    """``pa_decode_fp8``: decode over e4m3 pools; bf16 ``q`` and output.  Returns ``out``."""
    lay, kp, vp, ks, vs = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    if q.dim() != 3 or q.shape[2] != lay.head_dim:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    b, hq = int(q.shape[0]), int(q.shape[1])
    bt, mb, sl = _tables(block_tables, seq_lens, b)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    ws, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        ws, ws_bytes = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    _check(lib().pa_decode_fp8(ctypes.byref(lay), _dev(out, "out", torch.bfloat16),
                               _dev(q, "q", torch.bfloat16), kp, vp, ks, vs, bt, mb, sl, b, hq,
                               float(scale), ws, ws_bytes, _stream()))
    return out


def _tables(block_tables, seq_lens, num_seqs):
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if tuple(seq_lens.shape) != (num_seqs,):
        raise ValueError("seq_lens must be [num_seqs]")
    return (_dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
            _dev(seq_lens, "seq_lens", torch.int32))


def decode_workspace_size(k_pool, num_seqs: int, num_q_heads: int) -> int:
    """``pa_decode_workspace_size``: bytes of the balanced path's workspace."""
    lay = layout_of(k_pool)
    n = ctypes.c_size_t()
    _check(lib().pa_decode_workspace_size(ctypes.byref(lay), int(num_seqs), int(num_q_heads),
                                          ctypes.byref(n)))
    return n.value


def decode_workspace(k_pool, num_seqs: int, num_q_heads: int):
    """A device workspace for ``decode`` (None when the balanced path does not apply)."""
    n = decode_workspace_size(k_pool, num_seqs, num_q_heads)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=k_pool.device)


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale: float, out=None, workspace=None):
    """``pa_decode``: one query per sequence.  Returns ``out``.

    ``workspace`` (a uint8 device tensor from :func:`decode_workspace`)
    selects the load-balanced path; without it every (sequence, KV-head
    group) is one workgroup.
    """
    lay, kp, vp = _pools(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != lay.head_dim:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    b, hq = int(q.shape[0]), int(q.shape[1])
    bt, mb, sl = _tables(block_tables, seq_lens, b)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    ws = ctypes.c_void_p(0)
    ws_bytes = 0
    if workspace is not None:
        ws = _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    _check(lib().pa_decode(ctypes.byref(lay), _dev(out, "out", k_pool.dtype),
                           _dev(q, "q", k_pool.dtype), kp, vp, bt, mb, sl, b, hq, float(scale),
                           ws, ws_bytes, _stream()))
    return out


def decode_noalloc(q, k_pool, v_pool, block_tables, seq_lens, scale: float, out):
    """``pa_decode_noalloc``: the balanced decode on the library's own scratch
    (``out`` is required: this call allocates nothing)."""
    lay, kp, vp = _pools(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != lay.head_dim:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    if out is None or out.shape != q.shape:
        raise ValueError("out must have q's shape")
    b, hq = int(q.shape[0]), int(q.shape[1])
    bt, mb, sl = _tables(block_tables, seq_lens, b)
    _check(lib().pa_decode_noalloc(ctypes.byref(lay), _dev(out, "out", k_pool.dtype),
                                   _dev(q, "q", k_pool.dtype), kp, vp, bt, mb, sl, b, hq,
                                   float(scale), _stream()))
    return out


def max_partitions_for(max_blocks: int, block_size: int, partition_size: int,
                       prefill: bool = False) -> int:
    """Partitions a split workspace needs: the decode queries' ceil(capacity / P),
    and at least two when prefill chunks (``cu_q_lens``) are present."""
    return max(2 if prefill else 1, -(-(max_blocks * block_size) // partition_size))


class SplitLayout(ctypes.Structure):
    _fields_ = [("part_o_offset", ctypes.c_size_t), ("part_lse_offset", ctypes.c_size_t),
                ("control_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t)]


class SplitWorkspace:
    """Device workspace of the split path, laid out by ``pa_split_workspace_layout``.

    ``part_o`` / ``part_lse`` are views of its partial buffers; the control
    block starts zeroed (the library leaves it zeroed after every call).
    """

    def __init__(self, num_q_tokens: int, num_q_heads: int, head_dim: int,
                 max_partitions: int, device):
        lay = SplitLayout()
        _check(lib().pa_split_workspace_layout(int(num_q_tokens), int(num_q_heads),
                                               int(head_dim), int(max_partitions),
                                               ctypes.byref(lay)))
        self.shape = (int(num_q_tokens), int(num_q_heads), int(max_partitions), int(head_dim))
        self.layout = lay
        self.buffer = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=device)
        n_o = int(np.prod(self.shape))
        self.part_o = self.buffer[lay.part_o_offset:lay.part_o_offset + 4 * n_o] \
            .view(torch.float32).view(self.shape)
        n_l = n_o // self.shape[3]
        self.part_lse = self.buffer[lay.part_lse_offset:lay.part_lse_offset + 4 * n_l] \
            .view(torch.float32).view(self.shape[:3])

    def ptr(self):
        return ctypes.c_void_p(self.buffer.data_ptr()), self.layout.total_bytes


def split_workspace_bytes(num_q_tokens, num_q_heads, head_dim, max_partitions) -> int:
    """``pa_split_workspace_bytes``."""
    return int(lib().pa_split_workspace_bytes(int(num_q_tokens), int(num_q_heads),
                                              int(head_dim), int(max_partitions)))


def _split_args(q, block_tables, seq_lens, cu_q_lens, head_dim):
    if q.dim() != 3 or q.shape[2] != head_dim:
        raise ValueError("q must be [num_q_tokens, num_q_heads, head_dim]")
    b = int(seq_lens.shape[0])
    bt, mb, sl = _tables(block_tables, seq_lens, b)
    if cu_q_lens is not None and tuple(cu_q_lens.shape) != (b + 1,):
        raise ValueError("cu_q_lens must be [num_seqs + 1]")
    return b, bt, mb, sl


def _workspace_for(workspace, q, mb, block_size, partition_size, max_partitions, prefill):
    nq, hq, d = (int(x) for x in q.shape)
    if workspace is None:
        if max_partitions is None:
            max_partitions = max_partitions_for(mb, block_size, partition_size, prefill)
        workspace = SplitWorkspace(nq, hq, d, max_partitions, q.device)
    elif workspace.shape[:2] != (nq, hq) or workspace.shape[3] != d:
        raise ValueError("workspace was made for other sizes")
    return workspace


def decode_split(q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                 partition_size: int = 512, cu_q_lens=None, workspace=None,
                 max_partitions=None) -> SplitWorkspace:
    """``pa_decode_split``: per-partition summaries in a :class:`SplitWorkspace`."""
    lay, kp, vp = _pools(k_pool, v_pool)
    b, bt, mb, sl = _split_args(q, block_tables, seq_lens, cu_q_lens, lay.head_dim)
    ws = _workspace_for(workspace, q, mb, lay.block_size, partition_size, max_partitions,
                        cu_q_lens is not None)
    wp, wn = ws.ptr()
    _check(lib().pa_decode_split(ctypes.byref(lay), wp, wn, ws.shape[2], int(partition_size),
                                 _dev(q, "q", k_pool.dtype),
                                 _opt(cu_q_lens, "cu_q_lens", torch.int32), int(q.shape[0]), kp,
                                 vp, bt, mb, sl, b, int(q.shape[1]), float(scale), _stream()))
    return ws


def decode_split_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, scale: float,
                     partition_size: int = 512, cu_q_lens=None, workspace=None,
                     max_partitions=None) -> SplitWorkspace:
    """``pa_decode_split_fp8``: the split first pass over e4m3 pools (bf16 ``q``)."""
    lay, kp, vp, ks, vs = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    b, bt, mb, sl = _split_args(q, block_tables, seq_lens, cu_q_lens, lay.head_dim)
    ws = _workspace_for(workspace, q, mb, lay.block_size, partition_size, max_partitions,
                        cu_q_lens is not None)
    wp, wn = ws.ptr()
    _check(lib().pa_decode_split_fp8(ctypes.byref(lay), wp, wn, ws.shape[2], int(partition_size),
                                     _dev(q, "q", torch.bfloat16),
                                     _opt(cu_q_lens, "cu_q_lens", torch.int32), int(q.shape[0]),
                                     kp, vp, ks, vs, bt, mb, sl, b, int(q.shape[1]),
                                     float(scale), _stream()))
    return ws


def reduce(workspace: SplitWorkspace, seq_lens, partition_size: int, out_dtype=torch.bfloat16,
           cu_q_lens=None, out=None, lse_out=None):
    """``pa_reduce``: log-sum-exp merge of the partitions.  Returns ``out``."""
    nq, hq, maxp, d = workspace.shape
    b = int(seq_lens.shape[0])
    dev = workspace.buffer.device
    if out is None:
        out = torch.empty((nq, hq, d), dtype=out_dtype, device=dev)
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (nq, hq, d):
        raise ValueError("out must be [num_q_tokens, num_q_heads, head_dim] f32/bf16")
    wp, wn = workspace.ptr()
    _check(lib().pa_reduce(_dev(out, "out"), _DTYPES[out.dtype],
                           _opt(lse_out, "lse_out", torch.float32), wp, wn, maxp,
                           int(partition_size), _opt(cu_q_lens, "cu_q_lens", torch.int32),
                           _dev(seq_lens, "seq_lens", torch.int32), b, nq, hq, d, _stream()))
    return out


def paged_attention(q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                    partition_size: int = 512, cu_q_lens=None, workspace=None, out=None):
    """Split pass + reduce: attention output of every query token."""
    ws = decode_split(q, k_pool, v_pool, block_tables, seq_lens, scale,
                      partition_size=partition_size, cu_q_lens=cu_q_lens, workspace=workspace)
    return reduce(ws, seq_lens, partition_size, out_dtype=q.dtype, cu_q_lens=cu_q_lens, out=out)


def paged_attention_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens,
                        scale: float, partition_size: int = 512, cu_q_lens=None,
                        workspace=None, out=None):
    """Split pass + reduce over e4m3 pools: bf16 output of every query token."""
    ws = decode_split_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, scale,
                          partition_size=partition_size, cu_q_lens=cu_q_lens,
                          workspace=workspace)
    return reduce(ws, seq_lens, partition_size, out_dtype=torch.bfloat16, cu_q_lens=cu_q_lens,
                  out=out)


# --- host block pool ------------------------------------------------------------

def _i32_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr32(a: np.ndarray):
    return a.ctypes.data_as(_pi32)


def prefix_hash(parent: int, tokens, salt: int = 0) -> int:
    """``pa_prefix_hash``: the chained key of one full block."""
    t = _i32_array(tokens)
    return int(lib().pa_prefix_hash(ctypes.c_uint64(int(parent)), _ptr32(t), int(t.shape[0]),
                                    ctypes.c_uint64(int(salt))))


class BlockPool:
    """The library's host block pool (free list, reference counts, tables)."""

    def __init__(self, num_blocks: int, block_size: int, initial_free=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        handle = ctypes.c_void_p()
        free = None if initial_free is None else _i32_array(initial_free)
        if free is not None and free.shape != (self.num_blocks,):
            raise ValueError("initial_free must hold num_blocks ids")
        _check(lib().pa_pool_create(self.num_blocks, self.block_size,
                                    None if free is None else _ptr32(free),
                                    ctypes.byref(handle)))
        self._h = handle

    def close(self):
        if self._h:
            lib().pa_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(lib().pa_pool_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib().pa_pool_refcount(self._h, int(block)))

    def free_list(self) -> list:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_pool_free_list(self._h, _ptr32(out), self.num_blocks, ctypes.byref(n)))
        return out[: n.value].tolist()

    def new_seq(self) -> int:
        s = ctypes.c_int32()
        _check(lib().pa_seq_new(self._h, ctypes.byref(s)))
        return s.value

    def fork(self, parent: int) -> int:
        s = ctypes.c_int32()
        _check(lib().pa_seq_fork(self._h, int(parent), ctypes.byref(s)))
        return s.value

    def match_prefix(self, seq: int, keys) -> int:
        """``pa_seq_match_prefix``: map cached blocks of the key chain; returns the hits."""
        k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
        n = ctypes.c_int32()
        _check(lib().pa_seq_match_prefix(self._h, int(seq),
                                         k.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                         int(k.shape[0]), ctypes.byref(n)))
        return n.value

    def register_prefix(self, seq: int, keys) -> None:
        """``pa_seq_register_prefix``: publish the sequence's first full blocks."""
        k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
        _check(lib().pa_seq_register_prefix(self._h, int(seq),
                                            k.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                            int(k.shape[0])))

    def blocks_needed(self, seq: int, n_tokens: int) -> int:
        n = ctypes.c_int32()
        _check(lib().pa_seq_blocks_needed(self._h, int(seq), int(n_tokens), ctypes.byref(n)))
        return n.value

    def append(self, seq: int, n_tokens: int):
        """Returns ``(slots int32[n_tokens], [(old, new)] copy-on-write pairs)``."""
        slots = np.empty(max(int(n_tokens), 1), dtype=np.int32)
        cow = np.empty(2, dtype=np.int32)
        ncow = ctypes.c_int32()
        _check(lib().pa_seq_append(self._h, int(seq), int(n_tokens), _ptr32(slots), _ptr32(cow),
                                   1, ctypes.byref(ncow)))
        pairs = [(int(cow[0]), int(cow[1]))] if ncow.value else []
        return slots[: int(n_tokens)], pairs

    def release(self, seq: int) -> None:
        _check(lib().pa_seq_release(self._h, int(seq)))

    def seq_len(self, seq: int) -> int:
        n = ctypes.c_int32()
        _check(lib().pa_seq_len(self._h, int(seq), ctypes.byref(n)))
        return n.value

    def block_tables(self, seqs, max_blocks: int, fill: int = -1) -> np.ndarray:
        s = _i32_array(seqs)
        out = np.empty((len(s), int(max_blocks)), dtype=np.int32)
        _check(lib().pa_block_tables(self._h, _ptr32(s), len(s), int(max_blocks), int(fill),
                                     _ptr32(out)))
        return out
