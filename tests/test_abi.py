"""The C ABI: libpa.so loads, exports every function pa.h declares, and its
host-side validation rejects bad arguments before any kernel launch.

CPU only: every call here fails validation (or is a pure host call), so
nothing reaches the GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ["pa_kv_write", "pa_decode", "pa_decode_split", "pa_reduce", "pa_copy_blocks",
              "pa_pool_create", "pa_seq_append", "pa_block_tables"]:
        assert n in names


def test_library_exports_every_declared_symbol(built_library):
    lib = ctypes.CDLL(built_library)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []


def test_binding_covers_every_declared_symbol(built_library):
    from paged_kv_cache_303_amd import binding
    assert sorted(binding.exported_symbols()) == declared_functions()
    assert "gfx950" in binding.version()


def _lay(nb=16, bs=16, hkv=8, d=128, dtype=1):
    from paged_kv_cache_303_amd.binding import KVLayout
    return KVLayout(nb, bs, hkv, d, dtype)


def _err(lib):
    return lib.pa_last_error().decode()


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, 2), ("head_dim", 96, 2), ("block_size", 12, 2), ("block_size", 512, 2),
    ("num_blocks", 0, 1), ("num_kv_heads", -1, 1)])
def test_layout_validation(built_library, field, value, status):
    from paged_kv_cache_303_amd import binding
    lib = binding.lib()
    lay = _lay()
    setattr(lay, field, value)
    dummy = ctypes.c_void_p(16)
    st = lib.pa_decode(ctypes.byref(lay), dummy, dummy, dummy, dummy, dummy, 4, dummy, 1, 32,
                       0.1, None, 0, None)
    assert st == status, _err(lib)
    assert "pa_decode" in _err(lib)


def test_decode_argument_validation(built_library):
    from paged_kv_cache_303_amd import binding
    lib = binding.lib()
    lay = _lay()
    d = ctypes.c_void_p(16)
    nul = ctypes.c_void_p(0)
    # query heads not a multiple of KV heads; unsupported ratio; NULL pointers
    assert lib.pa_decode(ctypes.byref(lay), d, d, d, d, d, 4, d, 1, 12, 0.1, None, 0, None) == 1
    assert lib.pa_decode(ctypes.byref(lay), d, d, d, d, d, 4, d, 1, 8 * 16, 0.1, None, 0, None) == 2
    assert lib.pa_decode(ctypes.byref(lay), d, nul, d, d, d, 4, d, 1, 32, 0.1, None, 0, None) == 1
    assert lib.pa_decode(ctypes.byref(lay), nul, d, d, d, d, 4, d, 1, 32, 0.1, None, 0, None) == 1
    assert lib.pa_decode(ctypes.byref(lay), d, d, d, d, d, 0, d, 1, 32, 0.1, None, 0, None) == 1
    assert lib.pa_decode(ctypes.byref(lay), d, d, d, d, d, 4, d, 1, 32, float("nan"), None, 0, None) == 1
    assert lib.pa_decode(ctypes.byref(lay), d, d, d, d, d, 4, d, 1, 32, -0.5, None, 0, None) == 1
    assert lib.pa_decode(ctypes.byref(lay), d, d, d, d, d, 4, d, 1, 32, 0.0, None, 0, None) == 1
    assert lib.pa_decode(None, d, d, d, d, d, 4, d, 1, 32, 0.1, None, 0, None) == 1
    # zero sequences is a no-op
    assert lib.pa_decode(ctypes.byref(lay), nul, nul, d, d, nul, 4, nul, 0, 32, 0.1, None, 0, None) == 0


def test_split_argument_validation(built_library):
    from paged_kv_cache_303_amd import binding
    lib = binding.lib()
    lay = _lay()
    d = ctypes.c_void_p(16)
    nul = ctypes.c_void_p(0)
    ws = ctypes.c_void_p(1 << 20)  # 256-byte aligned address (never dereferenced)
    big = 1 << 40
    args = lambda maxp, psize, cu, nq, w=ws, n=big: (ctypes.byref(lay), w, n, maxp, psize, d, cu,
                                                    nq, d, d, d, 64, d, 4, 32, 0.1, None)
    assert lib.pa_decode_split(*args(1, 512, nul, 4)) == 1   # 1*512 < 64*16
    assert lib.pa_decode_split(*args(2, 520, nul, 4)) == 1   # not a multiple of 16
    assert lib.pa_decode_split(*args(2, 8, nul, 4)) == 1     # not a multiple of block_size
    assert lib.pa_decode_split(*args(2, 512, nul, 5)) == 1   # nq != num_seqs without cu
    assert lib.pa_decode_split(*args(70000, 512, nul, 4)) == 1
    assert lib.pa_decode_split(*args(2, 512, nul, 4, d)) == 1      # workspace not aligned
    assert lib.pa_decode_split(*args(2, 512, nul, 4, nul)) == 1    # no workspace
    need = lib.pa_split_workspace_bytes(4, 32, 128, 2)
    assert lib.pa_decode_split(*args(2, 512, nul, 4, ws, need - 1)) == 1  # too small
    assert "workspace" in _err(lib)
    lay1 = _lay(bs=16)
    one = lambda cu: (ctypes.byref(lay1), ws, big, 1, 1024, d, cu, 4, d, d, d, 64, d, 4, 32, 0.1,
                      None)
    assert lib.pa_decode_split(*one(d)) == 1  # prefill chunks need two partition slots
    assert "max_partitions" in _err(lib)
    assert lib.pa_decode_split(*args(2, 512, d, 0)) == 0     # no query tokens: no-op


def test_split_workspace_layout(built_library):
    """Offsets and size of the split workspace follow the documented layout."""
    from paged_kv_cache_303_amd import binding
    lib = binding.lib()
    for nq, hq, d, maxp in [(1, 1, 32, 1), (520, 32, 128, 64), (256, 32, 128, 16), (3, 8, 256, 5)]:
        lay = binding.SplitLayout()
        assert lib.pa_split_workspace_layout(nq, hq, d, maxp, ctypes.byref(lay)) == 0
        a256 = lambda x: -(-x // 256) * 256
        o = a256(nq * hq * maxp * d * 4)
        ls = a256(nq * hq * maxp * 4)
        assert (lay.part_o_offset, lay.part_lse_offset, lay.control_offset) == (0, o, o + ls)
        assert lay.total_bytes == o + ls + 256
        assert lib.pa_split_workspace_bytes(nq, hq, d, maxp) == lay.total_bytes
    assert lib.pa_split_workspace_bytes(4, 0, 128, 2) == 0
    assert lib.pa_split_workspace_bytes(4, 8, 128, 0) == 0
    assert lib.pa_split_workspace_layout(4, 8, 128, 2, None) == 1


def test_other_calls_validation(built_library):
    from paged_kv_cache_303_amd import binding
    lib = binding.lib()
    lay = _lay()
    d = ctypes.c_void_p(16)
    nul = ctypes.c_void_p(0)
    assert lib.pa_kv_write(ctypes.byref(lay), d, d, d, d, d, -1, None) == 1
    assert lib.pa_kv_write(ctypes.byref(lay), nul, nul, nul, nul, nul, 0, None) == 0
    assert lib.pa_kv_write(ctypes.byref(lay), d, nul, d, d, d, 3, None) == 1
    assert lib.pa_copy_blocks(ctypes.byref(lay), d, d, nul, 2, None) == 1
    assert lib.pa_copy_blocks(ctypes.byref(lay), nul, nul, nul, 0, None) == 0
    ws = ctypes.c_void_p(1 << 20)
    big = 1 << 40
    assert lib.pa_reduce(d, 5, nul, ws, big, 4, 512, nul, d, 4, 4, 32, 128, None) == 2
    assert lib.pa_reduce(d, 1, nul, ws, big, 4, 512, nul, d, 4, 4, 32, 100, None) == 2
    assert lib.pa_reduce(d, 1, nul, ws, big, 4, 512, nul, d, 4, 5, 32, 128, None) == 1
    assert lib.pa_reduce(d, 1, nul, nul, big, 4, 512, nul, d, 4, 4, 32, 128, None) == 1
    assert lib.pa_reduce(d, 1, nul, ws, 16, 4, 512, nul, d, 4, 4, 32, 128, None) == 1
    assert lib.pa_reduce(d, 1, nul, ws, big, 4, 0, nul, d, 4, 4, 32, 128, None) == 1
