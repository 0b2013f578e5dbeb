"""Pins of the block-swap oracle (preemption by swapping, "LLM 推理引擎的内存管理与调度"
§9; "19.2 KV Cache 系统化管理" §19.2.6): a swap is a bit copy between two pools,
so out-and-back is the identity and untouched blocks do not change."""

import numpy as np
import pytest

from oracle import swap_blocks


def test_swap_out_and_back_is_identity():
    rng = np.random.default_rng(0)
    dev_k = rng.integers(0, 2**16, (12, 4, 2, 8), dtype=np.uint16)
    dev_v = rng.integers(0, 2**16, (12, 4, 2, 8), dtype=np.uint16)
    k0, v0 = dev_k.copy(), dev_v.copy()
    host_k = np.zeros((5, 4, 2, 8), np.uint16)
    host_v = np.zeros_like(host_k)
    out_pairs = [(7, 0), (3, 1), (9, 4)]
    swap_blocks(host_k, host_v, dev_k, dev_v, out_pairs)
    for s, d in out_pairs:
        assert np.array_equal(host_k[d], k0[s]) and np.array_equal(host_v[d], v0[s])
    assert (host_k[[2, 3]] == 0).all()
    dev_k[[7, 3, 9]] = 0xFFFF  # the device blocks are reused meanwhile
    in_pairs = [(0, 10), (1, 11), (4, 2)]
    swap_blocks(dev_k, dev_v, host_k, host_v, in_pairs)
    assert np.array_equal(dev_k[[10, 11, 2]], k0[[7, 3, 9]])
    assert np.array_equal(dev_v[[10, 11, 2]], v0[[7, 3, 9]])
    untouched = [0, 1, 4, 5, 6, 8]
    assert np.array_equal(dev_k[untouched], k0[untouched])


def test_swap_rejects_repeated_destinations():
    a = np.zeros((4, 2), np.float32)
    with pytest.raises(ValueError):
        swap_blocks(a, a.copy(), a.copy(), a.copy(), [(0, 1), (2, 1)])
