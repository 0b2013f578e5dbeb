"""GPU block swap (pa_swap_blocks) between the device pools and pinned host memory.

A preempted request's blocks go out to host pools and come back into other
physical blocks ("LLM 推理引擎的内存管理与调度" §9; "19.2 KV Cache 系统化管理"
§19.2.6).  The host pools are compared bit for bit with the oracle's own swap
of its own pools; after the swap-in (old device blocks poisoned, table remapped)
the decode output is bit-identical to the one before the swap.
"""

import numpy as np
import pytest
import torch

from oracle import runner as orun
from oracle import swap_blocks as oracle_swap
from paged_kv_cache_303_amd import workloads as wl
from tests.parity import pools_equal_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa(built_library, gpu):
    from paged_kv_cache_303_amd import binding, runner
    return binding, runner, gpu


def _workload():
    return wl.custom_decode(21, [40, 300, 129, 77], num_blocks=128, block_size=16,
                            num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=wl.BF16,
                            name="swap")


def _remap(table_row, nblk, used, num_blocks):
    """Fresh physical ids for the first nblk entries (ids not in `used`)."""
    free = [b for b in range(num_blocks - 1, -1, -1) if b not in used]
    new = table_row.copy()
    new[:nblk] = free[:nblk]
    return new


def test_swap_round_trip_bf16(pa):
    binding, runner, dev = pa
    w = _workload()
    st = runner.replay(w, dev)
    st_o = orun.replay(w)
    assert pools_equal_bits(st["k_pool"], st_o["k_pool"])
    args = (st["q"], st["k_pool"], st["v_pool"], st["block_tables"], st["seq_lens"], w.scale)
    ws = binding.decode_workspace(st["k_pool"], len(w.seq_lens), w.num_q_heads)
    before = [binding.decode(*args), binding.decode(*args, workspace=ws)]

    b = 1  # the preempted request
    tables = st["block_tables_host"].copy()
    nblk = -(-int(st["seq_lens_host"][b]) // w.block_size)
    dev_ids = tables[b, :nblk].tolist()
    host_k = torch.zeros((nblk,) + tuple(st["k_pool"].shape[1:]), dtype=torch.bfloat16,
                         pin_memory=True)
    host_v = torch.zeros_like(host_k).pin_memory()
    out_pairs = torch.tensor([[d, i] for i, d in enumerate(dev_ids)], dtype=torch.int32)
    binding.swap_blocks(host_k, host_v, st["k_pool"], st["v_pool"], out_pairs.to(dev))
    torch.cuda.synchronize()
    ok_k = np.zeros((nblk,) + st_o["k_pool"].shape[1:], np.uint16)
    ok_v = np.zeros_like(ok_k)
    oracle_swap(ok_k, ok_v, st_o["k_pool"], st_o["v_pool"], out_pairs.tolist())
    assert np.array_equal(host_k.view(torch.int16).numpy().view(np.uint16), ok_k)
    assert np.array_equal(host_v.view(torch.int16).numpy().view(np.uint16), ok_v)

    # the device blocks are reused by someone else meanwhile
    st["k_pool"][dev_ids] = float("nan")
    st["v_pool"][dev_ids] = float("nan")
    used = set(int(x) for x in tables[tables >= 0].ravel())
    new_row = _remap(tables[b], nblk, used, w.num_blocks)
    in_pairs = torch.tensor([[i, int(new_row[i])] for i in range(nblk)], dtype=torch.int32)
    binding.swap_blocks(st["k_pool"], st["v_pool"], host_k, host_v, in_pairs.pin_memory())
    tables[b] = new_row
    bt = torch.from_numpy(tables).to(dev)
    args2 = (st["q"], st["k_pool"], st["v_pool"], bt, st["seq_lens"], w.scale)
    after = [binding.decode(*args2), binding.decode(*args2, workspace=ws)]
    torch.cuda.synchronize()
    for x, y in zip(before, after):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_swap_round_trip_fp8_codes_and_scales(pa):
    binding, runner, dev = pa
    w = _workload()
    st = runner.replay(w, dev, poison=False)
    shape = tuple(st["k_pool"].shape)
    kc = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
    vc = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
    ks = torch.full(binding.fp8_scale_shape(kc), float("nan"), device=dev)
    vs = torch.full(binding.fp8_scale_shape(kc), float("nan"), device=dev)
    slots = np.concatenate([np.asarray(s, np.int32) for _, s, _ in st["log"]])
    binding.kv_write_fp8(kc, vc, ks, vs, runner.to_device(w.k_tokens, "bf16", dev),
                         runner.to_device(w.v_tokens, "bf16", dev),
                         torch.from_numpy(slots).to(dev))
    args = (st["q"], kc, vc, ks, vs, st["block_tables"], st["seq_lens"], w.scale)
    before = binding.decode_fp8(*args)
    b = 2
    tables = st["block_tables_host"].copy()
    nblk = -(-int(st["seq_lens_host"][b]) // w.block_size)
    dev_ids = tables[b, :nblk].tolist()
    hk = torch.zeros((nblk,) + shape[1:], dtype=torch.uint8, pin_memory=True)
    hv = torch.zeros_like(hk).pin_memory()
    hks = torch.zeros((nblk,) + binding.fp8_scale_shape(kc)[1:], dtype=torch.float32,
                      pin_memory=True)
    hvs = torch.zeros_like(hks).pin_memory()
    out_pairs = torch.tensor([[d, i] for i, d in enumerate(dev_ids)], dtype=torch.int32).to(dev)
    binding.swap_blocks(hk, hv, kc, vc, out_pairs)
    binding.swap_blocks(hks, hvs, ks, vs, out_pairs)
    torch.cuda.synchronize()
    kc[dev_ids] = 0x7F
    ks[dev_ids] = float("nan")
    used = set(int(x) for x in tables[tables >= 0].ravel())
    new_row = _remap(tables[b], nblk, used, w.num_blocks)
    in_pairs = torch.tensor([[i, int(new_row[i])] for i in range(nblk)],
                            dtype=torch.int32).to(dev)
    binding.swap_blocks(kc, vc, hk, hv, in_pairs)
    binding.swap_blocks(ks, vs, hks, hvs, in_pairs)
    tables[b] = new_row
    after = binding.decode_fp8(st["q"], kc, vc, ks, vs, torch.from_numpy(tables).to(dev),
                               st["seq_lens"], w.scale)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))


def test_swap_bandwidth_and_rejections(pa):
    binding, runner, dev = pa
    nb, blk = 2048, (16, 8, 128)  # 2048 blocks of 32 KiB for K and for V: 128 MiB
    dk = torch.randn((nb,) + blk, device=dev).to(torch.bfloat16)
    dv = torch.randn((nb,) + blk, device=dev).to(torch.bfloat16)
    hk = torch.empty((nb,) + blk, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk).pin_memory()
    pairs = torch.stack([torch.arange(nb), torch.arange(nb)], 1).to(torch.int32).to(dev)
    binding.swap_blocks(hk, hv, dk, dv, pairs)  # warm-up
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    binding.swap_blocks(hk, hv, dk, dv, pairs)
    e1.record()
    binding.swap_blocks(dk, dv, hk, hv, pairs)
    e2.record()
    torch.cuda.synchronize()
    gb = 2 * nb * 16 * 8 * 128 * 2 / 1e9
    print(f"[swap] {gb:.3f} GB out {gb / (e0.elapsed_time(e1) * 1e-3):.1f} GB/s, "
          f"in {gb / (e1.elapsed_time(e2) * 1e-3):.1f} GB/s", flush=True)
    assert torch.equal(hk[5].to(dev), dk[5])
    with pytest.raises(TypeError):  # pageable host memory is refused
        binding.swap_blocks(torch.empty_like(hk), hv, dk, dv, pairs)
