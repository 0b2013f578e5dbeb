"""Paged-decode throughput on one MI355X: effective KV GB/s and queries/s.

Workload (the GQA decode batch): 256 sequences, 32 query / 8 KV heads, head
dim 128, block size 16, bf16, lognormal lengths (median 1024, sigma 1,
clipped to [16, 8192]), 65536-block pool with a permuted free list.  Inputs
are seeded and synthetic (N(0,1) values); the context is written into the
pools before timing.

One step = the whole hot path for one decode round of the batch:
  pa_kv_write   (one new token per sequence, through slot_mapping)
  pa_decode     (balanced path: equal slices of the batch's work, one per
                 resident workgroup, then the merge of cut sequences)
all on torch's current HIP stream, inputs resident in HBM.  W warm-up steps,
then K timed steps bracketed by device synchronisation.  The fixed-partition
path (pa_decode_split + pa_reduce) is timed too, for comparison.

Reported:
  value          effective KV GB/s of the step = KV bytes / step time, with
                 KV bytes = sum(len) * kv_heads * head_dim * 2 (K,V) * 2 B
  roofline       the dominant call (pa_decode: the streaming kernel plus its
                 small merge kernel): algorithmic bytes (KV + Q + O +
                 block-table entries) over its average duration from HIP
                 events around it on the launch stream, against 8 TB/s;
                 `traffic` is filled from rocprofv3 counters when they were
                 taken for this kernel version (see --traffic)
  fp8_kv         the same batch decoded from an FP8 (e4m3) cache with
                 per-(token, KV head) scales (pa_kv_write_fp8 + pa_decode_fp8):
                 decode time, effective GB/s of codes + scales, queries/s
  mha_decode     the MHA batch (32 sequences, 40 heads, lengths U{128..2048}):
                 balanced decode time, KV GB/s, % of HBM peak, queries/s
  long_context   8 x 32768 decode + a 512-token causal prefill chunk in one
                 split launch + reduce: call time, its split/reduce parts,
                 GB/s and the fraction of its roofline time
  cpu_baseline   the CPU oracle (float64 NumPy) timed on a bounded sample of
                 the same queries (seeded order) on every host core the
                 process may use, and on one thread

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--partition", type=int, default=512)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run pa_copy_blocks over this many MiB (counter calibration)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--workload", choices=["gqa_decode", "long_context", "bs_sweep"],
                    default="gqa_decode",
                    help="gqa_decode: the headline measurement (default); long_context: time "
                         "the mixed split launch (8 x 32K decode + a 512-token causal chunk) "
                         "and its reduce, for profiling; bs_sweep: the headline batch at block "
                         "sizes 8, 16, 32 and 64 (decode time and tail-block waste)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; see the sharding notes of the design document.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_303_amd import build as pa_build
    if not os.path.exists(pa_build.library_path()):
        pa_build.build()
    if args.workload == "long_context":
        _long_context(args)
        return
    if args.workload == "bs_sweep":
        _bs_sweep(args)
        return
    from paged_kv_cache_303_amd import binding, runner, workloads as wl

    dev = torch.device("cuda", 0)
    t0 = time.time()
    w = wl.gqa_decode(seed=args.seed, partition_size=args.partition)
    log(f"workload drawn in {time.time() - t0:.1f}s: {len(w.seq_lens)} seqs, "
        f"{sum(w.seq_lens)} tokens, {w.kv_bytes / 1e9:.3f} GB of KV")

    # ---- set up: context in the pools, tables on the device ---------------------
    n_ctx = sum(w.seq_lens) - len(w.seq_lens)
    w_ctx_ops = w.ops[: 2 * len(w.seq_lens)]  # new + context appends
    st = runner.replay(_with_ops(w, w_ctx_ops), dev, poison=False)
    pool = st["pool"]
    handles = [st["handles"][s] for s in w.decode_seqs]
    slots = np.concatenate([pool.append(h, 1)[0] for h in handles]).astype(np.int32)
    seq_lens = np.array([pool.seq_len(h) for h in handles], dtype=np.int32)
    assert seq_lens.tolist() == w.seq_lens
    tables = pool.block_tables(handles, w.max_blocks)
    k_tok = runner.to_device(w.k_tokens[n_ctx:], w.dtype, dev)
    v_tok = runner.to_device(w.v_tokens[n_ctx:], w.dtype, dev)
    slot_d = torch.from_numpy(slots).to(dev)
    sl_d = torch.from_numpy(seq_lens).to(dev)
    bt_d = torch.from_numpy(tables).to(dev)
    q = runner.to_device(w.q, w.dtype, dev)
    k_pool, v_pool = st["k_pool"], st["v_pool"]
    maxp = binding.max_partitions_for(w.max_blocks, w.block_size, args.partition)
    split_ws = binding.SplitWorkspace(len(seq_lens), w.num_q_heads, w.head_dim, maxp, dev)
    out = torch.empty_like(q)
    ws = binding.decode_workspace(k_pool, len(seq_lens), w.num_q_heads)
    torch.cuda.synchronize()

    def step():
        binding.kv_write(k_pool, v_pool, k_tok, v_tok, slot_d)
        binding.decode(q, k_pool, v_pool, bt_d, sl_d, w.scale, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps (nothing but the step's launches) ---------
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = 1e3 * t_total / args.steps

    # the decode call alone, per call: HIP events on its stream around each call
    # of K more steps (outside the timed region: an event record in the stream
    # is work of its own)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i in range(args.steps):
        binding.kv_write(k_pool, v_pool, k_tok, v_tok, slot_d)
        events[i][0].record()
        binding.decode(q, k_pool, v_pool, bt_d, sl_d, w.scale, out=out, workspace=ws)
        events[i][1].record()
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in events])
    decode_ms = float(per_call.mean())

    # the cache write alone: one new token per sequence through the slot mapping
    kvw_ms = _timed(lambda: binding.kv_write(k_pool, v_pool, k_tok, v_tok, slot_d),
                    args.steps, args.warmup)
    kvw_bytes = len(seq_lens) * (2 * 2 * w.num_kv_heads * w.head_dim * 2 + 4)

    # the fixed-partition path (split + reduce), for context
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        binding.paged_attention(q, k_pool, v_pool, bt_d, sl_d, w.scale,
                                partition_size=args.partition, workspace=split_ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    split_ms = e0.elapsed_time(e1) / args.steps

    fp8 = _fp8_decode(binding, runner, w, st, slots, q, bt_d, sl_d, args, dev)

    if args.calib_copy_mib > 0:
        _calibration_copy(binding, k_pool, v_pool, args.calib_copy_mib, dev)
    del split_ws, st, k_pool, v_pool
    torch.cuda.empty_cache()
    mha = _mha_decode(args)
    lc = _long_context_metrics(args)

    kv_bytes = w.kv_bytes
    esize = 2
    q_bytes = len(seq_lens) * w.num_q_heads * w.head_dim * esize
    table_bytes = 4 * sum(-(-n // w.block_size) for n in w.seq_lens)
    alg_bytes = kv_bytes + 2 * q_bytes + table_bytes  # K, V, Q in, O out, table
    achieved = alg_bytes / (decode_ms * 1e-3) / 1e9
    traffic = _traffic(args.traffic)

    result = {
        "metric": "paged-decode effective KV GB/s (% of HBM peak) + queries/sec, GQA batch 256",
        "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gqa_decode: batch 256, 32/8 heads, head_dim 128, block_size 16, bf16, "
                        "lognormal lengths (median 1024, sigma 1.0, clip [16, 8192]), "
                        "65536-block pool, kv_write of one token/seq + balanced pa_decode",
            "global_batch": len(seq_lens),
            "total_tokens": int(sum(w.seq_lens)),
            "max_len": int(max(w.seq_lens)),
            "kv_bytes": int(kv_bytes),
            "decode_slices": _slices(ws, len(seq_lens), w.num_q_heads, w.head_dim),
            "seed": args.seed,
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "queries_per_s": round(len(seq_lens) / (ms_step * 1e-3), 1),
        "decode_only": {
            "ms": round(decode_ms, 4),
            "p10_ms": round(float(np.percentile(per_call, 10)), 4),
            "p50_ms": round(float(np.percentile(per_call, 50)), 4),
            "p90_ms": round(float(np.percentile(per_call, 90)), 4),
            "kv_GBps": round(kv_bytes / (decode_ms * 1e-3) / 1e9, 1),
            "queries_per_s": round(len(seq_lens) / (decode_ms * 1e-3), 1),
        },
        "kv_write": {
            "ms": round(kvw_ms, 4),
            "bytes": int(kvw_bytes),
            "GBps": round(kvw_bytes / (kvw_ms * 1e-3) / 1e9, 1),
        },
        "gpu": _gpu_info(),
        "split_path": {
            "partition_size": args.partition,
            "ms": round(split_ms, 4),
            "kv_GBps": round(kv_bytes / (split_ms * 1e-3) / 1e9, 1),
        },
        "fp8_kv": fp8,
        "mha_decode": mha,
        "long_context": lc,
        "roofline": {
            "kernel": "pa_decode (decode_stream_kernel<bf16,128,4> + stream_fixup_kernel)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": int(alg_bytes),
            "avg_launch_ms": round(decode_ms, 4),
        },
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = _cpu_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


def _fp8_decode(binding, runner, w, st, new_slots, q, bt_d, sl_d, args, dev):
    """The same batch from an FP8 (e4m3) cache: every token quantized into e4m3 pools
    with per-(token, KV head) scales, then the balanced decode over them (timed)."""
    import numpy as np
    import torch

    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc = torch.empty(shape, dtype=torch.uint8, device=dev)
    vc = torch.empty(shape, dtype=torch.uint8, device=dev)
    ks = torch.empty(binding.fp8_scale_shape(kc), dtype=torch.float32, device=dev)
    vs = torch.empty(binding.fp8_scale_shape(kc), dtype=torch.float32, device=dev)
    ctx = np.concatenate([np.asarray(sl, np.int32) for _, sl, _ in st["log"]])
    all_slots = torch.from_numpy(np.concatenate([ctx, new_slots]).astype(np.int32)).to(dev)
    binding.kv_write_fp8(kc, vc, ks, vs, runner.to_device(w.k_tokens, w.dtype, dev),
                         runner.to_device(w.v_tokens, w.dtype, dev), all_slots)
    ws = binding.decode_workspace(kc, len(w.seq_lens), w.num_q_heads)
    out = torch.empty_like(q)
    _warm_for(lambda: binding.decode_fp8(q, kc, vc, ks, vs, bt_d, sl_d, w.scale, out=out,
                                         workspace=ws), 0.2)  # after the set-up
    for _ in range(args.warmup):
        binding.decode_fp8(q, kc, vc, ks, vs, bt_d, sl_d, w.scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        binding.decode_fp8(q, kc, vc, ks, vs, bt_d, sl_d, w.scale, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens = int(sum(w.seq_lens))
    code_bytes = tokens * w.num_kv_heads * w.head_dim * 2        # K and V codes
    scale_bytes = tokens * w.num_kv_heads * 4 * 2                # K and V scales
    del kc, vc, ks, vs
    return {
        "format": "e4m3 codes + one fp32 scale per (token, KV head), bf16 q/out",
        "decode_ms": round(ms, 4),
        "kv_bytes": code_bytes + scale_bytes,
        "kv_GBps": round((code_bytes + scale_bytes) / (ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * (code_bytes + scale_bytes) / (ms * 1e-3) / 1e9
                              / HBM_PEAK_GBPS, 2),
        "queries_per_s": round(len(w.seq_lens) / (ms * 1e-3), 1),
    }


def _bs_sweep(args):
    """The GQA batch at several block sizes: balanced decode time, effective KV GB/s, and
    the pool slots lost to partly filled tail blocks ("LLM 推理引擎的内存管理与调度" §3.1
    on the block-size trade-off)."""
    import numpy as np
    import torch
    from paged_kv_cache_303_amd import binding, runner, workloads as wl

    dev = torch.device("cuda", 0)
    rows = []
    for bs in (8, 16, 32, 64):
        w = wl.gqa_decode(seed=args.seed, block_size=bs, num_blocks=65536 * 16 // bs)
        st = runner.replay(w, dev, poison=False)
        ws = binding.decode_workspace(st["k_pool"], len(w.seq_lens), w.num_q_heads)
        out = torch.empty_like(st["q"])
        call = (st["q"], st["k_pool"], st["v_pool"], st["block_tables"], st["seq_lens"], w.scale)
        for _ in range(args.warmup):
            binding.decode(*call, out=out, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            binding.decode(*call, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        lens = np.asarray(w.seq_lens, np.int64)
        slots = int((-(-lens // bs) * bs).sum())
        rows.append({"block_size": bs, "decode_ms": round(ms, 4),
                     "kv_GBps": round(w.kv_bytes / (ms * 1e-3) / 1e9, 1),
                     "pct_hbm_peak": round(100 * w.kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                     "tail_waste_pct": round(100.0 * (slots - int(lens.sum())) / slots, 3)})
        log(f"block size {bs}: {rows[-1]}")
        del st, ws, out
        torch.cuda.empty_cache()
    print(json.dumps({"workload": "bs_sweep: gqa_decode batch 256 (32/8 heads, head_dim 128, "
                                  "bf16, lognormal lengths) at block sizes 8..64",
                      "steps": args.steps, "rows": rows}), flush=True)


def _long_context(args):
    """Mixed split launch: 8 decode sequences of 32768 tokens and a causal
    512-token prefill chunk in one pa_decode_split, then pa_reduce."""
    print(json.dumps(_long_context_metrics(args)), flush=True)


def _warm_for(fn, seconds):
    """Call fn() repeatedly for about `seconds` of wall time (untimed)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def _timed(fn, steps, warmup):
    """Mean ms per call of fn() from HIP events on torch's current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _mha_decode(args):
    """The MHA batch: 32 sequences, 40 heads (MHA), head dim 128, block size 16, bf16,
    lengths uniform in [128, 2048], 4096-block pool; balanced pa_decode."""
    import torch
    from paged_kv_cache_303_amd import binding, runner, workloads as wl

    dev = torch.device("cuda", 0)
    w = wl.mha_decode()
    st = runner.replay(w, dev, poison=False)
    ws = binding.decode_workspace(st["k_pool"], len(w.seq_lens), w.num_q_heads)
    out = torch.empty_like(st["q"])
    call = (st["q"], st["k_pool"], st["v_pool"], st["block_tables"], st["seq_lens"], w.scale)
    _warm_for(lambda: binding.decode(*call, out=out, workspace=ws), 0.2)  # after the set-up
    ms = _timed(lambda: binding.decode(*call, out=out, workspace=ws), args.steps, args.warmup)
    n = len(w.seq_lens)
    alg = w.kv_bytes + 2 * n * w.num_q_heads * w.head_dim * 2 + \
        4 * sum(-(-x // w.block_size) for x in w.seq_lens)
    res = {"workload": "mha_decode: batch 32, 40/40 heads, head_dim 128, block_size 16, bf16, "
                       "lengths U{128..2048}, 4096-block pool, balanced pa_decode",
           "ms": round(ms, 4), "kv_bytes": int(w.kv_bytes),
           "kv_GBps": round(w.kv_bytes / (ms * 1e-3) / 1e9, 1),
           "pct_hbm_peak": round(100 * alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
           "queries_per_s": round(n / (ms * 1e-3), 1)}
    log(f"mha_decode: {res}")
    del st, ws, out
    torch.cuda.empty_cache()
    return res


def _long_context_metrics(args):
    """Long context + chunked prefill: 8 decode sequences of 32768 tokens and a
    causal 512-token chunk after 4096 cached tokens in one pa_decode_split
    launch, then pa_reduce.  Reported against the call's roofline
    t_min = max(bytes / HBM peak, flops / bf16 MFMA peak)."""
    import numpy as np
    import torch
    from paged_kv_cache_303_amd import binding, runner, workloads as wl

    dev = torch.device("cuda", 0)
    w = wl.long_context()
    st = runner.replay(w, dev, poison=False)
    ws = runner.split_workspace(w, st)
    out = torch.empty_like(st["q"])
    p = w.partition_size
    call = lambda: runner.attention(w, st, workspace=ws, out=out)
    split = lambda: binding.decode_split(st["q"], st["k_pool"], st["v_pool"], st["block_tables"],
                                         st["seq_lens"], w.scale, partition_size=p,
                                         cu_q_lens=st["cu_q_lens"], workspace=ws)
    red = lambda: binding.reduce(ws, st["seq_lens"], p, out_dtype=st["q"].dtype,
                                 cu_q_lens=st["cu_q_lens"], out=out)
    # the set-up above leaves the GPU idle for seconds: run the call until the
    # clocks are back at their working level (about 0.2 s) before timing, so
    # that the call and its parts below are measured in the same state
    _warm_for(call, 0.2)
    ms = _timed(call, args.steps, args.warmup)
    ms_split = _timed(split, args.steps, args.warmup)
    ms_reduce = _timed(red, args.steps, args.warmup)
    # the same launch over each kind of work alone: the decode sequences, then the chunk
    dec_idx = [i for i, ql in enumerate(w.q_lens) if ql == 1]
    pre_idx = [i for i, ql in enumerate(w.q_lens) if ql > 1]
    cu = np.concatenate([[0], np.cumsum(w.q_lens)]).astype(np.int64)

    def part(idx, multi):
        rows = torch.cat([torch.arange(int(cu[i]), int(cu[i + 1])) for i in idx]).to(dev)
        q_p = st["q"][rows].contiguous()
        sel = torch.tensor(idx, device=dev)
        bt_p = st["block_tables"][sel].contiguous()
        sl_p = st["seq_lens"][sel].contiguous()
        cu_p = None
        if multi:
            cu_p = torch.tensor(np.concatenate([[0], np.cumsum([w.q_lens[i] for i in idx])]),
                                dtype=torch.int32, device=dev)
        ws_p = binding.SplitWorkspace(q_p.shape[0], q_p.shape[1], q_p.shape[2], ws.shape[2], dev)
        return _timed(lambda: binding.decode_split(q_p, st["k_pool"], st["v_pool"], bt_p, sl_p,
                                                   w.scale, partition_size=p, cu_q_lens=cu_p,
                                                   workspace=ws_p), args.steps, args.warmup)

    ms_dec = part(dec_idx, False)
    ms_pre = part(pre_idx, True)
    # algorithmic work: every decode key once; the chunk's K/V once, its Q in and O out
    esize = 2
    row = w.num_kv_heads * w.head_dim * esize * 2
    dec = [n for n, ql in zip(w.seq_lens, w.q_lens) if ql == 1]
    pre = [(n, ql) for n, ql in zip(w.seq_lens, w.q_lens) if ql > 1]
    bytes_dec = sum(dec) * row + 2 * len(dec) * w.num_q_heads * w.head_dim * esize
    bytes_pre = sum(n * row + 2 * ql * w.num_q_heads * w.head_dim * esize for n, ql in pre)
    pairs = sum(sum(n - ql + i + 1 for i in range(ql)) for n, ql in pre)
    flops = pairs * w.num_q_heads * 4 * w.head_dim
    alg = bytes_dec + bytes_pre
    t_min = max(alg / (HBM_PEAK_GBPS * 1e9), flops / 2.5e15)
    res = {"workload": "long_context: 8 x 32768 decode + a 512-token causal chunk after 4096 "
                       "tokens, block_size 32, 32/8 heads, head_dim 128, bf16, partitions of 512; "
                       "one pa_decode_split launch + pa_reduce",
           "ms": round(ms, 4), "split_ms": round(ms_split, 4), "reduce_ms": round(ms_reduce, 4),
           "split_decode_only_ms": round(ms_dec, 4), "split_prefill_only_ms": round(ms_pre, 4),
           "decode_only_GBps": round(bytes_dec / (ms_dec * 1e-3) / 1e9, 1),
           "prefill_only_TFLOPs": round(flops / (ms_pre * 1e-3) / 1e12, 1),
           "alg_bytes": int(alg), "prefill_flops": int(flops),
           "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
           "t_min_us": round(1e6 * t_min, 1),
           "pct_of_t_min": round(100 * t_min / (ms * 1e-3), 2)}
    log(f"long_context: {res}")
    del st, ws, out
    torch.cuda.empty_cache()
    return res


def _slices(ws, num_seqs, hq, d):
    """Slices of the balanced decode, from its workspace size (layout of pa_decode)."""
    if ws is None:
        return None
    a256 = lambda x: (x + 255) // 256 * 256
    per_slice = 2 * hq * d * 4 + 2 * hq * 4
    rest = ws.numel() - a256((num_seqs + 1) * 4)
    return int(rest // per_slice)


def _with_ops(w, ops):
    import copy
    w2 = copy.copy(w)
    w2.ops = ops
    return w2


def _calibration_copy(binding, k_pool, v_pool, mib, dev):
    """pa_copy_blocks over `mib` MiB of K+V blocks: a plain copy of known size."""
    import torch
    block_bytes = k_pool[0].numel() * k_pool.element_size()
    n = max(1, (mib << 20) // (2 * block_bytes))
    n = min(n, k_pool.shape[0] // 2)
    pairs = torch.stack([torch.arange(n), torch.arange(n) + k_pool.shape[0] // 2], 1)
    pairs = pairs.to(torch.int32).to(dev)
    binding.copy_blocks(k_pool, v_pool, pairs)
    torch.cuda.synchronize()
    log(f"calibration copy: {n} block pairs, {2 * n * block_bytes} bytes read and written")


def _traffic(path):
    """HBM bytes per launch of the measured decode kernels, from rocprofv3 counters, if
    they were taken on the current version of those kernels' source."""
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    from paged_kv_cache_303_amd import build as pa_build
    if data.get("kernel_source_hash") != pa_build.source_hash(data.get("kernel_source")):
        return None
    return data.get("bytes_per_launch")


def _gpu_info():
    """Device name and the engine clock the driver reports as current, read from
    sysfs (no child process: a program started after the GPU is initialised
    would be refused on some hosts)."""
    import glob
    import torch
    info = {"name": torch.cuda.get_device_name(0), "sclk_mhz": None}
    try:
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            with open(path) as fh:
                cur = [l.split(":", 1)[1].strip().rstrip("*").strip()
                       for l in fh if l.rstrip().endswith("*")]
            if cur:
                info["sclk_mhz"] = cur[0]
                break
    except Exception:  # the clock is context only; its absence changes nothing else
        pass
    return info


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(w, budget_s):
    """The oracle as it stands, on a bounded, seeded sample of the same queries: once
    on every host core the process may use (one query per worker thread at a time;
    NumPy releases the GIL in its array loops) and once on one thread."""
    import concurrent.futures
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import runner as orun

    t0 = time.time()
    ost = orun.replay(w)
    log(f"oracle replay (setup, untimed) {time.time() - t0:.1f}s")
    order = np.random.default_rng(0).permutation(len(w.seq_lens)).tolist()
    cores = len(os.sched_getaffinity(0))

    def run(threads, budget):
        done = []
        stop = [False]

        def worker(k):
            i = k
            while not stop[0]:
                j = order[i % len(order)]
                orun.attention(w, ost, tokens=[j])
                done.append(j)
                i += threads

        with threadpool_limits(limits=1):
            start = time.perf_counter()
            with concurrent.futures.ThreadPoolExecutor(threads) as ex:
                futs = [ex.submit(worker, k) for k in range(threads)]
                time.sleep(budget)
                stop[0] = True
                for f in futs:
                    f.result()
            elapsed = time.perf_counter() - start
        keys = sum(w.seq_lens[j] for j in done)
        kv = keys * w.num_kv_heads * w.head_dim * 2 * 2
        return kv / elapsed / 1e9, len(done) / elapsed, len(done), keys, elapsed

    gbps, qps, n, keys, el = run(cores, budget_s)
    gbps1, qps1, n1, keys1, el1 = run(1, budget_s / 2)
    return {
        "value": round(gbps, 4),
        "unit": "GB/s",
        "queries_per_s": round(qps, 2),
        "cores": cores,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"{n} decode-query evaluations over the {len(w.seq_lens)} queries "
                  f"(seeded order, repeated), {keys} keys, {el:.1f}s, float64 NumPy, "
                  f"{cores} worker threads",
        "one_thread": {"value": round(gbps1, 4), "unit": "GB/s",
                       "queries_per_s": round(qps1, 2),
                       "sample": f"{n1} query evaluations, {keys1} keys, {el1:.1f}s"},
    }


if __name__ == "__main__":
    main()
