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
  cpu_baseline   the CPU oracle (float64 NumPy, single thread) timed on a
                 bounded sample of the same queries (seeded order, ~15 s)

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
    ap.add_argument("--cpu-budget", type=float, default=12.0,
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
    part_o = torch.empty((len(seq_lens), w.num_q_heads, maxp, w.head_dim), dtype=torch.float32,
                         device=dev)
    part_lse = torch.empty(part_o.shape[:3], dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    ws = binding.decode_workspace(k_pool, len(seq_lens), w.num_q_heads)
    torch.cuda.synchronize()

    def step(ev=None):
        binding.kv_write(k_pool, v_pool, k_tok, v_tok, slot_d)
        if ev is not None:
            ev[0].record()
        binding.decode(q, k_pool, v_pool, bt_d, sl_d, w.scale, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps ------------------------------------------
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = 1e3 * t_total / args.steps
    per_call = np.array([a.elapsed_time(b) for a, b in events])
    decode_ms = float(per_call.mean())

    # the fixed-partition path (split + reduce), for context
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        binding.decode_split(q, k_pool, v_pool, bt_d, sl_d, w.scale,
                             partition_size=args.partition, part_o=part_o, part_lse=part_lse,
                             max_partitions=maxp)
        binding.reduce(part_o, part_lse, sl_d, args.partition, out_dtype=q.dtype, out=out)
    e1.record()
    torch.cuda.synchronize()
    split_ms = e0.elapsed_time(e1) / args.steps

    fp8 = _fp8_decode(binding, runner, w, st, slots, q, bt_d, sl_d, args, dev)

    if args.calib_copy_mib > 0:
        _calibration_copy(binding, k_pool, v_pool, args.calib_copy_mib, dev)

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
        "split_path": {
            "partition_size": args.partition,
            "ms": round(split_ms, 4),
            "kv_GBps": round(kv_bytes / (split_ms * 1e-3) / 1e9, 1),
        },
        "fp8_kv": fp8,
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
    ks = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    vs = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    ctx = np.concatenate([np.asarray(sl, np.int32) for _, sl, _ in st["log"]])
    all_slots = torch.from_numpy(np.concatenate([ctx, new_slots]).astype(np.int32)).to(dev)
    binding.kv_write_fp8(kc, vc, ks, vs, runner.to_device(w.k_tokens, w.dtype, dev),
                         runner.to_device(w.v_tokens, w.dtype, dev), all_slots)
    ws = binding.decode_workspace(kc, len(w.seq_lens), w.num_q_heads)
    out = torch.empty_like(q)
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
    import torch
    from paged_kv_cache_303_amd import runner, workloads as wl

    dev = torch.device("cuda", 0)
    w = wl.long_context()
    st = runner.replay(w, dev, poison=False)
    for _ in range(args.warmup):
        runner.attention(w, st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        runner.attention(w, st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"workload": "long_context: 8 x 32768 decode + 512-token causal chunk "
                                  "after 4096 tokens, bs 32, 32/8 heads, d 128, bf16, P 512",
                      "ms_per_call": round(ms, 4), "steps": args.steps,
                      "kv_bytes": int(w.kv_bytes),
                      "kv_GBps": round(w.kv_bytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


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
    """HBM bytes per launch of the split kernel, from rocprofv3 counters, if current."""
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    from paged_kv_cache_303_amd import build as pa_build
    if data.get("kernel_source_hash") != pa_build.source_hash():
        return None
    return data.get("bytes_per_launch")


def _cpu_baseline(w, budget_s):
    """The oracle as it stands, on a bounded, seeded sample of the same queries."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import runner as orun

    t0 = time.time()
    ost = orun.replay(w)
    log(f"oracle replay (setup, untimed) {time.time() - t0:.1f}s")
    order = np.random.default_rng(0).permutation(len(w.seq_lens)).tolist()
    done = []  # query evaluations, in seeded order, cycling until the budget is spent
    with threadpool_limits(limits=1):
        start = time.perf_counter()
        while time.perf_counter() - start < budget_s:
            for j in order:
                orun.attention(w, ost, tokens=[j])
                done.append(j)
                if time.perf_counter() - start >= budget_s:
                    break
        elapsed = time.perf_counter() - start
    kv = sum(w.seq_lens[j] for j in done) * w.num_kv_heads * w.head_dim * 2 * 2
    return {
        "value": round(kv / elapsed / 1e9, 4),
        "unit": "GB/s",
        "queries_per_s": round(len(done) / elapsed, 2),
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(done)} decode-query evaluations over the {len(w.seq_lens)} queries "
                  f"(seeded order, repeated), {sum(w.seq_lens[j] for j in done)} keys, "
                  f"{elapsed:.1f}s, float64 NumPy, one thread",
    }


if __name__ == "__main__":
    main()
