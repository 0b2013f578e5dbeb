"""Tolerances and comparisons for GPU-vs-oracle parity.

* fp32 inputs: |gpu - oracle| <= 1e-5 everywhere (the bound of the pages'
  worked example, "19.2 KV Cache 系统化管理" §19.2.3).
* bf16 inputs, fp32 accumulation, bf16 output:
  |gpu - oracle| <= 1e-2 + 2e-2 * |oracle| elementwise.  The oracle works on
  the same stored bf16 values (widened exactly), so input rounding is shared;
  what remains is fp32 accumulation order (~1e-6 relative) and the final
  bf16 rounding of the output (<= 2^-9 relative).
* Integer and byte results (tables, slots, pools): bit for bit.
"""

from __future__ import annotations

import numpy as np
import torch

F32_ATOL = 1e-5
BF16_ATOL = 1e-2
BF16_RTOL = 2e-2


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check_attention(gpu: torch.Tensor, ref: np.ndarray, dtype: str, rows=None, what=""):
    """Elementwise parity of attention outputs; returns (max_err, max_err / rms(ref))."""
    g = to_f64(gpu)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    if dtype == "f32":
        bad = err > F32_ATOL
    else:
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at "
                             f"{tuple(idx)}: gpu {g[tuple(idx)]!r} oracle {ref[tuple(idx)]!r}; "
                             f"max err {err.max():.3e}")
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    return float(err.max()), float(err.max()) / rms


def pools_equal_bits(gpu_pool: torch.Tensor, oracle_pool: np.ndarray) -> bool:
    """Bit-for-bit equality of a device pool and an oracle pool (NaN bits included)."""
    if gpu_pool.dtype == torch.bfloat16:
        ref = torch.from_numpy(oracle_pool.view(np.int16)).to(gpu_pool.device)
        return bool(torch.equal(gpu_pool.view(torch.int16), ref))
    ref = torch.from_numpy(oracle_pool.view(np.int32)).to(gpu_pool.device)
    return bool(torch.equal(gpu_pool.view(torch.int32), ref))
