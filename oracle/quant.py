"""FP8 (e4m3) KV-cache quantization oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "19.2 KV Cache 系统化管理" §19.2.4 (KV Cache 量化压缩).  The page
lists FP8 and INT8 as one-byte KV formats (half the size of FP16) and says
that each token's KV vector is scaled and quantized on its own, and that
dequantization multiplies the scale back.  The formula itself is missing from
the page, so this module takes the plainest reading of "per-token scaling":

* one scale per (token, KV head), symmetric absmax:
  ``s = max_d |x_d| / 448`` (448 is the largest finite e4m3 value), computed
  in float32 (the precision of the kernel that takes the decision);
* codes ``q_d = e4m3(x_d / s)``, the division in float32, the result clamped
  to [-448, 448] and rounded to the nearest e4m3 value, ties to even;
* dequantized value ``q_d * s``;
* a row of zeros gets ``s = 0`` and all-zero codes;
* the sign of a value is kept in its code, also when it rounds to zero.

The e4m3 format is the OCP 8-bit float "E4M3": 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
``m / 8 * 2^-6``; the all-ones exponent with mantissa 7 (0x7F, 0xFF) is NaN
and there are no infinities, so the largest finite value is
``1.75 * 2^8 = 448`` (0x7E).

Pins (``tests/test_oracle_quant.py``): every code decodes as torch's
``float8_e4m3fn`` does; rounding agrees with torch's cast to that type on
random values and on every midpoint between neighbouring codes; closed forms
(1.0 -> 0x38, 448 -> 0x7E, 2^-9 -> 0x01); quantization invariants (the
absmax element maps to +-448, error at most half a code step times s).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 value of every e4m3 code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    sub = (man / 8.0) * 2.0 ** -6
    val = sign * np.where(exp == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# All finite non-negative code values in increasing order (codes 0x00..0x7E).
_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each (finite, |x| <= 448) value, ties to even.

    Round to nearest by comparing against the exact neighbours in the code
    table (float64 holds every e4m3 value and every float32 input exactly);
    on a tie the code with the even mantissa (even code) wins.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_encode takes finite values in [-448, 448]")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _POS_VALUES[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    # the sign is kept, also when the magnitude rounds to zero (-0 is 0x80)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_rows(x):
    """Per-row symmetric absmax quantization of ``x[..., D]``.

    Returns ``(codes uint8 [..., D], scales float32 [...])`` with the float32
    arithmetic stated in the module docstring.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(y)
    codes = np.where((scale > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale.astype(np.float32)


def dequantize(codes, scales) -> np.ndarray:
    """float64 values ``code * scale`` (scales broadcast over the last axis)."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def scale_pool_shape(num_blocks: int, block_size: int, num_kv_heads: int):
    """Shape of a scale pool: one float32 per (block, KV head, row of the block),
    the rows of one head contiguous (``[NB, Hkv, bs]``)."""
    return (num_blocks, num_kv_heads, block_size)


def dequantize_pool(codes, scales) -> np.ndarray:
    """float64 values of a code pool ``[NB, bs, Hkv, D]`` with its scale pool
    ``[NB, Hkv, bs]``: ``code * scale`` of the same (block, row, head)."""
    return dequantize(codes, np.asarray(scales).transpose(0, 2, 1))


def kv_write_fp8(k_codes, v_codes, k_scales, v_scales, k_new, v_new, slot_mapping,
                 block_size: int) -> None:
    """In place: quantize token t's K and V rows (per KV head) into slot s >= 0.

    Pools: codes ``[NB, bs, Hkv, D]`` uint8, scales ``[NB, Hkv, bs]`` float32
    (``scale_pool_shape``); new tokens ``[T, Hkv, D]`` as float32 values
    (bf16 inputs widened).
    """
    kc, ks = quantize_rows(k_new)
    vc, vs = quantize_rows(v_new)
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if s < 0:
            continue
        block, off = divmod(s, block_size)
        k_codes[block, off] = kc[t]
        v_codes[block, off] = vc[t]
        k_scales[block, :, off] = ks[t]
        v_scales[block, :, off] = vs[t]
