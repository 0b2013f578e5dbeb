"""Pins of the FP8 (e4m3) quantization oracle ("19.2 KV Cache 系统化管理" §19.2.4).

The e4m3 code table and its rounding are pinned to a library routine (torch's
``float8_e4m3fn``), to closed forms of the format, and the per-token absmax
quantization to invariants that a dropped term, a wrong sign or a wrong bias
would break.
"""

import numpy as np
import pytest
import torch

from oracle import quant as qn


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = qn.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.isnan(got).sum() == 2  # 0x7F and 0xFF only


def test_closed_forms():
    enc = lambda v: int(qn.e4m3_encode(np.array([v]))[0])
    assert enc(1.0) == 0x38          # exponent field 7 = bias, mantissa 0
    assert enc(448.0) == 0x7E        # largest finite: 1.75 * 2^8
    assert enc(-448.0) == 0xFE
    assert enc(2.0 ** -9) == 0x01    # smallest subnormal: 1/8 * 2^-6
    assert enc(2.0 ** -6) == 0x08    # smallest normal
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert qn.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert qn.e4m3_decode(np.array([0x07], np.uint8))[0] == 7 / 8 * 2.0 ** -6


def test_rounding_matches_torch_random_and_midpoints():
    rng = np.random.default_rng(0)
    x = np.clip(rng.standard_normal(50000).astype(np.float32) * 40, -448, 448)
    assert np.array_equal(qn.e4m3_encode(x), _torch_encode(x))
    v = qn._POS_VALUES
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)  # exact in f32
    for m in (mids, -mids):
        assert np.array_equal(qn.e4m3_encode(m), _torch_encode(m))
    # ties go to the even code: 1.0625 lies between 0x38 (1.0) and 0x39 (1.125)
    assert int(qn.e4m3_encode(np.array([1.0625]))[0]) == 0x38
    assert int(qn.e4m3_encode(np.array([1.1875]))[0]) == 0x3A


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        qn.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        qn.e4m3_encode(np.array([np.nan]))


def test_quantize_rows_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 8, 128)).astype(np.float32)
    codes, scales = qn.quantize_rows(x)
    assert codes.shape == x.shape and scales.shape == x.shape[:2]
    amax = np.abs(x).max(-1)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    # the absmax element of every row maps to +-448, with its sign
    idx = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    sign = np.take_along_axis(x, idx[..., None], -1)[..., 0] < 0
    assert np.array_equal(top, np.where(sign, 0xFE, 0x7E).astype(np.uint8))
    # error of every value: at most half the code step at its magnitude, times s
    deq = qn.dequantize(codes, scales)
    y = x / scales[..., None].astype(np.float64)
    v = qn._POS_VALUES
    hi = np.minimum(np.searchsorted(v, np.abs(y)), len(v) - 1)
    step = v[hi] - v[np.maximum(hi - 1, 0)]
    assert (np.abs(deq - x) <= 0.5 * step * scales[..., None] * (1 + 1e-6) + 1e-12).all()
    # relative error of a row's dot product stays small (3 mantissa bits)
    assert np.abs(deq - x).max() <= 0.0625 * amax.max()


def test_quantize_zero_row_and_sign():
    x = np.zeros((2, 16), np.float32)
    x[1, 3] = -2.5
    codes, scales = qn.quantize_rows(x)
    assert scales[0] == 0 and (codes[0] == 0).all()
    assert codes[1, 3] == 0xFE and scales[1] == np.float32(2.5) / np.float32(448)
    assert (np.delete(codes[1], 3) == 0).all()


def test_planted_mistakes_are_caught():
    # a bias of 8 (the other common 8-bit e4m3 variant) moves 1.0 to 0x40
    def decode_bias8(c):
        c = np.asarray(c, np.int64)
        e, m = (c >> 3) & 0xF, c & 7
        return np.where(e == 0, m / 8 * 2.0 ** -7, (1 + m / 8) * np.exp2(e - 8.0))
    assert decode_bias8([0x38])[0] != qn.e4m3_decode(np.array([0x38], np.uint8))[0]
    # dropping the scale (codes read as values) is far from the input
    x = np.random.default_rng(2).standard_normal((4, 64)).astype(np.float32)
    codes, scales = qn.quantize_rows(x)
    assert np.abs(qn.e4m3_decode(codes) - x).max() > 1.0
    assert np.abs(qn.dequantize(codes, scales) - x).max() < 0.2


def test_kv_write_fp8_places_rows():
    rng = np.random.default_rng(3)
    nb, bs, hkv, d = 4, 4, 2, 16
    kc = np.zeros((nb, bs, hkv, d), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.full(qn.scale_pool_shape(nb, bs, hkv), np.nan, np.float32)  # [NB, Hkv, bs]
    vs = ks.copy()
    k_new = rng.standard_normal((3, hkv, d)).astype(np.float32)
    v_new = rng.standard_normal((3, hkv, d)).astype(np.float32)
    qn.kv_write_fp8(kc, vc, ks, vs, k_new, v_new, [5, -1, 14], bs)
    c0, s0 = qn.quantize_rows(k_new[0])
    assert np.array_equal(kc[1, 1], c0) and np.array_equal(ks[1, :, 1], s0)
    c2, s2 = qn.quantize_rows(v_new[2])
    assert np.array_equal(vc[3, 2], c2) and np.array_equal(vs[3, :, 2], s2)
    assert np.isnan(ks).sum() == (nb * bs - 2) * hkv  # only the two slots written
    # the pool dequantizes row by row: slot 5's K values are its codes times its scales
    deq = qn.dequantize_pool(kc, ks)
    assert np.array_equal(deq[1, 1], qn.dequantize(c0, s0))
