"""Pins for the oracle's FP8 e4m3fn and bf16 decoding.

The e4m3fn decoder is the format's closed form; it is checked against the
format's fixed special values and against torch's independent float8_e4m3fn
conversion for all 256 codes.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, dequantize, e4m3fn_decode


def test_all_256_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert nan_ours.sum() == 2                       # S.1111.111 only
    np.testing.assert_array_equal(ours[~nan_ours], ref[~nan_ref])
    # sign of zero must survive as well
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0),             # e=7, m=0
    (0x7E, 448.0),           # largest finite: 2^8 * 1.75
    (0xFE, -448.0),
    (0x08, 2.0 ** -6),       # smallest normal
    (0x01, 2.0 ** -9),       # smallest subnormal: 2^-6 * 1/8
    (0x07, 7 * 2.0 ** -9),   # largest subnormal
    (0x3C, 1.5),
    (0x40, 2.0),
    (0xB8, -1.0),
    (0x30, 0.5),
])
def test_closed_form_values(code, value):
    assert e4m3fn_decode(np.array([code], dtype=np.uint8))[0] == value


def test_nan_codes_and_no_infinity():
    v = e4m3fn_decode(np.array([0x7F, 0xFF, 0x78, 0xF8], dtype=np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1])
    # 0x78 = S.1111.000 is a finite number in the fn variant (256), not infinity
    assert v[2] == 256.0 and v[3] == -256.0


def test_dequantize_scales_each_leading_row():
    codes = np.full((3, 2, 4), 0x38, dtype=np.uint8)          # all 1.0
    scales = np.array([0.5, 2.0, 3.0], dtype=np.float32)
    x = dequantize(codes, scales)
    assert x.shape == (3, 2, 4)
    for r in range(3):
        assert (x[r] == scales[r]).all()


def test_bf16_bits_match_torch():
    g = torch.Generator().manual_seed(7)
    vals = torch.randn(4096, generator=g) * 100
    bits = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = vals.to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
