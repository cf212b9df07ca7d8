"""Pins for the oracle's storage decoders (CPU only).

E4M3: all 256 codes against torch's float8_e4m3fn (a library definition of the
same OCP format) and spot values from the field formula.  bf16: random bit
patterns against torch.bfloat16 widening.
"""

import numpy as np
import pytest
import torch

from oracle.codecs import bf16_bits_to_f64, e4m3fn_codes_to_f64, decode_storage


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_codes_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours = np.isnan(ours)
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert nan_ours.sum() == 2 and nan_ours[0x7F] and nan_ours[0xFF]
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    # signed zeros
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x40, 2.0),
    (0x3C, 1.5), (0x77, 240.0),
])
def test_e4m3_spot_values(code, value):
    assert e4m3fn_codes_to_f64(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3_monotone_over_positive_codes():
    v = e4m3fn_codes_to_f64(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0x3F80],
                                          dtype=np.uint16)])
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert bf16_bits_to_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0


def test_decode_storage_f32_passthrough():
    x = np.array([1.5, -2.25, np.float32(1e-40)], dtype=np.float32)
    assert np.array_equal(decode_storage(x, "f32"), x.astype(np.float64))
    with pytest.raises(ValueError):
        decode_storage(x, "fp4")
