"""Pins for oracle.fp8 (CPU only).

The e4m3fn codec is checked against torch's own float8_e4m3fn conversion
(a library routine) exhaustively, and against values the OCP 8-bit float
specification fixes (1.0, 448, the smallest normal and subnormal).
"""
import numpy as np
import pytest
import torch

from oracle import fp8


def _all_finite_bf16_as_f32():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).float()
    return x[torch.isfinite(x)]


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    # NaN only at 0x7f / 0xff (e4m3fn has no infinities).
    assert set(np.flatnonzero(np.isnan(ours)).tolist()) == {0x7F, 0xFF}


def test_decode_spec_values():
    # OCP OFP8 E4M3: bias 7; 0x38 = 1.0, 0x7e = 448 (max), 0x08 = 2^-6 (min normal),
    # 0x01 = 2^-9 (min subnormal), 0x80 = -0.
    d = fp8.decode(np.array([0x38, 0x7E, 0x08, 0x01, 0xB8, 0x80], dtype=np.uint8))
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -6 and d[3] == 2.0 ** -9
    assert d[4] == -1.0 and d[5] == 0.0 and np.signbit(d[5])


@pytest.mark.parametrize("inv_scale", [1.0, 448.0 / 3.75, 448.0 / 5.3125, 0.37, 1000.0, 2.0 ** -7])
def test_quantize_exhaustive_bf16_vs_torch(inv_scale):
    x = _all_finite_bf16_as_f32()
    inv = np.float32(inv_scale)
    ours = fp8.quantize(x.numpy(), inv)
    y = (x * torch.tensor(inv, dtype=torch.float32)).clamp(-448.0, 448.0)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_ties_to_even():
    # Between 1.0 (0x38) and 1.125 (0x39): 1.0625 is a tie -> even code 0x38;
    # between 1.125 and 1.25 (0x3a): 1.1875 is a tie -> 0x3a.
    c = fp8.encode(np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10]))
    assert c.tolist() == [0x38, 0x3A, 0xB8, 0x00, 0x02]


def test_scales():
    s, inv = fp8.scales_from_amax(np.float32(3.75))
    assert s == np.float32(3.75) / np.float32(448.0)
    assert inv == np.float32(448.0) / np.float32(3.75)
    assert fp8.scales_from_amax(0.0) == (1.0, 1.0)
    # the amax element maps to +-448 exactly or within one rounding of it
    x = np.array([3.75, -3.75, 1.0], dtype=np.float32)
    codes = fp8.quantize(x, inv)
    assert fp8.decode(codes)[0] == 448.0 and fp8.decode(codes)[1] == -448.0


def test_amax_over_shards():
    a = [np.array([[1.0, -7.5]]), np.array([[3.0, 2.0]]), np.zeros((0,))]
    assert fp8.amax(a) == np.float32(7.5)
