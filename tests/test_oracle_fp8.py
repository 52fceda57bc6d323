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


def _dequant_attention_case(seed, amax_q, amax_k, softmax_scale):
    """fp8 codes of random q/k with per-tensor scales from the given amax values."""
    from oracle import attention as oa
    g = np.random.default_rng(seed)
    q = (g.standard_normal((1, 40, 2, 64)) * amax_q / 4).clip(-amax_q, amax_q)
    k = (g.standard_normal((1, 56, 2, 64)) * amax_k / 4).clip(-amax_k, amax_k)
    v = g.standard_normal((1, 56, 2, 64))
    sq, iq = fp8.scales_from_amax(amax_q)
    sk, ik = fp8.scales_from_amax(amax_k)
    qc, kc = fp8.quantize(q, iq), fp8.quantize(k, ik)
    return oa, qc, kc, v, sq, sk


@pytest.mark.parametrize("amax_q,amax_k,softmax_scale", [(3.75, 5.3125, 0.125), (0.02, 17.0, 0.0883883476),
                                                        (448.0, 1.0, 0.3), (1.0, 1.0, 0.125)])
def test_score_scale_is_the_dequantised_attention(amax_q, amax_k, softmax_scale):
    """LightX2V "Add optimized Ulysses attention path": the fp8 payload travels with its scale and
    the receiver dequantises with it.  Attention on the dequantised tensors (decode(code) * scale,
    exact in fp64) must equal attention on the raw codes with the folded score multiplier, up to
    the float32 rounding of that multiplier (two roundings: relative <= 2^-23)."""
    oa, qc, kc, v, sq, sk = _dequant_attention_case(3, amax_q, amax_k, softmax_scale)
    qd, kd = fp8.decode(qc), fp8.decode(kc)
    o_ref, lse_ref = oa.attention(qd * float(sq), kd * float(sk), v, softmax_scale)
    c = fp8.score_scale(softmax_scale, sq, sk)
    o, lse = oa.attention(qd, kd, v, float(c))
    exact = float(np.float32(softmax_scale)) * float(sq) * float(sk)
    assert abs(float(c) - exact) <= 2.0 ** -22 * exact
    # scores are at most a few units, so an O(2^-22) relative change of c moves lse and o by ~1e-6
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-5)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-5)


def test_score_scale_rounding_order():
    """The multiplier is float32((float32(softmax_scale * q_scale)) * k_scale): with unit scales it is
    the float32 softmax scale itself, and a planted mistake (using the inverse scales) is far off."""
    assert fp8.score_scale(0.1, np.float32(1), np.float32(1)) == np.float32(0.1)
    sq, iq = fp8.scales_from_amax(3.75)
    sk, ik = fp8.scales_from_amax(5.3125)
    assert fp8.score_scale(0.125, sq, sk) == np.float32(np.float32(np.float32(0.125) * sq) * sk)
    assert abs(float(fp8.score_scale(0.125, iq, ik)) / float(fp8.score_scale(0.125, sq, sk)) - 1) > 1.0


def test_scales_from_amax_definition():
    """scale = amax / 448 and inv = 448 / amax in float32; amax = 0 gives 1 and 1; decode(448 * inv)
    recovers the largest element."""
    for a in (3.75, 0.02, 17.0, 448.0, 1e-3):
        s, i = fp8.scales_from_amax(a)
        assert s == np.float32(np.float32(a) / np.float32(448.0))
        assert i == np.float32(np.float32(448.0) / np.float32(a))
        code = fp8.quantize(np.array([a, -a]), i)
        assert abs(fp8.decode(code)[0] * float(s) - a) <= a * 2.0 ** -3
        assert fp8.decode(code)[0] == 448.0 or abs(fp8.decode(code)[0] - 448.0) <= 32.0
    assert fp8.scales_from_amax(0.0) == (np.float32(1.0), np.float32(1.0))
