"""Pins for the oracle's E4M3 codec and per-tensor scale rule (CPU only).

Fixed outside the oracle by: the values the OCP 8-bit floating point
specification lists for E4M3 (largest normal 448, smallest normal 2^-6,
largest subnormal 0.875 * 2^-6, smallest subnormal 2^-9, NaN = S.1111.111),
and torch's float8_e4m3fn conversion (a library routine) on every code and on
every rounding midpoint inside the finite range.
"""

import numpy as np
import pytest
import torch

from oracle import fp8_ref as f8


def test_spec_values():
    t = f8.e4m3_decode_table()
    assert t[0x7E] == 448.0
    assert t[0x08] == 2.0 ** -6
    assert t[0x07] == 0.875 * 2.0 ** -6
    assert t[0x01] == 2.0 ** -9
    assert t[0x38] == 1.0
    assert t[0xC0] == -2.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.sum(np.isnan(t)) == 2


def test_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = f8.e4m3_decode_table()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(tv))
    ok = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[ok], tv[ok])


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_midpoints_and_neighbours():
    pos = f8.e4m3_decode_table()[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([pos, mids])
    vals32 = vals.astype(np.float32)
    # one fp32 ulp either side of every midpoint and value
    nb = np.concatenate([np.nextafter(vals32, np.float32(np.inf)), np.nextafter(vals32, np.float32(0))])
    allv = np.concatenate([vals32, nb]).astype(np.float32)
    allv = allv[np.abs(allv) <= 448.0]
    allv = np.concatenate([allv, -allv])
    np.testing.assert_array_equal(f8.e4m3_encode(allv), torch_encode(allv))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-12, 6, 200000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    np.testing.assert_array_equal(f8.e4m3_encode(x), torch_encode(x))


def test_saturation():
    codes = f8.e4m3_encode(np.array([448.0, 450.0, 463.9, 464.0, 1e4, -1e6], np.float32))
    np.testing.assert_array_equal(codes, np.array([0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE], np.uint8))


def test_ties_to_even():
    # 1 + 1/16 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): goes to 1.0
    # 1 + 3/16 halfway between 1.125 (odd) and 1.25 (0x3A, even): goes to 1.25
    codes = f8.e4m3_encode(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11], np.float32))
    np.testing.assert_array_equal(codes, np.array([0x38, 0x3A, 0x00, 0x01], np.uint8))


@pytest.mark.parametrize("seed", [0, 1])
def test_per_tensor_quantization(seed):
    """scale = 448 / (amax + 1e-12) in fp32; the largest element lands on 448;
    every element is within half an E4M3 step of x * scale."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal(50000).astype(np.float32) * 3).to(torch.bfloat16).float().numpy()
    codes, scale, amax = f8.quantize_per_tensor(x)
    assert amax == np.float32(np.abs(x).max())
    assert scale == np.float32(np.float32(448.0) / (amax + np.float32(1e-12)))
    assert f8.e4m3_decode(codes).max() == 448.0 or f8.e4m3_decode(codes).min() == -448.0
    y = x.astype(np.float64) * np.float64(scale)
    err = np.abs(f8.e4m3_decode(codes) - y)
    # half a step: 2^-4 relative for normals, 2^-10 absolute for subnormals
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-6)
    np.testing.assert_allclose(f8.dequantize(codes, scale), f8.e4m3_decode(codes) / float(scale))


def test_zero_tensor_scale_is_finite():
    codes, scale, amax = f8.quantize_per_tensor(np.zeros(16, np.float32))
    assert amax == 0 and np.isfinite(scale) and np.all(codes == 0)


def test_nan_and_infinity_codes():
    """NaN has the codes S.1111.111 in the format; the encoder writes 0xFF for
    every NaN (torch agrees the code decodes to NaN), and infinities saturate
    like every other magnitude at or past 464."""
    codes = f8.e4m3_encode(np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0]))
    np.testing.assert_array_equal(codes, np.array([0xFF, 0xFF, 0x7E, 0xFE, 0x00, 0x80], np.uint8))
    tv = torch.tensor([0xFF], dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    assert torch.isnan(tv).all()
    assert torch_encode(np.array([np.nan]))[0] & 0x7F == 0x7F   # torch's NaN is a NaN code too


def _planted_fmax_quantize(x, fp8_max=448.0, eps=1e-12):
    """A plausible mistake: Amax taken with a NaN-dropping max (like fmaxf)."""
    xf = np.asarray(x, np.float32)
    amax = np.float32(np.nanmax(np.abs(xf)))
    scale = f8.per_tensor_scale(amax, fp8_max, eps)
    return f8.e4m3_encode((np.nan_to_num(xf) * scale).astype(np.float32)), scale, amax


def test_per_tensor_nan_poisons_the_tensor():
    """One NaN makes Amax, the scale and every code NaN, so a diverging step
    cannot hide behind finite codes; the NaN-dropping max fails this."""
    x = np.linspace(-3, 3, 101).astype(np.float32)
    x[17] = np.nan
    codes, scale, amax = f8.quantize_per_tensor(x)
    assert np.isnan(amax) and np.isnan(scale)
    assert np.all(codes == 0xFF)
    pc, ps, pa = _planted_fmax_quantize(x)
    assert not np.all(pc == 0xFF) and np.isfinite(ps)


def test_per_tensor_infinity():
    """An infinity makes Amax inf and the scale 0: finite elements go to signed
    zero, the infinities (inf * 0) to NaN."""
    x = np.array([1.5, -2.0, np.inf, 0.25, -np.inf], np.float32)
    codes, scale, amax = f8.quantize_per_tensor(x)
    assert np.isinf(amax) and scale == 0.0
    np.testing.assert_array_equal(codes, np.array([0x00, 0x80, 0xFF, 0x00, 0xFF], np.uint8))


def test_unit_scale_with_eps_zero():
    """fp8_max equal to the tensor's Amax and eps = 0 give the scale 1.0 exactly,
    so the codes are the plain encoding of the values (the setting the device
    edge-case test uses)."""
    vals = np.array([448.0, -3.1, 2.0 ** -9, 2.0 ** -10, 0.0], np.float32)
    codes, scale, amax = f8.quantize_per_tensor(vals, fp8_max=448.0, eps=0.0)
    assert scale == 1.0 and amax == 448.0
    np.testing.assert_array_equal(codes, f8.e4m3_encode(vals))
    big = np.array([1000.0, 455.0, 464.0, -470.0], np.float32)
    codes, scale, amax = f8.quantize_per_tensor(big, fp8_max=1000.0, eps=0.0)
    assert scale == 1.0
    np.testing.assert_array_equal(codes, np.array([0x7E, 0x7E, 0x7E, 0xFE], np.uint8))
