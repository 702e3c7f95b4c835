"""The device's per-tensor e4m3 quantizer on the conversion's edge cases,
bit for bit against the oracle's codec (itself pinned to the OCP E4M3
definition and torch's float8_e4m3fn in test_oracle_fp8.py).

The scale rule is FP8max / (Amax + eps) over the whole tensor (OSP-Next
summary, 方法步骤详情 method steps).  Setting fp8_max to the tensor's own Amax
and eps to 0 makes the scale exactly 1.0, so each code is the conversion of
the input value itself and the rounding of the device's conversion is seen
directly:
- every finite e4m3 value, every rounding midpoint between neighbours, and
  one fp32 ulp either side of each (ties to even, and no drift next to them);
- the subnormal range on a grid four times finer than its step;
- +0 and -0;
- magnitudes from 448 up to 1000 (saturation, the 464 midpoint included),
  in a second tensor whose Amax is 1000;
- a NaN (it must poison Amax, the scale and every code) and an infinity.
"""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
from oracle import fp8_ref as f8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _in_range_values():
    pos = f8.e4m3_decode_table()[:127].astype(np.float32)            # 0 .. 448, increasing
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    base = np.concatenate([pos, mids])
    up = np.nextafter(base, np.float32(np.inf))
    down = np.nextafter(base, np.float32(0))
    sub = (np.arange(0, 4 * 8 + 1, dtype=np.float64) * 2.0 ** -11).astype(np.float32)   # [0, 2^-6] by 2^-11
    v = np.concatenate([base, up, down, sub])
    v = v[np.abs(v) <= 448.0]
    v = np.concatenate([v, -v, np.array([0.0, -0.0, 448.0, -448.0], np.float32)])
    return v.astype(np.float32)


def _device_quant(x_np, torch_dtype, fp8_max, eps):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(torch_dtype).to(DEV)
    y = torch.empty(x.numel(), dtype=torch.uint8, device=DEV)
    sc = torch.empty(2, dtype=torch.float32, device=DEV)
    sk.skiparse_quant_fp8(x, y, sc, fp8_max, eps)
    torch.cuda.synchronize()
    return y.cpu().numpy(), sc.cpu().numpy()


def _check(x_np, torch_dtype, fp8_max, eps, want_scale=None):
    xin = torch.from_numpy(x_np).to(torch_dtype).float().numpy()    # the values the device sees
    codes, scale, amax = f8.quantize_per_tensor(xin, fp8_max=fp8_max, eps=eps)
    got, sc = _device_quant(x_np, torch_dtype, fp8_max, eps)
    if want_scale is not None:
        assert np.array_equal(np.float32(scale), np.float32(want_scale), equal_nan=True)
    assert np.array_equal(sc[0], np.float32(scale), equal_nan=True), (sc, scale)
    bad = np.nonzero(got != codes)[0]
    assert bad.size == 0, [(float(xin[i]), int(got[i]), int(codes[i])) for i in bad[:10]]
    return got


@pytest.mark.parametrize("perm_seed", [None, 5])
def test_every_value_midpoint_and_neighbour_fp32(perm_seed):
    v = _in_range_values()
    if perm_seed is not None:   # the same values at other positions and vector lanes
        v = v[np.random.default_rng(perm_seed).permutation(v.size)]
    got = _check(v, torch.float32, 448.0, 0.0, want_scale=1.0)
    # the codes of the exact values are the values themselves
    pos = f8.e4m3_decode_table()[:127].astype(np.float32)
    idx = {float(x): i for i, x in enumerate(v)}
    for c in range(1, 127):   # 0.0 and -0.0 share one dict key; zeros are checked on their own
        assert got[idx[float(pos[c])]] == c


def test_signed_zeros_fp32():
    v = np.array([0.0, -0.0] * 8 + [448.0], np.float32)
    got = _check(v, torch.float32, 448.0, 0.0, want_scale=1.0)
    np.testing.assert_array_equal(got[:16], np.array([0x00, 0x80] * 8, np.uint8))


def test_values_and_midpoints_bf16():
    """bf16 input (widened exactly on the device): the e4m3 values, their
    midpoints and the bf16 neighbours of each are all bf16 numbers."""
    v = _in_range_values()
    vb = torch.from_numpy(v).to(torch.bfloat16)
    vf = vb.float().numpy()
    nb_up = (vb.view(torch.int16) + 1).view(torch.bfloat16).float().numpy()
    v2 = np.concatenate([vf, nb_up])
    v2 = v2[np.isfinite(v2) & (np.abs(v2) <= 448.0)]
    _check(v2.astype(np.float32), torch.bfloat16, 448.0, 0.0, want_scale=1.0)


def test_saturation_band():
    """Magnitudes past 448 saturate to +-448: the band up to the 464 midpoint,
    the midpoint itself, and beyond, with Amax = fp8_max = 1000 (scale 1)."""
    band = np.array([448.0, 450.0, 455.5, 456.0, 463.0, 464.0, 464.5, 470.0, 480.0, 512.0, 999.0, 1000.0],
                    np.float32)
    near = np.concatenate([np.nextafter(band, np.float32(0)), np.nextafter(band, np.float32(np.inf))])
    v = np.concatenate([band, near, np.array([1.0, 0.5, -3.0], np.float32)])
    v = v[np.abs(v) <= 1000.0]
    v = np.concatenate([v, -v]).astype(np.float32)
    got = _check(v, torch.float32, 1000.0, 0.0, want_scale=1.0)
    big = np.abs(v) >= 448.0
    np.testing.assert_array_equal(got[big] & 0x7F, np.full(int(big.sum()), 0x7E, np.uint8))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("where", [0, 4097, 70000])
def test_nan_poisons_the_tensor(dtype, where):
    v = np.linspace(-5, 5, 70001).astype(np.float32)
    v[where] = np.nan
    got = _check(v, dtype, 448.0, 1e-12)
    assert np.all(got == 0xFF)


def test_infinity():
    v = np.linspace(-5, 5, 4099).astype(np.float32)
    v[123] = np.inf
    v[4000] = -np.inf
    got = _check(v, torch.float32, 448.0, 1e-12, want_scale=0.0)
    assert got[123] == 0xFF and got[4000] == 0xFF
