"""Pins for the oracle's timed CPU baseline and for the part-wise dequantizer
the 8-bit GPU tests use (CPU only).

- ``cpu_baseline.run_units`` is the same method as ``skiparse_attention`` in
  fp32 BLAS blocks: run on every unit it must reproduce the float64 literal
  pad -> rearrange -> attention -> inverse path (itself pinned to block-masked
  brute force) within fp32 rounding, in both patterns and with padding, and
  its pair count must be the closed-form count.  A baseline that timed a wrong
  scale or a wrong subsequence would fail here.
- ``skiparse_bwd.dequantized_part`` forms a slice of a tensor quantized as a
  whole; it must equal the whole tensor's per-tensor quantization
  (``fp8_ref.quantize_per_tensor``), sliced.  The plausible mistake of scaling
  the slice by its own maximum is planted and must fail.
"""

import numpy as np
import pytest

import workloads as wl
from oracle import cpu_baseline as cb
from oracle import fp8_ref as f8
from oracle import skiparse_bwd as bwd
from oracle import skiparse_ref as ref


def _qkv(shape, seed):
    return [wl.normal_tensor(shape, seed, i).astype(np.float32) for i in range(3)]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape,kf", [((1, 2, 7, 10, 2, 64), 2), ((2, 1, 9, 9, 1, 128), 3),
                                      ((1, 3, 4, 6, 2, 64), 1)])
def test_run_units_matches_literal_attention(shape, kf, mode):
    B, T, H, W, nh, d = shape
    q, k, v = _qkv(shape, 11)
    want = ref.skiparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), kf, mode)
    N = T * H * W
    flat = [x.reshape(B, N, nh, d) for x in (q, k, v)]
    units = [(b, h, s) for b in range(B) for h in range(nh) for s in range(kf * kf)]
    got, pairs = cb.run_units(*flat, T, H, W, kf, mode, units, block=17)   # ragged query blocks
    got = got.reshape(shape)
    assert pairs * 1 == ref.pair_count(B, T, H, W, nh, kf, mode)
    err = np.max(np.abs(got - want)) / max(1.0, np.max(np.abs(want)))
    assert err < 1e-5, err


def test_run_units_partial_and_wrong_scale_detected():
    """A subset of units writes exactly those units' rows, and a wrong softmax
    scale (a plausible mistake) is outside the bar."""
    shape = (1, 2, 6, 10, 2, 64)
    B, T, H, W, nh, d = shape
    q, k, v = _qkv(shape, 12)
    N = T * H * W
    flat = [x.reshape(B, N, nh, d) for x in (q, k, v)]
    want = ref.skiparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 2, 0)
    want = want.reshape(B, N, nh, d)
    units = [(0, 1, 2), (0, 0, 3)]
    got, pairs = cb.run_units(*flat, T, H, W, 2, 0, units)
    mem = ref.subsequence_members(T, H, W, 2, 0)
    assert pairs == mem[2].size ** 2 + mem[3].size ** 2
    for (b, h, s) in units:
        np.testing.assert_allclose(got[b, mem[s], h], want[b, mem[s], h], atol=1e-5)
    untouched = np.ones((N, nh), bool)
    for (b, h, s) in units:
        untouched[mem[s], h] = False
    assert np.all(got[0][untouched] == 0)
    bad, _ = cb.run_units(*flat, T, H, W, 2, 0, units, scale=1.0)
    assert np.max(np.abs(bad[0, mem[2], 1] - want[0, mem[2], 1])) > 1e-3


def test_time_sample_counts_pairs():
    shape = (1, 2, 8, 8, 2, 64)
    B, T, H, W, nh, d = shape
    q, k, v = _qkv(shape, 13)
    flat = [x.reshape(B, T * H * W, nh, d) for x in (q, k, v)]
    units = [(0, h, s) for h in range(nh) for s in range(4)]
    sec, pairs = cb.time_sample(*flat, T, H, W, 2, 1, units, repeats=2)
    assert sec > 0 and pairs == ref.pair_count(B, T, H, W, nh, 2, 1)


def _own_amax_part(part, fp8_max=448.0, eps=1e-12):
    """Planted mistake: the slice scaled by its own maximum."""
    p = np.asarray(part, np.float32)
    return bwd.dequantized_part(p, np.float32(np.max(np.abs(p))), fp8_max, eps)


@pytest.mark.parametrize("fp8_max", [448.0, 224.0])
def test_dequantized_part_equals_whole_tensor_slice(fp8_max):
    x = wl.normal_tensor((1, 3, 5, 7, 4, 64), 21, 0).astype(np.float32)
    x[0, 1, 2, 3, 2, 9] = 40.0                  # the whole tensor's maximum, outside the slices below
    codes, scale, amax = f8.quantize_per_tensor(x.ravel(), fp8_max=fp8_max)
    whole = f8.dequantize(codes, scale).reshape(x.shape)
    for sl in [np.s_[:, :, :, :, 0:1], np.s_[:, 0], np.s_[..., 32:], np.s_[:, 2, 4, 6]]:
        got = bwd.dequantized_part(x[sl], amax, fp8_max=fp8_max)
        np.testing.assert_array_equal(got, whole[sl])
        assert not np.array_equal(_own_amax_part(x[sl], fp8_max), whole[sl])
