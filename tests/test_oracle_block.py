"""Pins of the fp8 attention-block oracle (oracle/block_ref.py): the rotary
embedding against its defining properties, and the block against
compositions that reduce it to pieces pinned elsewhere."""

import numpy as np
import pytest

import workloads as wl
from oracle import block_ref as blk
from oracle import fp8_ref as f8
from oracle import skiparse_ref as ref


def rnd(shape, seed, i):
    return wl.normal_tensor(shape, seed, i).astype(np.float64)


def test_rope_dims_split():
    assert blk.rope_dims(128) == (44, 42, 42)
    assert blk.rope_dims(64) == (24, 20, 20)
    for d in (64, 96, 128):
        assert sum(blk.rope_dims(d)) == d


def test_rope_identity_at_origin_and_norms():
    x = rnd((1, 3, 4, 5, 2, 128), 701, 0)
    r = blk.rope_3d(x)
    np.testing.assert_allclose(r[:, 0, 0, 0], x[:, 0, 0, 0], rtol=0, atol=0)   # position (0, 0, 0)
    pairs = lambda y: y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(pairs(r), pairs(x), rtol=1e-12)


def test_rope_single_pair_closed_form():
    d = 128
    x = np.zeros((1, 2, 1, 1, 1, d))
    x[..., 0] = 1.0                 # first pair of the t part, i = 0: angle = t
    r = blk.rope_3d(x)
    np.testing.assert_allclose(r[0, 1, 0, 0, 0, :2], [np.cos(1.0), np.sin(1.0)], rtol=1e-15)
    x = np.zeros((1, 1, 1, 3, 1, d))
    dt, dh, dw = blk.rope_dims(d)
    x[..., dt + dh + 2] = 1.0       # pair i = 1 of the w part: angle = w * 10000^(-2/dw)
    r = blk.rope_3d(x)
    a = 2 * 10000.0 ** (-2.0 / dw)
    np.testing.assert_allclose(r[0, 0, 0, 2, 0, dt + dh + 2:dt + dh + 4], [np.cos(a), np.sin(a)], rtol=1e-14)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_scores_depend_on_offsets_only(axis):
    """<R(q, p), R(k, p')> is unchanged when both positions move by the same
    amount along one axis (the property that makes the embedding relative)."""
    T, H, W, d = 6, 5, 7, 128
    q1 = rnd((d,), 702, 0)
    k1 = rnd((d,), 702, 1)
    grid_q = np.zeros((1, T, H, W, 1, d))
    grid_k = np.zeros((1, T, H, W, 1, d))
    grid_q[...] = q1
    grid_k[...] = k1
    rq, rk = blk.rope_3d(grid_q)[0, ..., 0, :], blk.rope_3d(grid_k)[0, ..., 0, :]
    p, pk = [1, 2, 3], [0, 1, 4]
    shift = [0, 0, 0]
    shift[axis] = 2
    s0 = rq[p[0], p[1], p[2]] @ rk[pk[0], pk[1], pk[2]]
    s1 = rq[p[0] + shift[0], p[1] + shift[1], p[2] + shift[2]] @ rk[pk[0] + shift[0], pk[1] + shift[1], pk[2] + shift[2]]
    np.testing.assert_allclose(s1, s0, rtol=1e-11)


def e4m3_weights(C, seed, tid, scale=1.0):
    """Dequantized e4m3 weights: a random (C, C) matrix of std scale/sqrt(C)
    through the per-tensor codec."""
    w = wl.normal_tensor((C, C), seed, tid) * (scale / np.sqrt(C))
    return blk.quant_dequant(w)[0]


def test_block_with_identity_projections_is_attention_of_quantized_x():
    """With all four projections the identity, the block is: quantize x,
    rotate it (as Q and as K), quantize Q, K and V, attend, quantize O."""
    shp = (1, 1, 1, 6, 2, 64)
    B, T, H, W, nh, d = shp
    C = nh * d
    x = rnd((B, T, H, W, C), 703, 0)
    I = np.eye(C)
    y = blk.block_fwd_fp8(x, I, I, I, I, nh, 1, ref.TOKEN)
    xd = blk.quant_dequant(x)[0].reshape(shp)
    q = blk.rope_3d(xd)
    qd, kd, vd = (blk.quant_dequant(t)[0] for t in (q, q, xd))
    o = ref.skiparse_attention(qd, kd, vd, 1, ref.TOKEN)
    want = blk.quant_dequant(o)[0].reshape(B, T, H, W, C)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_block_output_scales_with_wo_by_powers_of_two():
    shp = (1, 2, 4, 5, 2, 64)
    B, T, H, W, nh, d = shp
    C = nh * d
    x = rnd((B, T, H, W, C), 704, 0)
    wq, wk, wv, wo = (e4m3_weights(C, 704, i + 1) for i in range(4))
    y1 = blk.block_fwd_fp8(x, wq, wk, wv, wo, nh, 2, ref.GROUP)
    y2 = blk.block_fwd_fp8(x, wq, wk, wv, 4.0 * wo, nh, 2, ref.GROUP)
    np.testing.assert_allclose(y2, 4.0 * y1, rtol=1e-13)


def test_block_close_to_unquantized():
    """The fp8 block stays within a few percent of the same block computed
    without any quantization."""
    shp = (1, 2, 4, 6, 2, 64)
    B, T, H, W, nh, d = shp
    C = nh * d
    x = rnd((B, T, H, W, C), 705, 0)
    wq, wk, wv, wo = (e4m3_weights(C, 705, i + 1) for i in range(4))
    y = blk.block_fwd_fp8(x, wq, wk, wv, wo, nh, 2, ref.TOKEN)
    xm = x.reshape(-1, C)
    q, k, v = (xm @ w.T for w in (wq, wk, wv))
    q, k, v = (t.reshape(shp) for t in (q, k, v))
    o = ref.skiparse_attention(blk.rope_3d(q), blk.rope_3d(k), v, 2, ref.TOKEN)
    y0 = (o.reshape(-1, C) @ wo.T).reshape(B, T, H, W, C)
    assert np.max(np.abs(y - y0)) / np.max(np.abs(y0)) < 0.1
    # and the codes the oracle makes are those of its codec
    codes, scale, _ = f8.quantize_per_tensor(x.astype(np.float32).reshape(-1))
    np.testing.assert_array_equal(blk.quant_dequant(x)[1], codes)


def test_rope_matches_complex_rotation():
    """Each pair (x_2i, x_2i+1) of an axis part, read as the complex number
    x_2i + i x_2i+1, is multiplied by exp(i * pos * theta^(-2i/d_a))."""
    shp = (1, 3, 4, 5, 2, 64)
    x = rnd(shp, 706, 0)
    r = blk.rope_3d(x, theta=500.0)
    dims = blk.rope_dims(64)
    off = 0
    for axis, da in enumerate(dims):
        z = x[..., off:off + da:2] + 1j * x[..., off + 1:off + da:2]
        pos = np.arange(shp[1 + axis], dtype=np.float64)
        freq = np.exp(-np.log(500.0) * np.arange(0, da, 2) / da)
        view = [1, 1, 1, 1, 1, da // 2]
        view[1 + axis] = shp[1 + axis]
        zr = z * np.exp(1j * (pos[:, None] * freq[None, :])).reshape(view)
        np.testing.assert_allclose(r[..., off:off + da:2], zr.real, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r[..., off + 1:off + da:2], zr.imag, rtol=1e-12, atol=1e-12)
        off += da


def test_block_projections_follow_linear_layout():
    """Weights are (out, in), as a linear layer's: with every fp8 step
    removed (the codec bypassed) the block equals torch's linear layers around
    the attention oracle."""
    import torch
    shp = (1, 2, 3, 4, 2, 32)
    B, T, H, W, nh, d = shp
    C = nh * d
    x = rnd((B, T, H, W, C), 707, 0)
    ws = [rnd((C, C), 707, i + 1) / np.sqrt(C) for i in range(4)]
    ident = lambda t: (np.asarray(t, np.float64), None, None)
    orig = blk.quant_dequant
    blk.quant_dequant = ident
    try:
        y = blk.block_fwd_fp8(x, *ws, nh, 2, ref.GROUP)
    finally:
        blk.quant_dequant = orig
    xt = torch.from_numpy(x.reshape(-1, C))
    q, k, v = (torch.nn.functional.linear(xt, torch.from_numpy(w)).numpy().reshape(shp) for w in ws[:3])
    o = ref.skiparse_attention(blk.rope_3d(q), blk.rope_3d(k), v, 2, ref.GROUP)
    want = torch.nn.functional.linear(torch.from_numpy(o.reshape(-1, C)), torch.from_numpy(ws[3])).numpy()
    np.testing.assert_allclose(y, want.reshape(B, T, H, W, C), rtol=1e-10, atol=1e-12)
