"""One attention block of the video DiT on fp8, written out plainly in float64
(test infrastructure only).

The layers that carry Skiparse attention sit in a DiT whose 8-bit path
quantizes per tensor (OSP-Next summary, 核心方法 core method: the hybrid model
with full attention in its first and last blocks; 方法步骤详情 method steps:
per-tensor scaling, scale = max / (Amax + eps)).  The pages name the
pieces around the attention (QKV projection, rotary position embedding,
output projection) but define none of them, so the block here takes the
plainest form:

    x^  = q8(x)                                      per-tensor e4m3
    Q   = x^ Wq^,  K = x^ Wk^,  V = x^ Wv^          (W^ : e4m3 weights, per tensor)
    Q, K = rope(Q), rope(K)                          3-axis rotary embedding
    O   = SkiparseAttention(q8(Q), q8(K), q8(V))     (oracle.skiparse_ref)
    y   = q8(O) Wo^

Rotary embedding (reading): the head dimension d is cut into three parts
(d_t, d_h, d_w), by default d_t = d - 4*(d // 6) and d_h = d_w = 2*(d // 6)
(44/42/42 at d = 128, the split of the video DiT family the pages compare
against); inside the part of axis a the consecutive pairs (x_2i, x_2i+1),
i < d_a / 2, are rotated by the angle pos_a * theta^(-2i / d_a), pos_a being
the token's t, h or w and theta = 10000.

Every quantization step is the oracle's own e4m3 codec (oracle.fp8_ref)
applied to the float32 cast of the float64 value, so the fp8 decisions are
made from the same rule as on the device; products and sums are float64.
"""

from __future__ import annotations

import numpy as np

from . import fp8_ref as f8
from .skiparse_ref import skiparse_attention


def rope_dims(d: int):
    """(d_t, d_h, d_w) of the 3-axis rotary embedding."""
    dh = 2 * (d // 6)
    return d - 2 * dh, dh, dh


def rope_angles(n_pos: int, d_axis: int, theta: float = 10000.0) -> np.ndarray:
    """(n_pos, d_axis // 2) rotation angles pos * theta^(-2i / d_axis)."""
    i = np.arange(d_axis // 2, dtype=np.float64)
    return np.arange(n_pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / d_axis)[None, :]


def rope_3d(x, theta: float = 10000.0, dims=None) -> np.ndarray:
    """Rotate (B, T, H, W, heads, d) by the token's (t, h, w) position."""
    x = np.asarray(x, np.float64)
    B, T, H, W, nh, d = x.shape
    dt, dh, dw = rope_dims(d) if dims is None else dims
    assert dt + dh + dw == d and dt % 2 == 0 and dh % 2 == 0 and dw % 2 == 0
    out = x.copy()
    off = 0
    for axis, (n_pos, da) in enumerate(((T, dt), (H, dh), (W, dw))):
        ang = rope_angles(n_pos, da, theta)                     # (n_pos, da/2)
        shape = [1, 1, 1, 1, 1, da // 2]
        shape[1 + axis] = n_pos
        c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
        a = x[..., off:off + da:2]
        b = x[..., off + 1:off + da:2]
        out[..., off:off + da:2] = a * c - b * s
        out[..., off + 1:off + da:2] = a * s + b * c
        off += da
    return out


def quant_dequant(x):
    """Per-tensor e4m3 round trip of float values (scale rule of oracle.fp8_ref)."""
    flat = np.asarray(x, np.float64).astype(np.float32).reshape(-1)
    codes, scale, _ = f8.quantize_per_tensor(flat)
    return f8.dequantize(codes, scale).reshape(np.shape(x)), codes, scale


def block_fwd_fp8(x, wq, wk, wv, wo, heads: int, kf: int, mode: int, theta: float = 10000.0, dims=None):
    """y (B, T, H, W, C) of the fp8 attention block with ``heads`` heads.
    x: (B, T, H, W, C) floats; wq/wk/wv/wo: (C, C) dequantized e4m3 weights in
    (out, in) layout."""
    x = np.asarray(x, np.float64)
    B, T, H, W, C = x.shape
    d = C // heads
    xd, _, _ = quant_dequant(x)
    xm = xd.reshape(-1, C)
    q, k, v = (xm @ np.asarray(w, np.float64).T for w in (wq, wk, wv))
    q, k, v = (t.reshape(B, T, H, W, heads, d) for t in (q, k, v))
    q, k = rope_3d(q, theta, dims), rope_3d(k, theta, dims)
    qd, kd, vd = (quant_dequant(t)[0] for t in (q, k, v))
    o = skiparse_attention(qd, kd, vd, kf, mode)
    od, _, _ = quant_dequant(o)
    return (od.reshape(-1, C) @ np.asarray(wo, np.float64).T).reshape(B, T, H, W, C)
