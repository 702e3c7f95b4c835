"""GPU parity of the fp8 attention block (projections, rotary embedding,
Skiparse attention) through the C ABI against oracle/block_ref.py.

* The rotary embedding + quantization step alone (skiparse_rope_fp8): scale
  and e4m3 codes against the oracle's rotation in float64 quantized in fp32.
  Both sides decide each code from an fp32 product; the device's rotation is
  fp32 arithmetic, so a code may differ where the oracle's product lies within
  fp32 rounding of a rounding midpoint: at most a few such codes, each one step
  away.
* The block: y element by element against the oracle's fp8 block on small
  shapes; the weights' codes bit-exact first.  Bars, relative to the output's
  own scale since y's scale follows the weights: rms(y - y_ref) <= 0.06 rms(y_ref)
  and max|y - y_ref| <= 0.1 max|y_ref|.  e4m3 keeps 3 mantissa bits, so one
  rounding moves a value by at most 2^-4 of it, rms 2^-4/sqrt(3) = 0.036 for
  evenly spread residuals; the two sides round O (and, from float64 against
  bf16 projections, a share of Q, K, V) each on its own, so y's residuals
  differ by up to sqrt(2) * 0.036 = 0.051 rms from O alone, plus the attention
  kernel's e4m3 P.  And the device block is as accurate as the oracle's:
  against the exact float64 block without quantization, its rms error is at
  most 1.2 times the oracle's.
* The 720P-5s shape, all 40 heads (C = 5120): the oracle's fp8 block cannot be evaluated
  row by row (O's per-tensor scale needs every row), so sampled rows are
  checked against the exact float64 block without quantization, bars rms 0.1
  and max 0.15 (1.5 to 2 times the quantization error the oracle itself shows
  against the exact block on small shapes, rms 0.06-0.07, max 0.07-0.11); and
  y doubles bit-exactly when Wo's scale halves.
"""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import block_ref as blk
from oracle import fp8_ref as f8
from oracle import skiparse_ref as ref

pytestmark = pytest.mark.gpu

DEV = "cuda"
BLOCK_RMS = 0.06
BLOCK_MAX = 0.1


def bf16_input(shape, seed, tid, scale=1.0):
    x = torch.from_numpy(wl.normal_tensor(shape, seed, tid) * np.float32(scale)).to(torch.bfloat16)
    return x, x.float().numpy().astype(np.float64)


def code_steps(a, b):
    """Distance in representable steps between e4m3 codes of equal sign
    (codes are sign-magnitude and monotone in magnitude)."""
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    same_sign = (a & 0x80) == (b & 0x80)
    dist = np.where(same_sign, np.abs((a & 0x7F) - (b & 0x7F)), (a & 0x7F) + (b & 0x7F))
    return dist


# ---------------------------------------------------------------------------
# rotary embedding + quantization
# ---------------------------------------------------------------------------

ROPE_CASES = [
    ((1, 3, 5, 7, 2, 128), 10000.0, None),
    ((2, 2, 9, 17, 3, 128), 10000.0, None),
    ((1, 4, 6, 6, 1, 64), 500.0, (20, 22, 22)),
    ((1, 2, 3, 4, 2, 128), 10000.0, (128, 0, 0)),
    ((1, 1, 1, 1, 1, 128), 10000.0, None),
    ((1, 21, 45, 80, 2, 128), 10000.0, None),
    ((1, 2, 16, 200, 1, 128), 10000.0, None),    # table of 4580 entries: read from global memory, not LDS
]


@pytest.mark.parametrize("shp,theta,dims", ROPE_CASES)
def test_rope_fp8_codes(shp, theta, dims):
    B, T, H, W, nh, d = shp
    x, x64 = bf16_input(shp, 801, 0, 3.0)
    plan = sk.skiparse_plan_init(B, T, H, W, nh, d, 1, 0)
    y = torch.empty(shp, dtype=torch.uint8, device=DEV)
    sc = torch.empty(2, dtype=torch.float32, device=DEV)
    sk.skiparse_rope_fp8(plan, x.to(DEV), y, sc, theta, dims)
    torch.cuda.synchronize()
    r = blk.rope_3d(x64, theta, dims)
    codes, scale, _ = f8.quantize_per_tensor(r.astype(np.float32).reshape(-1))
    got_scale = sc.cpu().numpy()
    np.testing.assert_allclose(got_scale[0], scale, rtol=2.0 ** -22)
    got = y.cpu().numpy().reshape(-1)
    bad = np.nonzero(got != codes)[0]
    assert bad.size <= max(4, got.size // 100000), f"{bad.size} codes differ"
    if bad.size:
        assert np.all(code_steps(got[bad], codes[bad]) == 1)


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------

def weights(C, seed):
    """Four (C, C) fp32 weights of std 1/sqrt(C), their device codes/scales and
    the oracle's dequantized copies (codes checked equal)."""
    ws = [wl.normal_tensor((C, C), seed, 10 + i) * np.float32(1.0 / np.sqrt(C)) for i in range(4)]
    codes, scales = sk.quantize_weights(*(torch.from_numpy(w).to(DEV) for w in ws))
    torch.cuda.synchronize()
    deq = []
    for i, w in enumerate(ws):
        c_ref, s_ref, _ = f8.quantize_per_tensor(w.reshape(-1))
        np.testing.assert_array_equal(codes[i].cpu().numpy().reshape(-1), c_ref)
        np.testing.assert_allclose(scales[i, 0].item(), s_ref, rtol=0)
        deq.append(f8.dequantize(c_ref, s_ref).reshape(C, C))
    return codes, scales, deq, ws


def rms_err(y, y_ref):
    return float(np.sqrt(np.mean((y - y_ref) ** 2) / np.mean(y_ref ** 2)))


def max_err(y, y_ref):
    return float(np.max(np.abs(y - y_ref))) / float(np.max(np.abs(y_ref)))


def check_block(y, y_ref, label=""):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    r, m = rms_err(y, y_ref), max_err(y, y_ref)
    print(f"  block {label}: rms {r:.4f} max {m:.4f}")
    assert r <= BLOCK_RMS and m <= BLOCK_MAX


def exact_block(x64, ws, heads, kf, mode, theta=10000.0, dims=None):
    """The block in float64 with every quantization left out."""
    B, T, H, W, C = x64.shape
    xm = x64.reshape(-1, C)
    q, k, v = ((xm @ w.T).reshape(B, T, H, W, heads, C // heads) for w in ws[:3])
    o = ref.skiparse_attention(blk.rope_3d(q, theta, dims), blk.rope_3d(k, theta, dims), v, kf, mode)
    return (o.reshape(-1, C) @ ws[3].T).reshape(x64.shape)


BLOCK_CASES = [
    ((1, 3, 13, 22), 2, 2, ref.TOKEN),
    ((1, 3, 13, 22), 2, 2, ref.GROUP),
    ((2, 2, 9, 17), 3, 2, ref.GROUP),
    ((1, 2, 10, 10), 2, 1, ref.TOKEN),
    ((1, 2, 9, 17), 24, 2, ref.TOKEN),
    ((1, 1, 1, 1), 2, 2, ref.TOKEN),
    ((1, 2, 3, 5), 1, 2, ref.GROUP),
    ((1, 3, 6, 7), 2, 2, ref.TOKEN_1D),
    ((1, 3, 6, 7), 2, 2, ref.GROUP_1D),
]


@pytest.mark.parametrize("grid,heads,kf,mode", BLOCK_CASES)
def test_block_small(grid, heads, kf, mode):
    C = heads * 128
    codes, scales, deq, _ = weights(C, 802 + heads)
    x, x64 = bf16_input(grid + (C,), 803, 0)
    blockf = sk.BlockFP8(codes, scales, heads, kf, mode)
    y = blockf(x.to(DEV))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    want = blk.block_fwd_fp8(x64, *deq, heads, kf, mode)
    check_block(y, want, f"{grid} heads={heads} k={kf} mode={mode}")
    exact = exact_block(x64, deq, heads, kf, mode)
    assert rms_err(y, exact) <= 1.2 * rms_err(want, exact)


def test_block_rope_arguments_reach_the_kernels():
    """A custom split and theta change the result, and match the oracle with
    the same arguments."""
    grid, heads = (1, 3, 8, 9), 2
    C = heads * 128
    codes, scales, deq, _ = weights(C, 804)
    x, x64 = bf16_input(grid + (C,), 805, 0)
    blockf = sk.BlockFP8(codes, scales, heads, 2, ref.TOKEN, rope_theta=100.0, rope_dims=(32, 48, 48))
    y = blockf(x.to(DEV)).float().cpu().numpy()
    want = blk.block_fwd_fp8(x64, *deq, heads, 2, ref.TOKEN, theta=100.0, dims=(32, 48, 48))
    default = blk.block_fwd_fp8(x64, *deq, heads, 2, ref.TOKEN)
    check_block(y, want, "theta 100, split 32/48/48")
    assert rms_err(default, want) > 4 * rms_err(y, want)


def test_block_two_shapes_in_a_row():
    """One context and workspace serve a large call and then a smaller one."""
    heads = 2
    C = heads * 128
    codes, scales, deq, _ = weights(C, 806)
    blockf = sk.BlockFP8(codes, scales, heads, 2, ref.GROUP)
    for grid in ((1, 3, 13, 22), (1, 2, 5, 6)):
        x, x64 = bf16_input(grid + (C,), 807, 0)
        y = blockf(x.to(DEV))
        torch.cuda.synchronize()
        check_block(y.float().cpu().numpy(), blk.block_fwd_fp8(x64, *deq, heads, 2, ref.GROUP), str(grid))


def exact_block_rows(x64, ws, heads, kf, mode, tokens, theta=10000.0):
    """Rows y[0, token] of the exact float64 block (no quantization) for flat
    token indices; each row needs its subsequence's keys and values only."""
    B, T, H, W, C = x64.shape
    d = C // heads
    members, sub_of = ref._members_for((T, H, W, kf, ref.TOKEN if kf == 1 else mode))
    xf = x64.reshape(T * H * W, C)
    t_of = np.arange(T * H * W) // (H * W)
    h_of = (np.arange(T * H * W) // W) % H
    w_of = np.arange(T * H * W) % W
    dt, dh, dw = blk.rope_dims(d)

    def rope_rows(m, idx):      # m: (n, heads, d) at flat tokens idx
        out = m.copy()
        off = 0
        for pos, da in ((t_of[idx], dt), (h_of[idx], dh), (w_of[idx], dw)):
            ang = pos[:, None] * theta ** (-2.0 * np.arange(da // 2) / da)[None, :]
            c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
            a, b = m[..., off:off + da:2], m[..., off + 1:off + da:2]
            out[..., off:off + da:2] = a * c - b * s
            out[..., off + 1:off + da:2] = a * s + b * c
            off += da
        return out

    rows = np.zeros((len(tokens), C))
    for s in np.unique(sub_of[tokens]):
        sel = np.nonzero(sub_of[tokens] == s)[0]
        mem = members[s]
        kk = rope_rows((xf[mem] @ ws[1].T).reshape(-1, heads, d), mem)
        vv = (xf[mem] @ ws[2].T).reshape(-1, heads, d)
        tq = np.asarray(tokens)[sel]
        qq = rope_rows((xf[tq] @ ws[0].T).reshape(-1, heads, d), tq)
        o = np.zeros((len(sel), heads, d))
        for h in range(heads):
            sc = qq[:, h] @ kk[:, h].T / np.sqrt(d)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            o[:, h] = (p / p.sum(axis=1, keepdims=True)) @ vv[:, h]
        rows[sel] = o.reshape(len(sel), C) @ ws[3].T
    return rows


def test_block_480p_sampled():
    """The 480p workload shape (21 x 32 x 52 tokens, 12 heads of 128, C = 1536,
    k = 2 group-wise): sampled rows against the exact block, bars as at
    720P-5s, and exact doubling with Wo's scale halved."""
    w = wl.WORKLOADS["480p"]
    B, T, H, W, heads, d = w.shape
    C = heads * d
    codes, scales, deq, _ = weights(C, 811)
    x, x64 = bf16_input((1, T, H, W, C), 812, 0)
    xd = x.to(DEV)
    blockf = sk.BlockFP8(codes, scales, heads, 2, ref.GROUP)
    y1 = blockf(xd)
    torch.cuda.synchronize()
    yh = y1.float().cpu().numpy().reshape(T * H * W, C)
    assert np.all(np.isfinite(yh))
    rng = np.random.Generator(np.random.PCG64(813))
    members, _ = ref._members_for((T, H, W, 2, ref.GROUP))
    tokens = np.sort(np.concatenate([rng.choice(members[s], size=12, replace=False) for s in (0, 3)]))
    want = exact_block_rows(x64, deq, heads, 2, ref.GROUP, tokens)
    r, m = rms_err(yh[tokens], want), max_err(yh[tokens], want)
    print(f"480p block sampled rows vs exact: rms {r:.4f} max {m:.4f}")
    assert r <= 0.1 and m <= 0.15
    scales2 = scales.clone()
    scales2[3, 1] *= 2.0
    blockf.w_scales = scales2
    y2 = blockf(xd)
    torch.cuda.synchronize()
    assert torch.equal(y2.float(), 2.0 * y1.float())


def test_block_720p_tokens_12_heads_sampled():
    """The 720P-5s token grid (21 x 45 x 80 tokens, H padded to 48) with 12
    heads of 128 (C = 1536), k = 2 token-wise: sampled rows of two
    subsequences against the exact block, the 480p bars, and exact doubling
    with Wo's scale halved."""
    T, H, W, heads, d = 21, 45, 80, 12, 128
    C = heads * d
    codes, scales, deq, _ = weights(C, 821)
    x, x64 = bf16_input((1, T, H, W, C), 822, 0)
    xd = x.to(DEV)
    blockf = sk.BlockFP8(codes, scales, heads, 2, ref.TOKEN)
    y1 = blockf(xd)
    torch.cuda.synchronize()
    yh = y1.float().cpu().numpy().reshape(T * H * W, C)
    assert np.all(np.isfinite(yh))
    rng = np.random.Generator(np.random.PCG64(823))
    members, _ = ref._members_for((T, H, W, 2, ref.TOKEN))
    tokens = np.sort(np.concatenate([[members[3][-1]], rng.choice(members[0], size=12, replace=False),
                                     rng.choice(members[3], size=11, replace=False)]))
    tokens = np.unique(tokens)
    want = exact_block_rows(x64, deq, heads, 2, ref.TOKEN, tokens)
    r, m = rms_err(yh[tokens], want), max_err(yh[tokens], want)
    print(f"720p-token block (12 heads) sampled rows vs exact: rms {r:.4f} max {m:.4f}")
    assert r <= 0.1 and m <= 0.15
    scales2 = scales.clone()
    scales2[3, 1] *= 2.0
    blockf.w_scales = scales2
    y2 = blockf(xd)
    torch.cuda.synchronize()
    assert torch.equal(y2.float(), 2.0 * y1.float())


def test_block_workload_sampled():
    """720P-5s (21 x 45 x 80 tokens, 40 heads of 128, k = 2 token-wise): rows
    against the exact block, and exact doubling with Wo's scale halved."""
    w = wl.WORKLOADS["720p_5s"]
    B, T, H, W, heads, d = w.shape
    C = heads * d
    codes, scales, deq, _ = weights(C, 808)
    x, x64 = bf16_input((1, T, H, W, C), 809, 0)
    xd = x.to(DEV)
    blockf = sk.BlockFP8(codes, scales, heads, 2, ref.TOKEN)
    y1 = blockf(xd)
    torch.cuda.synchronize()
    yh = y1.float().cpu().numpy().reshape(T * H * W, C)
    assert np.all(np.isfinite(yh))
    rng = np.random.Generator(np.random.PCG64(810))
    members, _ = ref._members_for((T, H, W, 2, ref.TOKEN))
    # rows of subsequences 0 and 3 (both coordinates of the pattern move)
    tokens = np.sort(np.concatenate([rng.choice(members[s], size=12, replace=False) for s in (0, 3)]))
    want = exact_block_rows(x64, deq, heads, 2, ref.TOKEN, tokens)
    r, m = rms_err(yh[tokens], want), max_err(yh[tokens], want)
    print(f"720p block sampled rows vs exact: rms {r:.4f} max {m:.4f}")
    assert r <= 0.1 and m <= 0.15
    # Wo scale halved -> weights doubled -> y doubled exactly (power of two)
    scales2 = scales.clone()
    scales2[3, 1] *= 2.0
    blockf.w_scales = scales2
    y2 = blockf(xd)
    torch.cuda.synchronize()
    assert torch.equal(y2.float(), 2.0 * y1.float())
