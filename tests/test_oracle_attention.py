"""Pins for the oracle's attention (CPU only).

The literal pad -> rearrange -> masked attention -> rearrange back -> crop path
is checked against things fixed outside it: brute-force full attention under
the block mask built token by token, torch's scaled_dot_product_attention for
k = 1 (plain full attention, the hybrid model's full layers), closed forms
(uniform attention gives the subsequence mean; a constant V passes through;
dominant diagonal logits return each token's own V), frame-permutation
equivariance, and the two-layer chain written with explicit probability
matrices.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import skiparse_ref as ref


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


CASES = [
    # B, T, H, W, heads, d, k
    (1, 1, 4, 4, 1, 8, 2),
    (2, 2, 4, 8, 2, 16, 2),
    (1, 2, 3, 5, 2, 8, 2),      # padded on both axes
    (1, 1, 6, 10, 1, 8, 2),
    (1, 2, 9, 9, 1, 8, 3),      # exact for k=3
    (1, 1, 7, 11, 2, 8, 3),     # padded for k=3
    (1, 1, 5, 17, 1, 8, 4),
    (1, 2, 1, 1, 1, 8, 2),      # single token per frame
    (2, 1, 5, 6, 2, 8, 1),      # k = 1
]


@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("B,T,H,W,nh,d,k", CASES)
def test_literal_equals_block_masked_full_attention(B, T, H, W, nh, d, k, mode):
    shp = (B, T, H, W, nh, d)
    q, kk, v = rnd(shp, 1), rnd(shp, 2), rnd(shp, 3)
    lit = ref.skiparse_attention(q, kk, v, k, mode)
    bf = ref.masked_full_attention(q, kk, v, ref.block_mask(T, H, W, k, mode))
    np.testing.assert_allclose(lit, bf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,T,H,W,nh,d", [(1, 2, 4, 4, 2, 16), (2, 1, 5, 3, 3, 8)])
def test_k1_is_textbook_sdpa(B, T, H, W, nh, d):
    shp = (B, T, H, W, nh, d)
    q, kk, v = rnd(shp, 4), rnd(shp, 5), rnd(shp, 6)
    ours = ref.skiparse_attention(q, kk, v, 1, ref.GROUP)
    N = T * H * W
    tq = torch.from_numpy(q.reshape(B, N, nh, d)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(kk.reshape(B, N, nh, d)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v.reshape(B, N, nh, d)).permute(0, 2, 1, 3)
    sd = F.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).numpy().reshape(shp)
    np.testing.assert_allclose(ours, sd, rtol=1e-10, atol=1e-12)


def members_by_rule(T, H, W, k, mode):
    sub = {}
    for t in range(T):
        for h in range(H):
            for w in range(W):
                if k == 1:
                    s = 0
                elif mode == ref.TOKEN:
                    s = (h % k) * k + (w % k)
                else:
                    s = ((h // k) % k) * k + ((w // k) % k)
                sub.setdefault(s, []).append((t * H + h) * W + w)
    return sub


@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("B,T,H,W,nh,d,k", CASES)
def test_zero_queries_give_subsequence_mean(B, T, H, W, nh, d, k, mode):
    """q = 0 makes every logit 0, so each output is the plain mean of V over
    the real tokens of its subsequence (padding must not enter the mean)."""
    shp = (B, T, H, W, nh, d)
    v = rnd(shp, 7)
    out = ref.skiparse_attention(np.zeros(shp), rnd(shp, 8), v, k, mode)
    vf = v.reshape(B, -1, nh, d)
    of = out.reshape(B, -1, nh, d)
    for s, mem in members_by_rule(T, H, W, k, mode).items():
        mean = vf[:, mem].mean(axis=1, keepdims=True)
        np.testing.assert_allclose(of[:, mem], np.broadcast_to(mean, of[:, mem].shape), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
def test_constant_values_pass_through(mode):
    shp = (1, 2, 5, 7, 2, 8)
    c = rnd((1, 1, 1, 1, 2, 8), 9)
    v = np.broadcast_to(c, shp).copy()
    out = ref.skiparse_attention(rnd(shp, 10, 3.0), rnd(shp, 11, 3.0), v, 2, mode)
    np.testing.assert_allclose(out, v, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("T,H,W,k", [(1, 4, 8, 2), (2, 5, 7, 2), (1, 9, 9, 3)])
def test_dominant_self_logit_returns_own_value(T, H, W, k, mode):
    """With q = k = 40 * e_j, a distinct basis vector for each member of a
    subsequence, every query matches only its own key, so O = V token by
    token.  Any mix-up between query and key rows breaks this."""
    d = 64
    shp = (1, T, H, W, 1, d)
    q = np.zeros(shp)
    for s, mem in members_by_rule(T, H, W, k, mode).items():
        assert len(mem) <= d
        for j, tok in enumerate(mem):
            t, rem = divmod(tok, H * W)
            h, w = divmod(rem, W)
            q[0, t, h, w, 0, j] = 40.0
    v = rnd(shp, 12)
    out = ref.skiparse_attention(q, q, v, k, mode, scale=1.0)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
def test_frame_permutation_equivariance(mode):
    """Subsequences span every frame alike, so permuting frames of the input
    permutes frames of the output the same way."""
    shp = (1, 3, 6, 5, 2, 8)
    q, kk, v = rnd(shp, 13), rnd(shp, 14), rnd(shp, 15)
    perm = [2, 0, 1]
    a = ref.skiparse_attention(q, kk, v, 2, mode)[:, perm]
    b = ref.skiparse_attention(q[:, perm], kk[:, perm], v[:, perm], 2, mode)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_tiny_chain_token_then_group():
    """The 128-token, 2-head, d=64, k=2 workload: a token-wise layer followed
    by a group-wise layer with V2 = O1.  Layer by layer against brute force,
    and the pair against explicit probability matrices A_grp @ A_tok @ V,
    whose product is strictly positive (every token reaches every other token
    in two hops)."""
    shp = (1, 2, 8, 8, 2, 64)
    q, kk, v = rnd(shp, 16), rnd(shp, 17), rnd(shp, 18)
    o1 = ref.skiparse_attention(q, kk, v, 2, ref.TOKEN)
    o2 = ref.skiparse_attention(q, kk, o1, 2, ref.GROUP)
    np.testing.assert_allclose(o1, ref.masked_full_attention(q, kk, v, ref.block_mask(2, 8, 8, 2, ref.TOKEN)),
                               rtol=1e-12, atol=1e-12)
    N = 128
    for h in range(2):
        At = ref.probability_matrix(q, kk, 2, ref.TOKEN, 0, h)
        Ag = ref.probability_matrix(q, kk, 2, ref.GROUP, 0, h)
        np.testing.assert_allclose(At.sum(1), 1.0, rtol=1e-12)
        prod = Ag @ At
        assert np.all(prod > 0)
        expect = prod @ v.reshape(1, N, 2, 64)[0, :, h]
        np.testing.assert_allclose(o2.reshape(1, N, 2, 64)[0, :, h], expect, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("T,H,W,k", [(2, 5, 7, 2), (1, 9, 10, 3), (2, 6, 6, 1)])
def test_sampled_rows_match_full_output(T, H, W, k, mode):
    B, nh, d = 2, 2, 16
    shp = (B, T, H, W, nh, d)
    q, kk, v = rnd(shp, 19), rnd(shp, 20), rnd(shp, 21)
    full = ref.skiparse_attention(q, kk, v, k, mode).reshape(B, -1, nh, d)
    N = T * H * W
    rows = np.array([0, N - 1, N // 2, 3 % N, (7 * N) // 9])
    for b in range(B):
        for h in range(nh):
            got = ref.attention_rows(q.reshape(B, N, nh, d), kk.reshape(B, N, nh, d), v.reshape(B, N, nh, d),
                                     T, H, W, k, mode, b, h, rows)
            np.testing.assert_allclose(got, full[b, rows, h], rtol=1e-12, atol=1e-12)


def test_planted_mistakes_are_caught():
    """Plausible mistakes, planted in copies of the oracle on the CPU, fail the
    pins: letting padded keys in, using the wrong softmax scale, swapping the
    pattern."""
    shp = (1, 1, 3, 5, 1, 8)
    q, kk, v = rnd(shp, 22), rnd(shp, 23), rnd(shp, 24)
    bf = ref.masked_full_attention(q, kk, v, ref.block_mask(1, 3, 5, 2, ref.TOKEN))

    # padded keys (zeros) admitted: the padded tokens join the softmax
    Hp, Wp = ref.padded_extent(3, 2), ref.padded_extent(5, 2)
    qs = ref.rearrange_literal(ref.pad_tokens(q, 2), 2, ref.TOKEN)
    ks = ref.rearrange_literal(ref.pad_tokens(kk, 2), 2, ref.TOKEN)
    vs = ref.rearrange_literal(ref.pad_tokens(v, 2), 2, ref.TOKEN)
    out = np.zeros_like(qs)
    for s in range(4):
        out[0, s, 0] = ref.softmax_attention(qs[0, s, 0], ks[0, s, 0], vs[0, s, 0], 1 / np.sqrt(8))
    leaky = ref.inverse_rearrange_literal(out, 1, Hp, Wp, 2, ref.TOKEN)[:, :, :3, :5]
    assert not np.allclose(leaky, bf, atol=1e-6)

    wrong_scale = ref.skiparse_attention(q, kk, v, 2, ref.TOKEN, scale=1.0)
    assert not np.allclose(wrong_scale, bf, atol=1e-6)

    wrong_mode = ref.skiparse_attention(q, kk, v, 2, ref.GROUP)
    assert not np.allclose(wrong_mode, bf, atol=1e-6)
