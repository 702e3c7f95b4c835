"""Pins of the Skiparse-1D pattern in the oracle (the 1D skip rule on each
frame's flattened (h, w), stride K = k*k; see oracle.skiparse_ref.is_1d):
the rule applied token by token, the literal reshape/transpose against the
closed-form map, bijection and lengths, local equivalence over the repeating
unit of K^2 positions, the plan's fields, and attention / gradients against
brute force under the block mask."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import skiparse_bwd as bwd
from oracle import skiparse_ref as ref

MODES_1D = [ref.TOKEN_1D, ref.GROUP_1D]
SHAPES = [(1, 2, 3), (2, 3, 3), (1, 4, 5), (3, 5, 7), (2, 6, 10), (1, 1, 17), (2, 8, 8)]


def rule_member(l, K, mode):
    """The 1D rule on a flattened index, written out directly."""
    return l % K if mode == ref.TOKEN_1D else (l // K) % K


@pytest.mark.parametrize("mode", MODES_1D)
@pytest.mark.parametrize("T,H,W", SHAPES)
def test_members_follow_the_rule(T, H, W, mode):
    K = 4
    L = H * W
    want = [[] for _ in range(K)]
    for t in range(T):
        for l in range(L):
            want[rule_member(l, K, mode)].append(t * L + l)
    got = ref.subsequence_members(T, H, W, 2, mode)
    for s in range(K):
        np.testing.assert_array_equal(got[s], np.array(want[s], np.int64))


@pytest.mark.parametrize("mode", MODES_1D)
@pytest.mark.parametrize("T,H,W", SHAPES)
def test_literal_rearrange_matches_closed_form(T, H, W, mode):
    ids = np.arange(T * H * W, dtype=np.int64).reshape(1, T, H, W, 1, 1) + 1   # 0 marks padding
    lit = ref.to_subsequences(ids, 2, mode)[0, :, 0, :, 0] - 1
    np.testing.assert_array_equal(lit, ref.gather_map(T, H, W, 2, mode))
    back = ref.from_subsequences(ref.to_subsequences(ids, 2, mode), T, H, W, 2, mode)
    np.testing.assert_array_equal(back, ids)


@pytest.mark.parametrize("mode", MODES_1D)
@pytest.mark.parametrize("T,H,W", SHAPES)
def test_bijection_and_plan(T, H, W, mode):
    G = ref.gather_map(T, H, W, 2, mode)
    real = G[G >= 0]
    np.testing.assert_array_equal(np.sort(real), np.arange(T * H * W))
    p = ref.make_plan(1, T, H, W, 2, 64, 2, mode)
    assert p.n_sub == 4 and p.sub_h == 1 and p.Hp == 1
    assert p.Wp % 16 == 0 and p.Wp - 16 < H * W <= p.Wp
    assert sum(p.real_w) == H * W
    assert [len(m) for m in ref.subsequence_members(T, H, W, 2, mode)] == p.sub_len
    assert p.pairs == sum(n * n for n in p.sub_len) * 2
    if (H * W) % 16 == 0:   # unpadded: every subsequence holds 1/K of the tokens
        assert all(n == T * H * W // 4 for n in p.sub_len)


@pytest.mark.parametrize("mode", MODES_1D)
def test_local_equivalence(mode):
    """Rearranging the whole flattened sequence equals rearranging each unit of
    K^2 = 16 positions on its own and concatenating (the property the pages
    call local equivalence)."""
    units = 5
    whole = ref.gather_map(1, 1, 16 * units, 2, mode)
    unit = ref.gather_map(1, 1, 16, 2, mode)
    parts = np.concatenate([unit + 16 * u for u in range(units)], axis=1)
    np.testing.assert_array_equal(whole, parts)


@pytest.mark.parametrize("mode", MODES_1D)
@pytest.mark.parametrize("shp", [(1, 2, 3, 5, 2, 8), (2, 1, 5, 7, 1, 8), (1, 3, 4, 4, 2, 8)])
def test_attention_matches_block_masked_full(shp, mode):
    q, k, v = (wl.normal_tensor(shp, 501, i).astype(np.float64) for i in range(3))
    B, T, H, W, nh, d = shp
    got = ref.skiparse_attention(q, k, v, 2, mode)
    mask = ref.block_mask(T, H, W, 2, mode)
    want = ref.masked_full_attention(q, k, v, mask)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_k1_is_full_attention():
    shp = (1, 2, 3, 4, 2, 8)
    q, k, v = (wl.normal_tensor(shp, 502, i).astype(np.float64) for i in range(3))
    full = ref.skiparse_attention(q, k, v, 1, ref.TOKEN)
    for mode in MODES_1D:
        np.testing.assert_allclose(ref.skiparse_attention(q, k, v, 1, mode), full, rtol=0, atol=0)


@pytest.mark.parametrize("mode", MODES_1D)
def test_gradients_match_torch_autograd(mode):
    shp = (2, 2, 5, 6, 2, 8)
    q, k, v, do = (wl.normal_tensor(shp, 503, i).astype(np.float64) for i in range(4))
    B, T, H, W, nh, d = shp
    N = T * H * W
    got = bwd.skiparse_attention_bwd(q, k, v, do, 2, mode)
    tq, tk, tv = (torch.tensor(x.reshape(B, N, nh, d).transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(ref.block_mask(T, H, W, 2, mode)))
    o.backward(torch.tensor(do.reshape(B, N, nh, d).transpose(0, 2, 1, 3)))
    for g, t in zip(got, (tq, tk, tv)):
        np.testing.assert_allclose(g.reshape(B, N, nh, d), t.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)
