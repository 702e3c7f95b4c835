"""Pins for the oracle's index maps (CPU only).

What fixes the maps independently of the oracle's own closed form:
* hand-derived maps in tests/golden (from the membership rules on the OSP-Next
  summary page, 核心方法 core method and 方法步骤详情 method steps);
* torch's pixel_unshuffle, the library routine the token-wise pattern is named
  after, and the same routine applied to the k x k block grid for the
  group-wise pattern (patch unshuffle);
* brute-force enumeration token by token;
* the invariants the pages state: k^2 subsequences of N/k^2 tokens each, local
  equivalence of the rearrange, the same position following the same pattern
  at any resolution, and any two tokens meeting within one token-wise plus one
  group-wise hop.
"""

import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import skiparse_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            s, vals = line.split(":")
            rows[int(s)] = [int(v) for v in vals.split()]
    return np.array([rows[s] for s in sorted(rows)], dtype=np.int64)


@pytest.mark.parametrize("fname,T,H,W,k,mode", [
    ("map_token_T1_H4_W4_k2.txt", 1, 4, 4, 2, ref.TOKEN),
    ("map_group_T1_H4_W4_k2.txt", 1, 4, 4, 2, ref.GROUP),
    ("map_token_T1_H3_W5_k2.txt", 1, 3, 5, 2, ref.TOKEN),
    ("map_group_T1_H3_W5_k2.txt", 1, 3, 5, 2, ref.GROUP),
    ("map_group_T1_H8_W8_k2.txt", 1, 8, 8, 2, ref.GROUP),
    ("map_token_T2_H2_W2_k2.txt", 2, 2, 2, 2, ref.TOKEN),
    ("map_token1d_T1_H2_W3_k2.txt", 1, 2, 3, 2, ref.TOKEN_1D),
    ("map_group1d_T2_H3_W3_k2.txt", 2, 3, 3, 2, ref.GROUP_1D),
    ("map_token1d_T1_H4_W5_k2.txt", 1, 4, 5, 2, ref.TOKEN_1D),
    ("map_group1d_T1_H4_W5_k2.txt", 1, 4, 5, 2, ref.GROUP_1D),
])
def test_golden_maps(fname, T, H, W, k, mode):
    np.testing.assert_array_equal(ref.gather_map(T, H, W, k, mode), load_golden(fname))


def iota_map_via_literal(T, H, W, k, mode):
    """Token ids pushed through the reshape/transpose rearrange of the oracle."""
    Hp, Wp = ref.padded_extent(H, k), ref.padded_extent(W, k)
    ids = np.full((1, T, Hp, Wp, 1, 1), -1, np.int64)
    ids[0, :, :H, :W, 0, 0] = np.arange(T * H * W).reshape(T, H, W)
    return ref.rearrange_literal(ids, k, mode)[0, :, 0, :, 0]


SHAPES = [(1, 4, 4), (2, 8, 8), (1, 3, 5), (2, 6, 10), (3, 9, 7), (1, 16, 16), (2, 5, 17), (1, 1, 1),
          (2, 12, 20), (1, 45 % 13, 80 % 23)]


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("T,H,W", SHAPES)
def test_closed_form_equals_literal_rearrange(T, H, W, k, mode):
    np.testing.assert_array_equal(ref.gather_map(T, H, W, k, mode), iota_map_via_literal(T, H, W, k, mode))


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("T,H,W", [(1, 4, 4), (2, 8, 12), (3, 6, 9), (1, 16, 32)])
def test_token_wise_is_pixel_unshuffle(T, H, W, k):
    """Unpadded token-wise map == torch pixel_unshuffle of token ids (channel
    c*k^2 + p*k + q holds sub-map (p, q))."""
    Hp, Wp = ref.padded_extent(H, k), ref.padded_extent(W, k)
    ids = torch.full((T, 1, Hp, Wp), -1, dtype=torch.int64)
    ids[:, 0, :H, :W] = torch.arange(T * H * W).reshape(T, H, W)
    pu = F.pixel_unshuffle(ids, k)                     # (T, k*k, Hp/k, Wp/k)
    expect = pu.permute(1, 0, 2, 3).reshape(k * k, -1).numpy()
    np.testing.assert_array_equal(ref.gather_map(T, H, W, k, ref.TOKEN), expect)


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("T,H,W", [(1, 4, 4), (2, 8, 12), (1, 18, 9), (2, 5, 7)])
def test_group_wise_is_patch_unshuffle(T, H, W, k):
    """Group-wise map == pixel_unshuffle applied to the grid of k x k blocks:
    each block is a 'super-pixel' carrying its k*k tokens."""
    Hp, Wp = ref.padded_extent(H, k), ref.padded_extent(W, k)
    ids = torch.full((T, Hp, Wp), -1, dtype=torch.int64)
    ids[:, :H, :W] = torch.arange(T * H * W).reshape(T, H, W)
    # (T, Hb, k, Wb, k) -> (T, k*k [kh kw], Hb, Wb): blocks as channels
    blocks = ids.reshape(T, Hp // k, k, Wp // k, k).permute(0, 2, 4, 1, 3).reshape(T, k * k, Hp // k, Wp // k)
    pu = F.pixel_unshuffle(blocks, k)                  # (T, k*k*k*k, Hb/k, Wb/k); channel (kh kw p q)
    pu = pu.reshape(T, k, k, k, k, Hp // (k * k), Wp // (k * k))   # T kh kw p q hb wb
    # canonical order inside subsequence (p, q): t, hb, kh, wb, kw
    expect = pu.permute(3, 4, 0, 5, 1, 6, 2).reshape(k * k, -1).numpy()
    np.testing.assert_array_equal(ref.gather_map(T, H, W, k, ref.GROUP), expect)


def brute_force_map(T, H, W, k, mode):
    """Enumerate tokens one by one, file each under its subsequence by the
    membership rule, order by (t, h, w)."""
    members = {s: [] for s in range(k * k)}
    for t in range(T):
        for h in range(H):
            for w in range(W):
                if k == 1:
                    p = q = 0
                elif mode == ref.TOKEN:
                    p, q = h % k, w % k
                else:
                    p, q = (h // k) % k, (w // k) % k
                members[p * k + q].append((t * H + h) * W + w)
    return members


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("T,H,W", SHAPES)
def test_members_match_brute_force(T, H, W, k, mode):
    got = ref.subsequence_members(T, H, W, k, mode)
    bf = brute_force_map(T, H, W, k, mode)
    for s in range(k * k):
        np.testing.assert_array_equal(got[s], np.array(bf[s], np.int64))


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("T,H,W", SHAPES + [(21, 45, 80), (21, 48, 80), (21, 32, 52)])
def test_bijection_and_lengths(T, H, W, k, mode):
    G = ref.gather_map(T, H, W, k, mode)
    N = T * H * W
    real = G[G >= 0]
    assert real.size == N
    np.testing.assert_array_equal(np.sort(real), np.arange(N))
    Hp, Wp = ref.padded_extent(H, k), ref.padded_extent(W, k)
    assert (G < 0).sum() == T * Hp * Wp - N
    assert G.shape == (k * k, T * Hp * Wp // (k * k))
    if H % (k * k) == 0 and W % (k * k) == 0:
        # k^2 subsequences, each 1/k^2 of the tokens (方法步骤详情 method steps)
        assert all((row >= 0).sum() == N // (k * k) for row in G)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
@pytest.mark.parametrize("T,H,W", SHAPES + [(21, 45, 80)])
def test_real_members_form_prefix_box(T, H, W, k, mode):
    """Real slots of each subsequence are the box [0,T) x [0,Hr) x [0,Wr) of
    its local grid, with Hr, Wr the plan's real extents."""
    plan = ref.make_plan(1, T, H, W, 1, 64, k, mode)
    G = ref.gather_map(T, H, W, k, mode).reshape(k * k, T, plan.sub_h, plan.sub_w)
    for p in range(k):
        for q in range(k):
            ok = G[p * k + q] >= 0
            expect = np.zeros_like(ok)
            expect[:, :plan.real_h[p], :plan.real_w[q]] = True
            np.testing.assert_array_equal(ok, expect)
            assert plan.sub_len[p * k + q] == ok.sum()


def test_real_extent_closed_forms():
    """Hr(p) = floor(H/k) + [p < H mod k] (token-wise) and
    Hr(p) = floor(H/k^2)*k + clamp(H mod k^2 - p*k, 0, k) (group-wise)."""
    for k in range(1, 9):
        for H in range(0, 100):
            for p in range(k):
                tok = H // k + (1 if p < H % k else 0)
                grp = (H // (k * k)) * k + min(max(H % (k * k) - p * k, 0), k)
                if k == 1:
                    tok = grp = H
                assert ref.real_extent(H, k, ref.TOKEN, p) == tok
                assert ref.real_extent(H, k, ref.GROUP, p) == grp


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
def test_local_equivalence(k, mode):
    """Rearranging the whole sequence == rearranging each minimal repeating
    unit (k^2 rows) on its own and concatenating (OSP-Next summary, 核心方法
    core method; OSP-Next abstract)."""
    T, W = 2, 2 * k * k
    units = 3
    H = units * k * k
    G = ref.gather_map(T, H, W, k, mode)
    sh = H // k
    Gv = G.reshape(k * k, T, sh, W // k)
    for u in range(units):
        Gc = ref.gather_map(T, k * k, W, k, mode).reshape(k * k, T, k, W // k)
        # chunk-local token ids -> global ids: row h_local + u*k^2
        t, hc, w = Gc // (k * k * W), (Gc // W) % (k * k), Gc % W
        glob = (t * H + hc + u * k * k) * W + w
        np.testing.assert_array_equal(Gv[:, :, u * k:(u + 1) * k, :], glob)


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
def test_same_position_same_pattern_any_resolution(k, mode):
    """A token at (h, w) joins the same subsequence whatever H and W are
    (any-resolution rule, 方法步骤详情 method steps)."""
    def sub_at(H, W):
        G = ref.gather_map(1, H, W, k, mode)
        s = np.full(H * W, -1)
        for si, row in enumerate(G):
            s[row[row >= 0]] = si
        return s.reshape(H, W)
    big = sub_at(4 * k * k + 1, 4 * k * k + 3)
    for H, W in [(k * k, k * k), (5, 7), (k * k + 1, 3 * k * k - 1), (2, 2)]:
        np.testing.assert_array_equal(sub_at(H, W), big[:H, :W])


def connectivity_ok(T, H, W, k, first, second):
    M1 = ref.block_mask(T, H, W, k, first).astype(np.int64)
    M2 = ref.block_mask(T, H, W, k, second).astype(np.int64)
    return bool(np.all((M2 @ M1) > 0))


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("T,H,W", [(1, 6, 10), (2, 9, 9), (1, 4, 4), (1, 9, 12)])
def test_two_hop_connectivity(T, H, W, k):
    """Any two tokens interact within one token-wise plus one group-wise
    attention, in either order (OSP-Next summary, 核心方法 core method).
    Holds whenever H, W >= k^2."""
    if H < k * k or W < k * k:
        pytest.skip("needs H, W >= k^2")
    assert connectivity_ok(T, H, W, k, ref.TOKEN, ref.GROUP)
    assert connectivity_ok(T, H, W, k, ref.GROUP, ref.TOKEN)


def test_two_hop_connectivity_exact_condition():
    """Brute force over small grids (k <= 3, H, W <= 11): two hops connect
    every pair exactly when each axis extent n satisfies n >= k^2, n < k or
    n mod k == 0 -- so always once H, W >= k^2."""
    def axis_ok(n, k):
        return n >= k * k or n < k or n % k == 0
    for k in (2, 3):
        for H in range(1, 12):
            for W in range(1, 12):
                expect = axis_ok(H, k) and axis_ok(W, k)
                assert connectivity_ok(1, H, W, k, ref.TOKEN, ref.GROUP) == expect, (k, H, W)
                assert connectivity_ok(1, H, W, k, ref.GROUP, ref.TOKEN) == expect, (k, H, W)


def test_k1_is_identity():
    for T, H, W in [(1, 3, 5), (2, 4, 4)]:
        G = ref.gather_map(T, H, W, 1, ref.GROUP)
        np.testing.assert_array_equal(G, np.arange(T * H * W)[None])


def test_plan_pair_counts_at_workload_shapes():
    """Sub-lengths and pair counts at the 720P, 768P, 480P shapes, counted from
    the map, agree with the plan's closed-form extents."""
    cases = [
        ((1, 21, 45, 80, 40, 128, 2, ref.TOKEN), [19320, 19320, 18480, 18480]),
        ((1, 21, 45, 80, 40, 128, 2, ref.GROUP), [19320, 19320, 18480, 18480]),
        ((2, 21, 48, 80, 40, 128, 2, ref.TOKEN), [20160] * 4),
        ((1, 21, 32, 52, 12, 128, 2, ref.GROUP), [8736] * 4),
    ]
    for args, lens in cases:
        plan = ref.make_plan(*args)
        assert plan.sub_len == lens
        B, T, H, W, nh, d, k, mode = args
        assert plan.pairs == ref.pair_count(B, T, H, W, nh, k, mode)
    p4 = ref.make_plan(1, 21, 45, 80, 40, 128, 4, ref.TOKEN)
    assert sorted(set(p4.sub_len)) == [4620, 5040]
    g4 = ref.make_plan(1, 21, 45, 80, 40, 128, 4, ref.GROUP)
    assert sorted(set(g4.sub_len)) == [3780, 5040]
    # 720P: (2*19320^2 + 2*18480^2) * 40 heads pairs, 4*d FLOP each
    assert ref.make_plan(1, 21, 45, 80, 40, 128, 2, ref.TOKEN).flops == 4 * 128 * 40 * (2 * 19320**2 + 2 * 18480**2)


def test_planted_map_mistakes_are_caught():
    """Plausible mistakes in the index function fail the pins above (the
    mistake is planted in a copy of the oracle's closed form, on the CPU)."""
    T, H, W, k = 1, 4, 4, 2

    def swapped(Tt, Hh, Ww, kk, mode):            # p and q exchanged
        G = ref.gather_map(Tt, Hh, Ww, kk, mode)
        return G.reshape(kk, kk, -1).transpose(1, 0, 2).reshape(kk * kk, -1)

    def group_as_token(Tt, Hh, Ww, kk, mode):      # group-wise rule forgotten
        return ref.gather_map(Tt, Hh, Ww, kk, ref.TOKEN)

    gold_tok = load_golden("map_token_T1_H4_W4_k2.txt")
    gold_grp = load_golden("map_group_T1_H4_W4_k2.txt")
    assert not np.array_equal(swapped(T, H, W, k, ref.TOKEN), gold_tok)
    assert not np.array_equal(group_as_token(T, H, W, k, ref.GROUP), gold_grp)
