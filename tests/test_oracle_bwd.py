"""Pins of the backward oracle (oracle/skiparse_bwd.py) against what the
mathematics fixes independently of the formulas it writes out:

* central finite differences of the forward oracle (the gradient's definition);
* torch's float64 autograd through its scaled_dot_product_attention, at k = 1
  (plain attention) and under the equivalent block mask for k > 1;
* invariants per subsequence: the dK rows sum to zero, the dV rows sum to the
  dO rows;
* log-sum-exp against torch.logsumexp;
* the sampled-row evaluators against the full oracle;
* planted mistakes (in copies of the formulas here) fail the finite-difference
  check, so the check is sharp enough to catch them.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import skiparse_bwd as bwd
from oracle import skiparse_ref as ref


def rand(shape, seed, i):
    return wl.normal_tensor(shape, seed, i).astype(np.float64)


def loss_grad_fd(fwd, args, g, which, idx, h=1e-5):
    """Central difference of L = sum(fwd(*args) * g) w.r.t. args[which].flat[idx]."""
    out = []
    for j in idx:
        a_p = [x.copy() for x in args]
        a_m = [x.copy() for x in args]
        a_p[which].flat[j] += h
        a_m[which].flat[j] -= h
        out.append((np.sum(fwd(*a_p) * g) - np.sum(fwd(*a_m) * g)) / (2 * h))
    return np.array(out)


FD_CASES = [((1, 2, 5, 6, 2, 8), 2, 0), ((1, 2, 5, 6, 2, 8), 2, 1), ((1, 1, 7, 7, 1, 4), 3, 1),
            ((2, 2, 3, 4, 1, 8), 1, 0)]


@pytest.mark.parametrize("shp,kf,mode", FD_CASES)
def test_bwd_matches_finite_differences(shp, kf, mode):
    q, k, v, g = (rand(shp, 301, i) for i in range(4))
    grads = bwd.skiparse_attention_bwd(q, k, v, g, kf, mode)
    fwd = lambda q_, k_, v_: ref.skiparse_attention(q_, k_, v_, kf, mode)
    rng = np.random.default_rng(7)
    for which in range(3):
        idx = rng.choice(q.size, size=min(40, q.size), replace=False)
        fd = loss_grad_fd(fwd, [q, k, v], g, which, idx)
        an = grads[which].flat[idx]
        np.testing.assert_allclose(an, fd, rtol=1e-6, atol=1e-8)


def torch_sdpa_grads(q, k, v, do, mask=None):
    """float64 autograd through torch's SDPA; (B, N, heads, d) in, grads out."""
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=None if mask is None else torch.tensor(mask))
    o.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
    return tuple(t.grad.numpy().transpose(0, 2, 1, 3) for t in (tq, tk, tv))


@pytest.mark.parametrize("shp,kf,mode", [((1, 2, 4, 6, 2, 16), 1, 0), ((2, 2, 6, 10, 2, 16), 2, 0),
                                         ((2, 2, 6, 10, 2, 16), 2, 1), ((1, 1, 9, 11, 1, 8), 3, 1)])
def test_bwd_matches_torch_autograd(shp, kf, mode):
    q, k, v, do = (rand(shp, 302, i) for i in range(4))
    B, T, H, W, nh, d = shp
    N = T * H * W
    got = bwd.skiparse_attention_bwd(q, k, v, do, kf, mode)
    mask = None if kf == 1 else ref.block_mask(T, H, W, kf, mode)
    want = torch_sdpa_grads(*(x.reshape(B, N, nh, d) for x in (q, k, v, do)), mask=mask)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g.reshape(B, N, nh, d), w, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("shp,kf,mode", [((1, 2, 5, 7, 2, 8), 2, 0), ((2, 1, 9, 10, 1, 8), 3, 1), ((1, 3, 4, 4, 1, 8), 1, 0)])
def test_bwd_invariants_per_subsequence(shp, kf, mode):
    q, k, v, do = (rand(shp, 303, i) for i in range(4))
    B, T, H, W, nh, d = shp
    N = T * H * W
    _, dk, dv = bwd.skiparse_attention_bwd(q, k, v, do, kf, mode)
    dk, dv, dof = (x.reshape(B, N, nh, d) for x in (dk, dv, do))
    for mem in ref.subsequence_members(T, H, W, kf, mode):
        if mem.size == 0:
            continue
        np.testing.assert_allclose(dk[:, mem].sum(axis=1), 0.0, atol=1e-11)
        np.testing.assert_allclose(dv[:, mem].sum(axis=1), dof[:, mem].sum(axis=1), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("shp,kf,mode", [((1, 2, 4, 6, 2, 16), 1, 0), ((1, 2, 6, 10, 2, 16), 2, 1)])
def test_lse_matches_torch_logsumexp(shp, kf, mode):
    q, k, v = (rand(shp, 304, i) for i in range(3))
    B, T, H, W, nh, d = shp
    N = T * H * W
    lse = bwd.attention_lse(q, k, kf, mode)
    s = torch.einsum("bind,bjnd->bnij", torch.tensor(q.reshape(B, N, nh, d)), torch.tensor(k.reshape(B, N, nh, d)))
    s = s / np.sqrt(d)
    if kf > 1:
        s = s.masked_fill(~torch.tensor(ref.block_mask(T, H, W, kf, mode)), float("-inf"))
    want = torch.logsumexp(s, dim=-1).numpy().transpose(0, 2, 1)
    np.testing.assert_allclose(lse, want, rtol=1e-12, atol=1e-12)
    # the weights exp(s - LSE) of each row sum to one
    np.testing.assert_allclose(torch.exp(s - torch.tensor(want.transpose(0, 2, 1))[..., None]).sum(-1).numpy(), 1.0,
                               rtol=1e-12)


@pytest.mark.parametrize("kf,mode", [(2, 0), (2, 1), (1, 0)])
def test_sampled_rows_match_full_oracle(kf, mode):
    shp = (2, 2, 9, 14, 2, 16)
    q, k, v, do = (rand(shp, 305, i) for i in range(4))
    B, T, H, W, nh, d = shp
    N = T * H * W
    dq, dk, dv = (x.reshape(B, N, nh, d) for x in bwd.skiparse_attention_bwd(q, k, v, do, kf, mode))
    qf, kf_, vf, dof = (x.reshape(B, N, nh, d) for x in (q, k, v, do))
    toks = np.array([0, 5, 17, N // 2, N - 1])
    for b in range(B):
        for h in range(nh):
            np.testing.assert_allclose(bwd.dq_rows(qf, kf_, vf, dof, T, H, W, kf, mode, b, h, toks), dq[b, toks, h],
                                       rtol=1e-10, atol=1e-12)
            gk, gv = bwd.dkv_rows(qf, kf_, vf, dof, T, H, W, kf, mode, b, h, toks, chunk=37)
            np.testing.assert_allclose(gk, dk[b, toks, h], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(gv, dv[b, toks, h], rtol=1e-10, atol=1e-12)


# --- planted mistakes: each copy below breaks one step; the FD check must catch it

def _grads_with(q, k, v, do, scale, mistake):
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    dv = (p if mistake == "p_not_transposed" else p.T) @ do
    dp = do @ v.T
    if mistake == "drop_rowsum":
        ds = p * dp
    else:
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = (1.0 if mistake == "dq_scale" else scale) * (ds @ k)
    dk = scale * ((ds if mistake == "dk_no_transpose" else ds.T) @ q)
    return dq, dk, dv


@pytest.mark.parametrize("mistake", ["p_not_transposed", "drop_rowsum", "dq_scale", "dk_no_transpose"])
def test_planted_mistakes_fail_finite_differences(mistake):
    n, d = 6, 6
    q, k, v, g = (rand((n, d), 306, i) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    fwd = lambda q_, k_, v_: ref.softmax_attention(q_, k_, v_, scale)
    ok = _grads_with(q, k, v, g, scale, None)
    bad = _grads_with(q, k, v, g, scale, mistake)
    idx = np.arange(n * d)
    worst = 0.0
    for which in range(3):
        fd = loss_grad_fd(fwd, [q, k, v], g, which, idx)
        np.testing.assert_allclose(ok[which].ravel(), fd, rtol=1e-6, atol=1e-8)   # the correct copy passes
        worst = max(worst, float(np.max(np.abs(bad[which].ravel() - fd))))
    assert worst > 1e-3


# ---------------------------------------------------------------------------
# 8-bit training: quantize per tensor, then the gradients of the dequantized
# tensors.  Inputs built on the e4m3 grid with amax 224 (Q, K, V) and 112 (dO)
# have per-tensor scales 448 / 224 = 2 and 448 / 112 = 4 exactly in fp32 (the
# 1e-12 of the rule is far below half an ulp of either amax), so quantization
# is exact and the 8-bit gradients must equal the plain ones on the same
# values; a path that forgot to dequantize, or scaled one tensor with
# another's maximum, is off by a power of two.
# ---------------------------------------------------------------------------

def grid_tensor(shape, seed, amax, min_abs=0.0):
    """Values code / (448 / amax) for random finite e4m3 codes, one of them 448;
    with min_abs, codes below it in magnitude (other than zero) are left out."""
    from oracle import fp8_ref as f8
    table = f8.e4m3_decode_table()
    finite = np.flatnonzero(np.isfinite(table) & ((np.abs(table) >= min_abs) | (table == 0)))
    rng = np.random.default_rng(seed)
    vals = table[rng.choice(finite, size=int(np.prod(shape)))].astype(np.float64)
    vals[rng.integers(vals.size)] = 448.0
    return (vals * (amax / 448.0)).reshape(shape)


@pytest.mark.parametrize("shp,kf,mode", [((1, 2, 5, 6, 2, 8), 2, 0), ((1, 2, 9, 7, 1, 8), 3, 1)])
def test_fp8_bwd_equals_plain_bwd_on_exact_grid(shp, kf, mode):
    q, k, v = (grid_tensor(shp, 61 + i, 224.0) for i in range(3))
    do = grid_tensor(shp, 64, 112.0)
    dq, dk, dv, t = bwd.skiparse_attention_bwd_fp8(q, k, v, do, kf, mode)
    assert (t["s_q"], t["s_k"], t["s_v"], t["s_do"]) == (2.0, 2.0, 2.0, 4.0)
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        np.testing.assert_array_equal(t[name], x)
    want = bwd.skiparse_attention_bwd(q, k, v, do, kf, mode)
    for got, w in zip((dq, dk, dv), want):
        np.testing.assert_array_equal(got, w)


def test_fp8_gradient_maximum_applies_to_do_only():
    shp = (1, 2, 5, 6, 1, 8)
    q, k, v = (grid_tensor(shp, 71 + i, 224.0) for i in range(3))
    # with maximum 224 the codes of dO are the grid values halved: normal
    # values of at least 2^-5 stay exact when halved (e4m3's smallest normal
    # is 2^-6)
    do = grid_tensor(shp, 74, 112.0, min_abs=2.0 ** -5)
    t = bwd.quantized_inputs(q, k, v, do, fp8_max=448.0, fp8_max_grad=224.0)
    assert (t["s_q"], t["s_k"], t["s_v"], t["s_do"]) == (2.0, 2.0, 2.0, 2.0)
    np.testing.assert_array_equal(t["do"], do)
    q2 = grid_tensor(shp, 75, 224.0, min_abs=2.0 ** -5)
    t2 = bwd.quantized_inputs(q2, k, v, do, fp8_max=224.0, fp8_max_grad=448.0)
    assert (t2["s_q"], t2["s_do"]) == (1.0, 4.0)
    np.testing.assert_array_equal(t2["q"], q2)


@pytest.mark.parametrize("shp,kf,mode", [((1, 2, 5, 6, 2, 8), 2, 0), ((1, 1, 7, 7, 1, 4), 3, 1),
                                         ((1, 1, 1, 1, 1, 8), 2, 0)])
def test_bwd_with_given_output_equals_jacobian_form(shp, kf, mode):
    """The row term from a given output, rowsum(dO * O), equals the Jacobian's
    rowsum(P * dP) when O is the exact forward output (sum_j P_ij dO_i . v_j =
    dO_i . sum_j P_ij v_j); with a perturbed O the gradients move."""
    q, k, v, do = (rand(shp, 81, i) for i in range(4))
    o = ref.skiparse_attention(q, k, v, kf, mode)
    a = bwd.skiparse_attention_bwd(q, k, v, do, kf, mode)
    b = bwd.skiparse_attention_bwd(q, k, v, do, kf, mode, o=o)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)
    c = bwd.skiparse_attention_bwd(q, k, v, do, kf, mode, o=o * (1 + 1e-3))
    assert np.max(np.abs(c[0] - a[0])) > 1e-6
    np.testing.assert_array_equal(c[2], a[2])         # dV does not involve the row term
