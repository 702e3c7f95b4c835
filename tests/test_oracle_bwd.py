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
