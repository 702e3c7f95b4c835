"""GPU parity of the training path: the forward's log-sum-exp and the backward
pass (dQ, dK, dV) through the C ABI, against the oracle's float64 gradients
(oracle/skiparse_bwd.py) on the same bf16 inputs.

Bars.  Log-sum-exp: within 2e-4 (absolute, natural log).  When it keeps the
log-sum-exp the kernel sums the unrounded exponentials in fp32 beside the
bf16-rounded ones that normalize O (so O is the same as without it), and
the scores are exact products of the bf16 inputs accumulated in fp32: the
error is that of fp32 accumulation and of v_exp_f32 (about 1e-5 at the
tested sizes, a few hundred sequential additions of 2^-24 each at most),
far inside the bar, while a wrong scale, offset or dropped tile moves it by
far more.  Gradients: max|g - g_ref| <= 2e-2 * max|g_ref| per tensor, the
bf16 bar taken relative to the tensor's largest entry (gradients are often
well below 1, where a max(1, .) normalisation would not test anything).  The
kernels see the bf16 output O of the forward pass, the oracle the exact one;
that difference is inside the bar.  Small shapes are compared element by
element over several 32-row tiles with ragged tails; the 720P-5s shape on
sampled rows.
"""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import skiparse_bwd as bwd
from oracle import skiparse_ref as ref

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2
LSE_TOL = 2e-4


def check_lse(got, q, k, kf, mode):
    want = bwd.attention_lse(np64(q), np64(k), kf, mode)
    np.testing.assert_allclose(np.asarray(got, np.float64), want, rtol=0, atol=LSE_TOL)


def rel_err(got, want):
    """max|got - want| / max|want|, the denominator floored at 1e-3: a gradient
    that is zero in exact arithmetic (a one-member subsequence has P = 1 and
    dS = 0) is held to TOL * 1e-3 absolute, well above its fp32 rounding noise
    (~1e-7) and far below any real mistake."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), "non-finite gradient"
    return float(np.max(np.abs(got - want))) / max(1e-3, float(np.max(np.abs(want))))


def np64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def inputs(shp, seed):
    return [torch.from_numpy(wl.normal_tensor(shp, seed, i)).to(torch.bfloat16) for i in range(4)]


SMALL = [
    ((1, 3, 13, 22, 2, 128), 2, 0),
    ((1, 3, 13, 22, 2, 128), 2, 1),
    ((2, 2, 9, 17, 2, 128), 3, 1),
    ((1, 2, 10, 10, 2, 128), 1, 0),      # k = 1: plain attention over 200 tokens
    ((1, 5, 8, 40, 1, 128), 4, 0),
    ((1, 1, 1, 1, 1, 128), 2, 0),        # one token: three empty subsequences
    ((1, 4, 2, 3, 2, 128), 4, 1),        # most subsequences empty
    ((1, 2, 4, 16, 1, 128), 2, 1),       # 32-member subsequences: exact tiles
    ((1, 2, 70, 66, 1, 128), 8, 0),      # k = 8: 64 subsequences, heavy padding
]


@pytest.mark.parametrize("shp,kf,mode", SMALL)
def test_fwd_lse_small(shp, kf, mode):
    q, k, v, _ = inputs(shp, 401)
    out, lse = sk.attention_train(q.to(DEV), k.to(DEV), v.to(DEV), kf, mode)
    plain = sk.attention(q.to(DEV), k.to(DEV), v.to(DEV), kf, mode)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)                      # the same kernel, LSE written on the side
    check_lse(lse.cpu().numpy(), q, k, kf, mode)


@pytest.mark.parametrize("shp,kf,mode", SMALL)
def test_bwd_small_full_compare(shp, kf, mode):
    q, k, v, do = inputs(shp, 402)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = sk.attention_train(qd, kd, vd, kf, mode)
    dq, dk, dv = sk.attention_bwd(qd, kd, vd, out, dod, lse, kf, mode)
    torch.cuda.synchronize()
    want = bwd.skiparse_attention_bwd(np64(q), np64(k), np64(v), np64(do), kf, mode)
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert rel_err(np64(g), w) <= TOL, name


def test_bwd_deterministic_and_autograd():
    shp, kf, mode = (1, 3, 13, 22, 2, 128), 2, 1
    q, k, v, do = (t.to(DEV) for t in inputs(shp, 403))
    out, lse = sk.attention_train(q, k, v, kf, mode)
    a = sk.attention_bwd(q, k, v, out, do, lse, kf, mode)
    b = sk.attention_bwd(q, k, v, out, do, lse, kf, mode)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o2 = sk.SkiparseAttention.apply(qa, ka, va, kf, mode)
    o2.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o2.detach(), out)
    for x, y, g in zip(a, b, (qa.grad, ka.grad, va.grad)):
        assert torch.equal(x, y)
        assert torch.equal(x, g)


def test_autograd_on_permuted_views():
    """Q, K, V given as dense permuted views of (B, heads, T, H, W, d) storage
    (not contiguous in the (B, T, H, W, heads, d) order the library reads):
    the op's output and all three gradients equal those of the contiguous
    tensors, in the caller's layout."""
    shp, kf, mode = (1, 3, 13, 22, 2, 128), 2, 0
    q, k, v, do = (t.to(DEV) for t in inputs(shp, 405))
    ref_in = [t.clone().requires_grad_(True) for t in (q, k, v)]
    o_ref = sk.SkiparseAttention.apply(*ref_in, kf, mode)
    o_ref.backward(do)
    # the same values stored head-major, viewed back as (B, T, H, W, heads, d)
    perm = [t.permute(0, 4, 1, 2, 3, 5).contiguous().permute(0, 2, 3, 4, 1, 5) for t in (q, k, v)]
    assert not perm[0].is_contiguous() and torch.equal(perm[0], q)
    views = [t.detach().requires_grad_(True) for t in perm]
    o_view = sk.SkiparseAttention.apply(*views, kf, mode)
    o_view.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o_view.detach(), o_ref.detach())
    for a, b in zip(views, ref_in):
        assert torch.equal(a.grad, b.grad)


def test_bwd_subsequence_ranges():
    """Runs over [0, 1) and [1, 4) give the full call's gradients bit for bit,
    and rows outside the run subsequences are left untouched."""
    shp, kf, mode = (1, 2, 11, 14, 2, 128), 2, 0
    q, k, v, do = (t.to(DEV) for t in inputs(shp, 404))
    out, lse = sk.attention_train(q, k, v, kf, mode)
    full = sk.attention_bwd(q, k, v, out, do, lse, kf, mode)
    plan = sk.skiparse_plan_init(*shp, kf, mode)
    parts = [torch.full(shp, float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    sk.skiparse_attn_bwd(plan, sk.BF16, q, k, v, out, do, lse, *parts, sub_begin=1, sub_count=3)
    torch.cuda.synchronize()
    members = ref.subsequence_members(*shp[1:4], kf, mode)
    rows = lambda t: t.reshape(shp[0], -1, shp[4], shp[5])
    for p in parts:
        assert torch.isnan(rows(p)[:, members[0]].float()).all()
    sk.skiparse_attn_bwd(plan, sk.BF16, q, k, v, out, do, lse, *parts, sub_begin=0, sub_count=1)
    torch.cuda.synchronize()
    for p, f in zip(parts, full):
        assert torch.equal(p, f)


def sampled(members, rng, per_sub=6):
    toks = []
    for mem in members:
        if mem.size:
            toks += [mem[0], mem[-1]] + list(rng.choice(mem, size=min(per_sub, mem.size), replace=False))
    return np.unique(np.array(toks, np.int64))


def check_full_size(shp, kf, mode, seed, heads_q, heads_kv, per_sub=6):
    B, T, H, W, nh, d = shp
    N = T * H * W
    cpu = [torch.from_numpy(wl.normal_tensor(shp, seed, i)).to(torch.bfloat16) for i in range(4)]
    q, k, v, do = (t.to(DEV) for t in cpu)
    out, lse = sk.attention_train(q, k, v, kf, mode)
    dq, dk, dv = sk.attention_bwd(q, k, v, out, do, lse, kf, mode)
    torch.cuda.synchronize()
    qn, kn, vn, don = (t.float().numpy().reshape(B, N, nh, d) for t in cpu)
    g = [t.float().cpu().numpy().reshape(B, N, nh, d) for t in (dq, dk, dv)]
    members = ref.subsequence_members(T, H, W, kf, mode)
    rng = np.random.default_rng(seed)
    worst = [0.0, 0.0, 0.0]
    for h in heads_q:
        toks = sampled(members, rng, per_sub)
        want = bwd.dq_rows(qn, kn, vn, don, T, H, W, kf, mode, 0, h, toks)
        worst[0] = max(worst[0], rel_err(g[0][0, toks, h], want))
    for h in heads_kv:
        toks = sampled(members, rng, per_sub)
        wk, wv = bwd.dkv_rows(qn, kn, vn, don, T, H, W, kf, mode, 0, h, toks)
        worst[1] = max(worst[1], rel_err(g[1][0, toks, h], wk))
        worst[2] = max(worst[2], rel_err(g[2][0, toks, h], wv))
    assert max(worst) <= TOL, worst


@pytest.mark.parametrize("mode", [0, 1])
def test_bwd_workload_sampled(mode):
    w = wl.WORKLOADS["720p_5s"]
    check_full_size(w.shape, w.k, mode, w.seed + 10, heads_q=[0, w.heads - 1], heads_kv=[w.heads // 2])


def test_bwd_k1_workload_sampled():
    """Full attention (k = 1) at the 720P-5s shape: one subsequence of 75600
    tokens, so the training forward and the dQ kernel stream 1182 and 2363 key
    tiles per work-group, the running max and sums run over the whole frame
    stack, and dQ takes rows from the index function (n is past the token
    table).  Sampled dQ rows in two heads against the oracle.  dK and dV run
    the same kernel as at k = 2 with a longer query loop; the oracle's rows for
    them would take minutes here (every query's softmax over 75600 keys)."""
    w = wl.WORKLOADS["720p_5s"]
    check_full_size(w.shape, 1, 0, w.seed + 30, heads_q=[0, w.heads - 1], heads_kv=[], per_sub=24)


def test_bwd_index_function_path():
    """n = 24200 members exceeds the token-table capacity: rows come from the
    index function."""
    check_full_size((1, 1, 22, 1100, 1, 128), 1, 0, 405, heads_q=[0], heads_kv=[0], per_sub=24)


def test_bwd_repeatable_at_720p():
    """Two training steps (forward keeping the log-sum-exp, then the
    backward) on the same 720P-5s inputs give bit-identical O, log-sum-exp
    and gradients: 302 tiles per subsequence in each kernel's loop."""
    shape = wl.WORKLOADS["720p_5s"].shape
    g = torch.Generator(device=DEV)
    g.manual_seed(1007)
    q, k, v, do = (torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16) for _ in range(4))
    runs = []
    for _ in range(2):
        o, lse = sk.attention_train(q, k, v, 2, sk.MODE_TOKEN)
        runs.append((o, lse) + tuple(sk.attention_bwd(q, k, v, o, do, lse, 2, sk.MODE_TOKEN)))
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)
