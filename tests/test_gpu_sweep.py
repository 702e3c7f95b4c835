"""A seeded sweep over 64 small random shapes: every pattern (token-wise,
group-wise, and the two Skiparse-1D rules), k from 1 to 8, ragged H and W
(padding, subsequences of one member or none), one to three heads, batch 1 or
2.  Each case is compared element by element with the oracle on four paths,
at the bars the other tests derive: the bf16 forward (2e-2 of max(1, max|O|)),
the e4m3 forward on the oracle's own quantization (codes and scales bit for
bit, 6e-2), the bf16 training forward and backward (log-sum-exp within 2e-4,
gradients within 2e-2 of each tensor's largest entry), and the 8-bit backward
given the oracle's output and log-sum-exp (2e-2, the row term of dS formed
from that same output)."""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import fp8_ref as f8
from oracle import skiparse_bwd as bwd
from oracle import skiparse_ref as ref

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make_cases(n=64, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        mode = int(rng.integers(0, 4))
        kf = int(rng.integers(1, 3)) if mode >= 2 else int(rng.integers(1, 9))
        B, T = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        H, W = int(rng.integers(1, 38)), int(rng.integers(1, 38))
        heads = int(rng.integers(1, 4))
        if B * T * H * W > 3000:
            continue
        cases.append(((B, T, H, W, heads, 128), kf, mode))
    return cases


CASES = make_cases()


def np64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel_max1(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert np.all(np.isfinite(got))
    return float(np.max(np.abs(got - want))) / max(1.0, float(np.max(np.abs(want))))


def rel_grad(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert np.all(np.isfinite(got))
    return float(np.max(np.abs(got - want))) / max(1e-3, float(np.max(np.abs(want))))


@pytest.mark.parametrize("shp,kf,mode", CASES, ids=[f"{s}-k{k}-m{m}" for s, k, m in CASES])
def test_sweep(shp, kf, mode):
    q, k, v, do = (torch.from_numpy(wl.normal_tensor(shp, 77, i)).to(torch.bfloat16) for i in range(4))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    q64, k64, v64, do64 = (np64(t) for t in (q, k, v, do))

    # bf16 forward
    out = sk.attention(qd, kd, vd, kf, mode)
    torch.cuda.synchronize()
    assert rel_max1(np64(out), ref.skiparse_attention(q64, k64, v64, kf, mode)) <= 2e-2

    # e4m3 forward
    out8, codes, scales = sk.attention_fp8(qd, kd, vd, kf, mode)
    torch.cuda.synchronize()
    t = bwd.quantized_inputs(q64, k64, v64, do64)
    for name, c, i in zip("qkv", codes, range(3)):
        np.testing.assert_array_equal(c.cpu().numpy(), t[name + "8"])
        assert scales[i, 0].item() == float(t["s_" + name])
    o_ref8 = ref.skiparse_attention(t["q"], t["k"], t["v"], kf, mode)
    assert rel_max1(np64(out8), o_ref8) <= 6e-2

    # bf16 training forward and backward
    o, lse = sk.attention_train(qd, kd, vd, kf, mode)
    grads = sk.attention_bwd(qd, kd, vd, o, dod, lse, kf, mode)
    torch.cuda.synchronize()
    assert torch.equal(o, out)
    np.testing.assert_allclose(lse.cpu().numpy().astype(np.float64), bwd.attention_lse(q64, k64, kf, mode),
                               rtol=0, atol=2e-4)
    for g, w in zip(grads, bwd.skiparse_attention_bwd(q64, k64, v64, do64, kf, mode)):
        assert rel_grad(np64(g), w) <= 2e-2

    # 8-bit backward, given the oracle's output and log-sum-exp
    o_in = torch.from_numpy(o_ref8.astype(np.float32)).to(torch.bfloat16)
    lse_in = torch.from_numpy(bwd.attention_lse(t["q"], t["k"], kf, mode).astype(np.float32)).to(DEV)
    dscale = torch.empty(2, dtype=torch.float32, device=DEV)
    do8 = sk.quantize_fp8(dod, scale_out=dscale)[0]
    plan = sk.skiparse_plan_init(*shp, kf, mode)
    g8 = [torch.empty(shp, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    sk.skiparse_attn_bwd_fp8(plan, *codes, scales, o_in.to(DEV), do8, dscale, lse_in, *g8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(do8.cpu().numpy(), t["do8"])
    want8 = bwd.skiparse_attention_bwd(t["q"], t["k"], t["v"], t["do"], kf, mode, o=np64(o_in))
    for g, w in zip(g8, want8):
        assert rel_grad(np64(g), w) <= 2e-2
