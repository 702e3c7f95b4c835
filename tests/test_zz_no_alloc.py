"""The allocation-free quantizer (skiparse_quant_fp8_noalloc) against the
workspace one (skiparse_quant_fp8), both through the C ABI: codes and scales
bit for bit, on two calls in a row, the second on a smaller input (the
library-held scratch keeps the first call's partial maxima, which the second
must not read)."""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(x, y, sc, fp8_max=448.0, eps=1e-12, x_dtype=None):
    """The C entry point itself (argument types set by the binding's loader)."""
    f = sk.lib().skiparse_quant_fp8_noalloc
    if x_dtype is None:
        x_dtype = sk.BF16 if x.dtype == torch.bfloat16 else sk.F32
    return f(x.data_ptr(), x_dtype, x.numel(), y.data_ptr(), sc.data_ptr(), fp8_max, eps,
             torch.cuda.current_stream().cuda_stream)


def _pair(x, fp8_max=448.0):
    y_ref = torch.empty(x.numel(), dtype=torch.uint8, device=DEV)
    s_ref = torch.empty(2, dtype=torch.float32, device=DEV)
    sk.skiparse_quant_fp8(x, y_ref, s_ref, fp8_max)
    y = torch.full((x.numel(),), 0xAB, dtype=torch.uint8, device=DEV)
    s = torch.full((2,), float("nan"), dtype=torch.float32, device=DEV)
    assert _noalloc(x, y, s, fp8_max) == sk.OK, sk.skiparse_last_error()
    torch.cuda.synchronize()
    return y_ref.cpu(), s_ref.cpu(), y.cpu(), s.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    # first call: a large tensor with a big outlier, so the scratch holds large
    # partial maxima; second call: a smaller tensor (fewer work-groups)
    big = torch.from_numpy(wl.normal_tensor((1, 1, 1, 1, 1, 9 * 2**20 + 3), 71, 0)).to(dtype)
    big[..., 12345] = 900.0
    small = torch.from_numpy(wl.normal_tensor((1, 1, 1, 1, 1, 70001), 72, 0)).to(dtype)
    for x in (big, small):
        xd = x.to(DEV)
        y_ref, s_ref, y, s = _pair(xd)
        assert torch.equal(s, s_ref), (s, s_ref)
        assert torch.equal(y, y_ref)
    # the second call's scale is its own tensor's, not the first call's maximum
    assert s[0].item() == np.float32(448.0) / (np.float32(np.abs(small.float().numpy()).max()) + np.float32(1e-12))


def test_noalloc_argument_errors():
    x = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(64, dtype=torch.uint8, device=DEV)
    s = torch.empty(2, dtype=torch.float32, device=DEV)
    assert _noalloc(x, y, s, x_dtype=7) == sk.EINVAL
    assert _noalloc(x, y, s, fp8_max=0.0) == sk.EINVAL
    assert _noalloc(x, x.view(torch.uint8)[:64], s) == sk.EINVAL          # y overlaps x


def test_noalloc_under_graph_capture():
    """The callers it is for: quantization of Q, K, V through the shared
    scratch and the e4m3 attention, captured in one graph and replayed three
    times.  Between replays an eager call quantizes another tensor through the
    same scratch; every replay must still equal the eager result bit for bit
    (each call writes every partial maximum it reads)."""
    shp = (1, 3, 13, 22, 2, 128)
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 1201, i)).to(torch.bfloat16).to(DEV) for i in range(3))
    plan = sk.skiparse_plan_init(*shp, 2, sk.MODE_GROUP)
    codes = [torch.empty(shp, dtype=torch.uint8, device=DEV) for _ in range(3)]
    scales = torch.empty((3, 2), dtype=torch.float32, device=DEV)
    o = torch.empty_like(q)

    def run(stream=None):
        for t, c_, i in zip((q, k, v), codes, range(3)):
            sk.skiparse_quant_fp8_noalloc(t, c_, scales[i], stream=stream)   # raises on an error code
        sk.skiparse_attn_fwd(plan, sk.FP8_E4M3, *codes, o, descale_qkv=scales, stream=stream)

    run()
    torch.cuda.synchronize()
    want = [o.clone(), scales.clone()] + [c_.clone() for c_ in codes]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(s)
    other = torch.from_numpy(wl.normal_tensor((1, 1, 1, 1, 1, 3 * 2**20 + 5), 1202, 0) * np.float32(50.0)).to(DEV)
    oy = torch.empty(other.numel(), dtype=torch.uint8, device=DEV)
    osc = torch.empty(2, dtype=torch.float32, device=DEV)
    for rep in range(3):
        for t in [o, scales]:
            t.fill_(float("nan"))
        for c_ in codes:
            c_.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp in zip([o, scales] + codes, want):
            assert torch.equal(got, exp), f"replay {rep} differs from the eager result"
        assert _noalloc(other, oy, osc) == sk.OK     # overwrites the scratch between replays
        torch.cuda.synchronize()
