"""GPU parity of the fp8 path: per-tensor e4m3 quantization on the device, then
the e4m3 attention kernel, against the oracle run in float64 on inputs the
oracle quantizes and dequantizes itself (from the same bf16 values).  Bar:
6e-2 of max(1, max|O_ref|); codes and scales bit-exact."""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import fp8_ref as f8
from oracle import skiparse_ref as ref

pytestmark = pytest.mark.gpu

TOL = 6e-2
DEV = "cuda"


def err_ratio(got, expect):
    got = np.asarray(got, np.float64)
    expect = np.asarray(expect, np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - expect))) / max(1.0, float(np.max(np.abs(expect))))


def oracle_dequant(x_bf16):
    codes, scale, _ = f8.quantize_per_tensor(x_bf16.float().numpy().reshape(-1))
    return f8.dequantize(codes, scale).reshape(x_bf16.shape), codes, scale


SMALL = [
    ((1, 3, 13, 22, 2, 128), 2, 0),
    ((1, 3, 13, 22, 2, 128), 2, 1),
    ((2, 2, 9, 17, 2, 128), 3, 1),
    ((1, 2, 10, 10, 2, 128), 1, 0),
    ((1, 5, 8, 40, 1, 128), 4, 0),
    ((1, 1, 1, 1, 1, 128), 2, 0),
    ((1, 2, 70, 66, 1, 128), 8, 1),     # k = 8: 64 subsequences, heavy padding
]


@pytest.mark.parametrize("shp,kf,mode", SMALL)
def test_fp8_small_full_compare(shp, kf, mode):
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 55, i, outliers=True)).to(torch.bfloat16) for i in range(3))
    out, codes, scales = sk.attention_fp8(q.to(DEV), k.to(DEV), v.to(DEV), kf, mode)
    torch.cuda.synchronize()
    deq = []
    for t, c_dev, i in zip((q, k, v), codes, range(3)):
        dq, c_ref, s_ref = oracle_dequant(t)
        np.testing.assert_array_equal(c_dev.cpu().numpy().reshape(-1), c_ref)
        assert scales[i, 0].item() == float(s_ref)
        deq.append(dq)
    r = ref.skiparse_attention(*deq, kf, mode)
    assert err_ratio(out.float().cpu().numpy(), r) <= TOL


class LazyDequant:
    """(B, N, heads, d) view of a bf16 tensor that encodes and decodes only
    the rows asked for, with the oracle's per-tensor scale of the whole
    tensor."""

    def __init__(self, x_bf16, B, N, nh, d):
        self.x = x_bf16.view(torch.int16).numpy().reshape(B, N, nh, d)
        amax = np.float32(np.abs(x_bf16.float().numpy()).max())
        self.scale = f8.per_tensor_scale(amax)
        self.shape = (B, N, nh, d)

    def __getitem__(self, idx):
        raw = self.x[idx]
        vals = (raw.astype(np.int32) << 16).view(np.float32)   # bf16 -> f32, exact
        codes = f8.e4m3_encode((vals * self.scale).astype(np.float32))
        return f8.dequantize(codes, self.scale)


@pytest.mark.parametrize("kf,mode", [(2, 0), (2, 1), (4, 0), (4, 1)])
def test_fp8_workload_sampled(kf, mode):
    w = wl.WORKLOADS["720p_5s_fp8"]
    cpu = wl.make_inputs(w)
    out, _, _ = sk.attention_fp8(*(t.to(DEV) for t in cpu), kf, mode)
    torch.cuda.synchronize()
    B, T, H, W, nh, d = w.shape
    N = T * H * W
    lq, lk, lv = (LazyDequant(t, B, N, nh, d) for t in cpu)
    on = out.float().cpu().numpy().reshape(B, N, nh, d)
    rng = np.random.default_rng(kf * 7 + mode)
    members = ref.subsequence_members(T, H, W, kf, mode)
    worst = 0.0
    for h in (0, nh - 1):
        toks = []
        for mem in members:
            if mem.size:
                toks += [mem[0], mem[-1]] + list(rng.choice(mem, size=min(12, mem.size), replace=False))
        toks = np.unique(np.array(toks, np.int64))
        r = ref.attention_rows(lq, lk, lv, T, H, W, kf, mode, 0, h, toks)
        worst = max(worst, err_ratio(on[0, toks, h], r))
    print(f"\n[sampled parity] 720p_5s_fp8 k={kf} mode={mode} e4m3: max err {worst:.3e} of max(1, max|O|)")
    assert worst <= TOL, worst


@pytest.mark.parametrize("mode", [sk.MODE_TOKEN, sk.MODE_GROUP])
def test_fp8_repeatable_at_720p(mode):
    """Three calls of the e4m3 path on the same 720P-5s inputs are
    bit-identical (302 key tiles per subsequence; see the bf16 check)."""
    shape = wl.WORKLOADS["720p_5s_fp8"].shape
    g = torch.Generator(device=DEV)
    g.manual_seed(1005)
    q, k, v = (torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16) for _ in range(3))
    outs = [sk.attention_fp8(q, k, v, 2, mode)[0] for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
