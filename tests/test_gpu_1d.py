"""GPU parity of the Skiparse-1D modes (the 1D skip rule on each frame's
flattened (h, w), stride k*k) through the C ABI against the oracle: device
index map bit-exact; fp32, bf16 and fp8 forward element by element on small
shapes; the bf16 forward and backward on sampled rows of the 720P-5s shape;
the backward element by element on small shapes.  Bars as in the 2D tests."""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import skiparse_bwd as bwd
from oracle import skiparse_ref as ref
from test_gpu_bwd import check_full_size, check_lse, inputs, np64, rel_err
from test_gpu_fp8 import oracle_dequant
from test_gpu_parity import TOL, check_sampled, err_ratio, run, to_np64, workload_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
MODES = [sk.MODE_TOKEN_1D, sk.MODE_GROUP_1D]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("T,H,W", [(1, 2, 3), (2, 3, 3), (1, 4, 5), (21, 45, 80), (3, 9, 70), (1, 1, 1)])
def test_device_index_map_bit_exact_1d(T, H, W, k, mode):
    plan = sk.skiparse_plan_init(1, T, H, W, 1, 128, k, mode)
    out = torch.full((plan.n_sub * plan.sub_len_padded,), -7, dtype=torch.int32, device=DEV)
    sk.skiparse_index_map_device(plan, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(plan.n_sub, plan.sub_len_padded)
    np.testing.assert_array_equal(got, ref.gather_map(T, H, W, k, mode))


SMALL = [((1, 3, 13, 22, 2, 128), 2), ((2, 2, 9, 17, 3, 128), 2), ((1, 3, 13, 22, 2, 64), 2),
         ((1, 1, 1, 1, 1, 128), 2), ((1, 4, 2, 3, 2, 128), 2), ((1, 2, 10, 10, 2, 128), 1)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shp,kf", SMALL)
def test_bf16_small_1d(shp, kf, mode):
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 601, i)).to(torch.bfloat16) for i in range(3))
    o = run(q, k, v, kf, mode)
    r = ref.skiparse_attention(to_np64(q), to_np64(k), to_np64(v), kf, mode)
    assert err_ratio(to_np64(o), r) <= TOL["bf16"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_small_1d(d, mode):
    shp = (2, 3, 7, 11, 2, d)
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 602, i)) for i in range(3))
    o = run(q, k, v, 2, mode)
    r = ref.skiparse_attention(to_np64(q), to_np64(k), to_np64(v), 2, mode)
    assert err_ratio(to_np64(o), r) <= TOL["f32"]


@pytest.mark.parametrize("mode", MODES)
def test_fp8_small_1d(mode):
    shp = (1, 3, 13, 22, 2, 128)
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 603, i, outliers=True)).to(torch.bfloat16) for i in range(3))
    out, codes, scales = sk.attention_fp8(q.to(DEV), k.to(DEV), v.to(DEV), 2, mode)
    torch.cuda.synchronize()
    deq = []
    for t, c_dev, i in zip((q, k, v), codes, range(3)):
        dq, c_ref, s_ref = oracle_dequant(t)
        np.testing.assert_array_equal(c_dev.cpu().numpy().reshape(-1), c_ref)
        deq.append(dq)
    r = ref.skiparse_attention(*deq, 2, mode)
    assert err_ratio(out.float().cpu().numpy(), r) <= TOL["fp8"]


@pytest.mark.parametrize("mode", MODES)
def test_bf16_workload_sampled_1d(mode):
    w, cpu, dev = workload_inputs("720p_5s")
    out = sk.attention(*dev, 2, mode)
    torch.cuda.synchronize()
    check_sampled(w, cpu, out, 2, mode, [0, w.heads - 1], seed=70 + mode, tol=TOL["bf16"])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shp,kf", SMALL[:2] + SMALL[3:5])
def test_bwd_small_1d(shp, kf, mode):
    q, k, v, do = inputs(shp, 604)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = sk.attention_train(qd, kd, vd, kf, mode)
    grads = sk.attention_bwd(qd, kd, vd, out, dod, lse, kf, mode)
    torch.cuda.synchronize()
    want = bwd.skiparse_attention_bwd(np64(q), np64(k), np64(v), np64(do), kf, mode)
    check_lse(lse.cpu().numpy(), q, k, kf, mode)
    for name, g, w_ in zip(("dq", "dk", "dv"), grads, want):
        assert rel_err(np64(g), w_) <= 2e-2, name


@pytest.mark.parametrize("mode", MODES)
def test_bwd_workload_sampled_1d(mode):
    w = wl.WORKLOADS["720p_5s"]
    check_full_size(w.shape, 2, mode, w.seed + 20 + mode, heads_q=[0], heads_kv=[w.heads - 1])
