"""The library's entry points under HIP graph capture: every call only
enqueues kernels on the given stream (no allocation, no memset, no
synchronization), so a captured sequence replays the same work.  Each graph
is replayed several times with eager work and synchronizations in between,
and every replay must equal the eager result bit for bit (the kernels are
deterministic)."""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bf16(shape, seed, tid):
    return torch.from_numpy(wl.normal_tensor(shape, seed, tid)).to(torch.bfloat16).to(DEV)


def replay_and_check(graph, outputs, expected, stream, eager_between):
    for rep in range(3):
        for o in outputs:
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, expected):
            assert torch.equal(o, e), f"replay {rep} differs from the eager result"
        eager_between()
        torch.cuda.synchronize()


def capture(fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


@pytest.mark.parametrize("mode", [sk.MODE_TOKEN, sk.MODE_GROUP])
def test_graph_bf16_forward(mode):
    shp = (1, 3, 13, 22, 2, 128)
    q, k, v = (bf16(shp, 1101, i) for i in range(3))
    plan = sk.skiparse_plan_init(*shp, 2, mode)
    o = torch.empty_like(q)
    sk.skiparse_attn_fwd(plan, sk.BF16, q, k, v, o)
    torch.cuda.synchronize()
    want = o.clone()
    s = torch.cuda.Stream()
    g = capture(lambda: sk.skiparse_attn_fwd(plan, sk.BF16, q, k, v, o, stream=s), s)
    other = torch.empty_like(q)
    replay_and_check(g, [o], [want], s, lambda: sk.skiparse_attn_fwd(plan, sk.BF16, k, q, v, other))


def test_graph_training_step():
    """Forward keeping the log-sum-exp and the backward pass, one graph."""
    shp = (1, 2, 9, 17, 2, 128)
    q, k, v, do = (bf16(shp, 1102, i) for i in range(4))
    plan = sk.skiparse_plan_init(*shp, 2, sk.MODE_GROUP)
    o = torch.empty_like(q)
    B, T, H, W, nh, d = shp
    lse = torch.empty((B, T * H * W, nh), dtype=torch.float32, device=DEV)
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(sk.skiparse_attn_bwd_workspace_bytes(plan), dtype=torch.uint8, device=DEV)

    def step(stream=None):
        sk.skiparse_attn_fwd_lse(plan, sk.BF16, q, k, v, o, lse, stream=stream)
        sk.skiparse_attn_bwd(plan, sk.BF16, q, k, v, o, do, lse, *grads, workspace=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    want = [o.clone(), lse.clone()] + [g_.clone() for g_ in grads]
    s = torch.cuda.Stream()
    g = capture(lambda: step(s), s)
    replay_and_check(g, [o, lse] + grads, want, s, lambda: sk.attention(v, k, q, 2, sk.MODE_TOKEN))


def test_graph_fp8_path():
    """Per-tensor quantization of Q, K, V and the e4m3 attention, one graph."""
    shp = (1, 3, 13, 22, 2, 128)
    q, k, v = (bf16(shp, 1103, i) for i in range(3))
    plan = sk.skiparse_plan_init(*shp, 2, sk.MODE_TOKEN)
    codes = [torch.empty(shp, dtype=torch.uint8, device=DEV) for _ in range(3)]
    scales = torch.empty((3, 2), dtype=torch.float32, device=DEV)
    wss = [torch.empty(sk.skiparse_quant_fp8_workspace_bytes(q.numel()), dtype=torch.uint8, device=DEV)
           for _ in range(3)]
    o = torch.empty_like(q)

    def run(stream=None):
        for t, c_, i in zip((q, k, v), codes, range(3)):
            sk.skiparse_quant_fp8(t, c_, scales[i], workspace=wss[i], stream=stream)
        sk.skiparse_attn_fwd(plan, sk.FP8_E4M3, *codes, o, descale_qkv=scales, stream=stream)

    run()
    torch.cuda.synchronize()
    want = [o.clone(), scales.clone()] + [c_.clone() for c_ in codes]
    s = torch.cuda.Stream()
    g = capture(lambda: run(s), s)
    replay_and_check(g, [o, scales] + codes, want, s, lambda: sk.attention_fp8(v, q, k, 2, sk.MODE_GROUP))


def test_graph_fp8_block():
    """The whole fp8 attention block (19 launches), one graph."""
    grid, heads = (1, 3, 13, 22), 2
    C = heads * 128
    x = torch.from_numpy(wl.normal_tensor(grid + (C,), 1104, 0)).to(torch.bfloat16).to(DEV)
    ws_ = [torch.from_numpy(wl.normal_tensor((C, C), 1104, 1 + i) * np.float32(1.0 / np.sqrt(C))).to(DEV)
           for i in range(4)]
    w_codes, w_scales = sk.quantize_weights(*ws_)
    plan = sk.skiparse_plan_init(*grid, heads, 128, 2, sk.MODE_GROUP)
    work = torch.empty(sk.skiparse_block_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(x)
    sk.skiparse_block_fwd_fp8(plan, x, w_codes, w_scales, y, workspace=work)
    torch.cuda.synchronize()
    want = y.clone()
    s = torch.cuda.Stream()
    g = capture(lambda: sk.skiparse_block_fwd_fp8(plan, x, w_codes, w_scales, y, workspace=work, stream=s), s)
    x2 = x.flip(1).contiguous()
    y2 = torch.empty_like(x)
    replay_and_check(g, [y], [want], s,
                     lambda: sk.skiparse_block_fwd_fp8(plan, x2, w_codes, w_scales, y2, workspace=work))


def test_graph_fp8_training_step():
    """The 8-bit training step, one graph: quantization of Q, K, V, the e4m3
    forward keeping the log-sum-exp, quantization of dO with the gradient
    maximum, the backward pass on the codes."""
    shp = (1, 2, 9, 17, 2, 128)
    q, k, v, do = (bf16(shp, 1105, i) for i in range(4))
    plan = sk.skiparse_plan_init(*shp, 2, sk.MODE_TOKEN)
    B, T, H, W, nh, d = shp
    codes = [torch.empty(shp, dtype=torch.uint8, device=DEV) for _ in range(4)]
    scales = torch.empty((3, 2), dtype=torch.float32, device=DEV)
    dscale = torch.empty(2, dtype=torch.float32, device=DEV)
    qws = torch.empty(sk.skiparse_quant_fp8_workspace_bytes(q.numel()), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, T * H * W, nh), dtype=torch.float32, device=DEV)
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(sk.skiparse_attn_bwd_workspace_bytes(plan), dtype=torch.uint8, device=DEV)

    def step(stream=None):
        for i, t in enumerate((q, k, v)):
            sk.skiparse_quant_fp8(t, codes[i], scales[i], workspace=qws, stream=stream)
        sk.skiparse_attn_fwd_lse_fp8(plan, codes[0], codes[1], codes[2], scales, o, lse, stream=stream)
        sk.skiparse_quant_fp8(do, codes[3], dscale, workspace=qws, stream=stream)
        sk.skiparse_attn_bwd_fp8(plan, codes[0], codes[1], codes[2], scales, o, codes[3], dscale, lse, *grads,
                                 workspace=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    outs = [o, lse, scales, dscale] + codes + grads
    want = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    g = capture(lambda: step(s), s)
    replay_and_check(g, outs, want, s, lambda: sk.attention_train_fp8(v, k, q, 2, sk.MODE_GROUP))
