"""The bf16 forward past the 32-bit offset limits.  A (1, 1, 4096, 4096, 1,
128) tensor has 2^24 tokens and 4 GiB per batch sample, so the kernels find
rows through the index function with 64-bit offsets.  At k = 8 the 64
subsequences hold 262,144 tokens each.  The inputs come from the counter-based
generator of the workloads module (drawn on the device; the oracle forms only
the rows it needs on the host), with Q and K scaled by 8 so that each query's
softmax is peaked and its output depends on which key rows were read.  Sampled
rows of three subsequences (the first, a middle one, the last, which holds the
tensor's last token) against the oracle at the bf16 bar."""

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import skiparse_ref as ref

pytestmark = pytest.mark.gpu

SHAPE = (1, 1, 4096, 4096, 1, 128)
KF = 8
GAIN = (8.0, 8.0, 1.0)          # Q, K, V
TOL = 2e-2


class HashRows:
    """The (B, N, heads, d) view of a hash tensor that the oracle indexes with
    [b, token indices, head]; rows are formed on demand."""

    def __init__(self, tensor_id, gain, shape=SHAPE):
        B, T, H, W, nh, d = shape
        self.shape = (B, T * H * W, nh, d)
        self.t, self.gain = tensor_id, gain

    def __getitem__(self, key):
        b, idx, h = key
        B, N, nh, d = self.shape
        idx = np.asarray(idx, np.int64)
        flat = ((b * N + idx)[:, None] * nh + h) * d + np.arange(d)[None, :]
        return wl.hash_values(self.t, flat, self.gain)


@pytest.mark.parametrize("mode", [sk.MODE_TOKEN, sk.MODE_GROUP])
def test_bf16_past_32bit_offsets(mode):
    B, T, H, W, nh, d = SHAPE
    N = T * H * W
    assert N >= 1 << 24 and N * nh * d * 2 >= 1 << 32
    q, k, v = (wl.hash_fill_(torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda"), i, GAIN[i])
               for i in range(3))
    o = sk.attention(q, k, v, KF, mode)
    torch.cuda.synchronize()
    members = ref.subsequence_members(T, H, W, KF, mode)
    rng = np.random.default_rng(7)
    toks = []
    for s in (0, len(members) // 2, len(members) - 1):
        mem = members[s]
        toks += [int(mem[0]), int(mem[-1])] + [int(x) for x in rng.choice(mem, 2, replace=False)]
    toks = np.array(sorted(set(toks)), np.int64)
    assert toks[-1] == N - 1                            # the tensor's last token is sampled
    got = o.view(B, N, nh, d)[0, torch.from_numpy(toks).cuda(), 0].float().cpu().numpy().astype(np.float64)
    del q, k, v, o
    qs, ks, vs = (HashRows(i, GAIN[i]) for i in range(3))
    want = ref.attention_rows(qs, ks, vs, T, H, W, KF, mode, 0, 0, toks)
    assert np.max(np.abs(want)) > 0.05                 # peaked softmax: the rows carry V's values
    err = np.max(np.abs(got - want)) / max(1.0, np.max(np.abs(want)))
    assert err <= TOL, err


def exact_amax_index(tensor_id, n):
    """An element index below n whose hash is below 256 (value exactly -0.5
    times the gain, the largest magnitude the generator makes), found by
    solving i * HASH_MUL + t * HASH_TENSOR = r (mod 2^32) for r = 0, 1, ...;
    None if there is none below 2^14 tries."""
    inv = pow(wl.HASH_MUL, -1, 1 << 32)
    c = tensor_id * wl.HASH_TENSOR
    for r in range(1 << 14):
        i = ((r - c) * inv) % (1 << 32)
        if i < n and ((i * wl.HASH_MUL + c) % (1 << 32)) < 256:
            return i
    return None


class DequantRows(HashRows):
    """Rows of a hash tensor after per-tensor e4m3 quantization with the
    oracle's codec at the scale 448 / (amax + 1e-12), amax = 0.5 * gain."""

    def __init__(self, tensor_id, gain, shape=SHAPE):
        super().__init__(tensor_id, gain, shape)
        from oracle import fp8_ref as f8
        self.f8 = f8
        self.scale = f8.per_tensor_scale(np.float32(0.5 * gain))

    def __getitem__(self, key):
        v = super().__getitem__(key)
        codes = self.f8.e4m3_encode((v * self.scale).astype(np.float32))
        return self.f8.dequantize(codes, self.scale)


def test_fp8_past_32bit_offsets():
    """Per-tensor quantization over 2^31 elements and the e4m3 forward on the
    64-bit path, token-wise, at the fp8 bar."""
    mode = sk.MODE_TOKEN
    B, T, H, W, nh, d = SHAPE
    N = T * H * W
    numel = N * nh * d
    assert numel >= 1 << 31
    for i in range(3):                                   # amax = 0.5 * gain exactly
        assert exact_amax_index(i, numel) is not None
    q, k, v = (wl.hash_fill_(torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda"), i, GAIN[i])
               for i in range(3))
    o, codes, scales = sk.attention_fp8(q, k, v, KF, mode)
    torch.cuda.synchronize()
    dq = [DequantRows(i, GAIN[i]) for i in range(3)]
    got_scales = scales.cpu().numpy()
    for i in range(3):
        assert got_scales[i, 0] == dq[i].scale, (i, got_scales[i], dq[i].scale)
    members = ref.subsequence_members(T, H, W, KF, mode)
    rng = np.random.default_rng(8)
    toks = []
    for s in (0, len(members) // 2, len(members) - 1):
        mem = members[s]
        toks += [int(mem[0]), int(mem[-1])] + [int(x) for x in rng.choice(mem, 2, replace=False)]
    toks = np.array(sorted(set(toks)), np.int64)
    assert toks[-1] == N - 1
    sel = torch.from_numpy(toks).cuda()
    got = o.view(B, N, nh, d)[0, sel, 0].float().cpu().numpy().astype(np.float64)
    got_codes = codes[2].view(B, N, nh, d)[0, sel, 0].cpu().numpy()
    del q, k, v, o, codes
    want_codes = dq[2].f8.e4m3_encode((HashRows(2, GAIN[2])[0, toks, 0] * dq[2].scale).astype(np.float32))
    np.testing.assert_array_equal(got_codes, want_codes)    # V's codes at the sampled rows, bit for bit
    want = ref.attention_rows(*dq, T, H, W, KF, mode, 0, 0, toks)
    assert np.max(np.abs(want)) > 0.05
    err = np.max(np.abs(got - want)) / max(1.0, np.max(np.abs(want)))
    assert err <= 6e-2, err


# The training path past the same limit with many heads instead of many
# tokens: 2^19 tokens of 64 heads (16 KB per token), 8 GiB per tensor, so byte
# offsets within a sample reach 2^33 while the oracle's key gradients stay
# cheap (8192-member subsequences at k = 8).  The training forward, dQ and
# dK/dV all take the index-function row source with 64-bit offsets here.
BWD_SHAPE = (1, 2, 512, 512, 64, 128)
BWD_GAIN = (4.0, 4.0, 1.0, 1.0)     # Q, K, V, dO


def test_bwd_past_32bit_offsets():
    """dQ, dK, dV of sampled rows (the first and the last subsequence, which
    holds the tensor's last token; the first and the last head) against the
    oracle's float64 gradients, at the bf16 backward's bar (2e-2 of each
    tensor's largest sampled entry)."""
    from oracle import skiparse_bwd as bwd
    mode = sk.MODE_TOKEN
    B, T, H, W, nh, d = BWD_SHAPE
    N = T * H * W
    assert N * nh * d * 2 > 1 << 32
    q, k, v, do = (wl.hash_fill_(torch.empty(BWD_SHAPE, dtype=torch.bfloat16, device="cuda"), i, BWD_GAIN[i])
                   for i in range(4))
    out, lse = sk.attention_train(q, k, v, KF, mode)
    dq, dk, dv = sk.attention_bwd(q, k, v, out, do, lse, KF, mode)
    torch.cuda.synchronize()
    del q, k, v, do, out, lse
    members = ref.subsequence_members(T, H, W, KF, mode)
    rows = [HashRows(i, BWD_GAIN[i], BWD_SHAPE) for i in range(4)]
    rng = np.random.default_rng(9)
    worst = 0.0
    for h in (0, nh - 1):
        toks = []
        for s in (0, len(members) - 1):
            mem = members[s]
            toks += [int(mem[0]), int(mem[-1])] + [int(x) for x in rng.choice(mem, 2, replace=False)]
        toks = np.array(sorted(set(toks)), np.int64)
        assert toks[-1] == N - 1
        sel = torch.from_numpy(toks).cuda()
        got = [g.view(B, N, nh, d)[0, sel, h].float().cpu().numpy().astype(np.float64) for g in (dq, dk, dv)]
        want = [bwd.dq_rows(*rows, T, H, W, KF, mode, 0, h, toks)]
        want += list(bwd.dkv_rows(*rows, T, H, W, KF, mode, 0, h, toks))
        for name, g_, w_ in zip(("dq", "dk", "dv"), got, want):
            scale = np.max(np.abs(w_))
            assert scale > 1e-3, name                     # a gradient worth checking
            worst = max(worst, np.max(np.abs(g_ - w_)) / scale)
    del dq, dk, dv
    torch.cuda.empty_cache()
    print(f"\n[64-bit backward] worst error {worst:.3e} of each gradient's largest sampled entry")
    assert worst <= TOL, worst


def test_bwd_fp8_past_32bit_offsets():
    """The 8-bit backward on the same shape, on the e4m3 codes of Q, K, V and
    dO (each amax is 0.5 * gain exactly, from the generator), all on 64-bit
    offsets.  As in the small 8-bit tests, the backward alone is checked: the
    forward's output and log-sum-exp rows of the sampled subsequences are
    replaced by the oracle's (O rounded to bf16), so the bar is the bf16
    backward's 2e-2; the chained step's extra error from the e4m3 forward is
    covered by the sampled 720P-5s test."""
    from oracle import skiparse_bwd as bwd
    mode = sk.MODE_GROUP
    B, T, H, W, nh, d = BWD_SHAPE
    N = T * H * W
    numel = N * nh * d
    assert numel * 2 > 1 << 32
    for i in range(4):
        assert exact_amax_index(i, numel) is not None
    q, k, v, do = (wl.hash_fill_(torch.empty(BWD_SHAPE, dtype=torch.bfloat16, device="cuda"), i, BWD_GAIN[i])
                   for i in range(4))
    out, lse, codes, scales = sk.attention_train_fp8(q, k, v, KF, mode)
    del q, k, v
    members = ref.subsequence_members(T, H, W, KF, mode)
    rows = [DequantRows(i, BWD_GAIN[i], BWD_SHAPE) for i in range(4)]
    h = nh // 2
    subs = (0, len(members) - 1)
    for s in subs:                                   # the oracle's O and log-sum-exp for these rows
        mem = members[s]
        qq, kk, vv = (r[0, mem, h] for r in rows[:3])
        sc = (qq @ kk.T) / np.sqrt(d)
        m = sc.max(axis=1, keepdims=True)
        e = np.exp(sc - m)
        z = e.sum(axis=1, keepdims=True)
        sel = torch.from_numpy(mem).cuda()
        out.view(B, N, nh, d)[0, sel, h] = torch.from_numpy(((e / z) @ vv).astype(np.float32)).to(torch.bfloat16).cuda()
        lse.view(B, N, nh)[0, sel, h] = torch.from_numpy((m + np.log(z))[:, 0].astype(np.float32)).cuda()
    dq, dk, dv = sk.attention_bwd_fp8(codes, scales, out, do, lse, KF, mode)
    torch.cuda.synchronize()
    del do, out, lse, codes, scales
    rng = np.random.default_rng(10)
    toks = []
    for s in subs:
        mem = members[s]
        toks += [int(mem[0]), int(mem[-1])] + [int(x) for x in rng.choice(mem, 2, replace=False)]
    toks = np.array(sorted(set(toks)), np.int64)
    assert toks[-1] == N - 1
    sel = torch.from_numpy(toks).cuda()
    got = [g.view(B, N, nh, d)[0, sel, h].float().cpu().numpy().astype(np.float64) for g in (dq, dk, dv)]
    want = [bwd.dq_rows(*rows, T, H, W, KF, mode, 0, h, toks)]
    want += list(bwd.dkv_rows(*rows, T, H, W, KF, mode, 0, h, toks))
    worst = 0.0
    for name, g_, w_ in zip(("dq", "dk", "dv"), got, want):
        scale = np.max(np.abs(w_))
        assert scale > 1e-3, name
        worst = max(worst, np.max(np.abs(g_ - w_)) / scale)
    del dq, dk, dv
    torch.cuda.empty_cache()
    print(f"\n[64-bit 8-bit backward] worst error {worst:.3e} of each gradient's largest sampled entry")
    assert worst <= TOL, worst
