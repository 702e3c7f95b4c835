"""GPU parity: the HIP library through its C ABI against the oracle.

Bars: index maps bit-exact; fp32 within 1e-5, bf16 within 2e-2, fp8 within
6e-2 of max(1, max|O_ref|) (max-abs error on the softmax-normalised outputs).
Small shapes are compared element by element over several tiles and ragged
tails; the full workload shapes are compared on sampled rows (first/last rows,
the padding edge, every subsequence) that the oracle computes one by one.
"""

import types

import numpy as np
import pytest
import torch

import fixed_pattern_sparse_amd as sk
import workloads as wl
from oracle import fp8_ref as f8
from oracle import skiparse_ref as ref

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
DEV = "cuda"


def err_ratio(got, expect):
    got = np.asarray(got, np.float64)
    expect = np.asarray(expect, np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - expect))) / max(1.0, float(np.max(np.abs(expect))))


def to_np64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def run(q, k, v, kf, mode, **kw):
    out = sk.attention(q.to(DEV), k.to(DEV), v.to(DEV), kf, mode, **kw)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# index maps
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,H,W", [(2, 8, 8), (1, 3, 5), (21, 45, 80), (21, 48, 80), (21, 32, 52), (3, 9, 70), (1, 1, 1)])
def test_device_index_map_bit_exact(T, H, W, k, mode):
    plan = sk.skiparse_plan_init(1, T, H, W, 1, 128, k, mode)
    out = torch.full((plan.n_sub * plan.sub_len_padded,), -7, dtype=torch.int32, device=DEV)
    sk.skiparse_index_map_device(plan, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(plan.n_sub, plan.sub_len_padded)
    np.testing.assert_array_equal(got, ref.gather_map(T, H, W, k, mode))


# ---------------------------------------------------------------------------
# fp32: the 128-token workload, token-wise then group-wise
# ---------------------------------------------------------------------------

def test_tiny_fp32_chain():
    w = wl.WORKLOADS["tiny"]
    q, k, v = wl.make_inputs(w)
    o1 = run(q, k, v, 2, sk.MODE_TOKEN)
    o2 = run(q, k, o1, 2, sk.MODE_GROUP)
    qn, kn, vn = (to_np64(t) for t in (q, k, v))
    r1 = ref.skiparse_attention(qn, kn, vn, 2, ref.TOKEN)
    r2 = ref.skiparse_attention(qn, kn, to_np64(o1), 2, ref.GROUP)
    assert err_ratio(to_np64(o1), r1) <= TOL["f32"]
    assert err_ratio(to_np64(o2), r2) <= TOL["f32"]
    # the pair against the f64 chain end to end (fp32 layer-1 rounding included)
    r2_chain = ref.skiparse_attention(qn, kn, r1, 2, ref.GROUP)
    assert err_ratio(to_np64(o2), r2_chain) <= TOL["f32"]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kf,mode", [(1, 0), (2, 0), (2, 1), (3, 1)])
def test_fp32_small(d, kf, mode):
    shp = (2, 3, 7, 11, 2, d)
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 77, i)) for i in range(3))
    o = run(q, k, v, kf, mode)
    r = ref.skiparse_attention(to_np64(q), to_np64(k), to_np64(v), kf, mode)
    assert err_ratio(to_np64(o), r) <= TOL["f32"]


# ---------------------------------------------------------------------------
# bf16: element-by-element on shapes spanning several tiles with ragged tails
# ---------------------------------------------------------------------------

SMALL_BF16 = [
    # (B, T, H, W, heads, d), k, mode
    ((1, 3, 13, 22, 2, 128), 2, 0),
    ((1, 3, 13, 22, 2, 128), 2, 1),
    ((2, 2, 9, 17, 3, 128), 3, 1),
    ((1, 2, 10, 10, 2, 128), 1, 0),
    ((1, 5, 8, 40, 1, 128), 2, 1),
    ((1, 3, 13, 22, 2, 64), 2, 0),
    ((1, 2, 9, 17, 2, 64), 3, 1),
    ((1, 1, 1, 1, 1, 128), 2, 0),       # one token: three empty subsequences
    ((1, 4, 2, 3, 2, 128), 4, 1),       # most subsequences empty
    ((1, 2, 70, 66, 1, 128), 8, 0),     # k = 8: 64 subsequences, H and W padded to 128
    ((1, 2, 70, 66, 1, 128), 8, 1),
]


@pytest.mark.parametrize("shp,kf,mode", SMALL_BF16)
def test_bf16_small_full_compare(shp, kf, mode):
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 91, i)).to(torch.bfloat16) for i in range(3))
    o = run(q, k, v, kf, mode)
    r = ref.skiparse_attention(to_np64(q), to_np64(k), to_np64(v), kf, mode)
    assert err_ratio(to_np64(o), r) <= TOL["bf16"]


@pytest.mark.parametrize("direction", ["rising", "falling"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_running_max_moves(direction, dtype):
    """Key norms ramp along the token order, so the row max moves across key
    tiles.  Rising: the max has to be raised on most tiles; falling: only on
    the first.  Several 64-key tiles and a ragged tail per subsequence.
    bf16 ramps to 40x: scores reach ~190 in log2 units, so an exp2 taken
    against a stale max would overflow fp32.  f32 ramps to 8x: at 40x, fp32
    rounding of the 128-term dot products alone moves the output by ~1.7e-5
    (plain float32 numpy attention does the same), beyond the 1e-5 bar that
    holds for N(0,1) inputs."""
    shp = (1, 3, 16, 42, 2, 128)
    kf, mode = 2, 0
    q, k, v = (wl.normal_tensor(shp, 17, i) for i in range(3))
    N = shp[1] * shp[2] * shp[3]
    top = 40.0 if dtype == "bf16" else 8.0
    ramp = np.linspace(1.0, top, N) if direction == "rising" else np.linspace(top, 1.0, N)
    k = k * ramp.reshape(1, shp[1], shp[2], shp[3], 1, 1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(tdt) for x in (q, k, v))
    o = run(q, k, v, kf, mode)
    r = ref.skiparse_attention(to_np64(q), to_np64(k), to_np64(v), kf, mode)
    assert err_ratio(to_np64(o), r) <= TOL[dtype]


def test_bf16_writes_exactly_the_real_rows_of_run_subsequences():
    """NaN-prefilled output: a call over subsequences [1, 3) writes every row of
    those subsequences and no other row."""
    shp = (1, 2, 11, 14, 2, 128)
    kf, mode = 2, 1
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 5, i)).to(torch.bfloat16).to(DEV) for i in range(3))
    o = torch.full(shp, float("nan"), dtype=torch.bfloat16, device=DEV)
    plan = sk.skiparse_plan_init(*shp, kf, mode)
    sk.skiparse_attn_fwd(plan, sk.BF16, q, k, v, o, sub_begin=1, sub_count=2)
    torch.cuda.synchronize()
    written = torch.isfinite(o.float()).all(dim=-1).cpu().numpy().reshape(shp[0], -1, shp[4])
    members = ref.subsequence_members(shp[1], shp[2], shp[3], kf, mode)
    expect = np.zeros(written.shape[1], bool)
    for s in (1, 2):
        expect[members[s]] = True
    for b in range(shp[0]):
        for h in range(shp[4]):
            np.testing.assert_array_equal(written[b, :, h], expect)


def test_bf16_deterministic():
    shp = (1, 3, 13, 22, 2, 128)
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 6, i)).to(torch.bfloat16).to(DEV) for i in range(3))
    a = sk.attention(q, k, v, 2, 0)
    b = sk.attention(q, k, v, 2, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def device_normal(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return [torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16) for _ in range(3)]


def test_bf16_repeatable_at_720p():
    """Three calls on the same 720P-5s inputs are bit-identical.  Each
    subsequence streams 302 key tiles, so a scheduling or synchronisation
    defect that shows only on long loops would change the output between
    calls; the small-shape check above covers four tiles."""
    shape = wl.WORKLOADS["720p_5s"].shape
    q, k, v = device_normal(shape, 1001)
    outs = [sk.attention(q, k, v, 2, mode) for mode in (sk.MODE_TOKEN, sk.MODE_GROUP) for _ in range(3)]
    torch.cuda.synchronize()
    for i in (0, 3):
        assert torch.equal(outs[i], outs[i + 1]) and torch.equal(outs[i], outs[i + 2])


# ---------------------------------------------------------------------------
# bf16 at the workload shapes: sampled rows
# ---------------------------------------------------------------------------

def sample_tokens(T, H, W, kf, mode, rng, per_sub=48):
    """Per subsequence: first and last member, members on the padding edge
    (last real row/column), and random members."""
    members = ref.subsequence_members(T, H, W, kf, mode)
    picks = []
    for mem in members:
        if mem.size == 0:
            continue
        hw = mem % (H * W)
        h, w = hw // W, hw % W
        edge = mem[(h == H - 1) | (w == W - 1)]
        sel = [mem[0], mem[-1]]
        if edge.size:
            sel += list(rng.choice(edge, size=min(8, edge.size), replace=False))
        sel += list(rng.choice(mem, size=min(per_sub, mem.size), replace=False))
        picks.append(np.unique(np.array(sel, np.int64)))
    return np.concatenate(picks)


_INPUT_CACHE = {}


def workload_inputs(name):
    if name not in _INPUT_CACHE:
        _INPUT_CACHE.clear()
        w = wl.WORKLOADS[name]
        cpu = wl.make_inputs(w)
        _INPUT_CACHE[name] = (w, cpu, tuple(t.to(DEV) for t in cpu))
    return _INPUT_CACHE[name]


def check_sampled(w, cpu, out, kf, mode, heads, seed, tol):
    B, T, H, W, nh, d = w.shape
    N = T * H * W
    qn, kn, vn = (t.float().numpy().reshape(B, N, nh, d) for t in cpu)
    on = out.float().cpu().numpy().reshape(B, N, nh, d)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for b in range(B):
        for h in heads:
            toks = sample_tokens(T, H, W, kf, mode, rng)
            r = ref.attention_rows(qn, kn, vn, T, H, W, kf, mode, b, h, toks)
            worst = max(worst, err_ratio(on[b, toks, h], r))
    assert worst <= tol, worst
    return worst


@pytest.mark.parametrize("name,kf,mode", [
    ("480p", 2, 0), ("480p", 2, 1), ("480p", 1, 0),
    ("720p_5s", 2, 0), ("720p_5s", 2, 1), ("720p_5s", 1, 0),
    ("768p_5s", 2, 0), ("768p_5s", 2, 1),
])
def test_bf16_workload_sampled(name, kf, mode):
    w, cpu, dev = workload_inputs(name)
    out = sk.attention(*dev, kf, mode)
    torch.cuda.synchronize()
    heads = [0, w.heads // 2, w.heads - 1]
    worst = check_sampled(w, cpu, out, kf, mode, heads, seed=kf * 10 + mode, tol=TOL["bf16"])
    print(f"\n[sampled parity] {name} k={kf} mode={mode} bf16: max err {worst:.3e} of max(1, max|O|)")


@pytest.mark.parametrize("shp,kf,mode", [
    ((1, 1, 48, 2200, 1, 64), 2, 0),   # n = 26400 over the token-table cap, 1100 local columns: index function per row
    ((1, 2, 120, 440, 1, 64), 2, 0),   # n = 26400 over the cap, row/column tables fit: table walker
    ((1, 1, 8, 2200, 1, 64), 2, 1),    # n = 4400 with 1100 local columns: token table
    ((1, 2, 60, 220, 1, 64), 1, 0),    # k = 1, n = 26400: the member index is the token
])
def test_bf16_row_sources(shp, kf, mode):
    """The kernel finds a key row's token in one of four ways, chosen by k and
    the subsequence sizes; each is checked on sampled rows."""
    q, k, v = (torch.from_numpy(wl.normal_tensor(shp, 23, i)).to(torch.bfloat16) for i in range(3))
    out = run(q, k, v, kf, mode)
    check_sampled(types.SimpleNamespace(shape=shp), (q, k, v), out, kf, mode, [0], seed=3, tol=TOL["bf16"])


# ---------------------------------------------------------------------------
# per-tensor fp8 quantization: bytes and scale bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("numel,dtype,outl", [(1000, torch.bfloat16, False), (4099, torch.float32, True),
                                              (3 * 2**20 + 5, torch.bfloat16, True), (8, torch.bfloat16, False)])
def test_quant_fp8_bit_exact(numel, dtype, outl):
    x = torch.from_numpy(wl.normal_tensor((1, 1, 1, 1, 1, numel), 3, 0)).to(dtype)
    if outl:
        x[..., 7] = 37.5
    y, sc = sk.quantize_fp8(x.to(DEV))
    torch.cuda.synchronize()
    codes, scale, amax = f8.quantize_per_tensor(x.float().numpy().reshape(-1))
    assert sc[0].item() == float(scale)
    assert sc[1].item() == float(np.float32(np.float32(1.0) / scale))
    np.testing.assert_array_equal(y.cpu().numpy().reshape(-1), codes)
