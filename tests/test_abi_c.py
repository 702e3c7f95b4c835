"""The C ABI from a plain C program (tests/c_caller.c, built next to the
library by the package build): the host plan and gather map against the
oracle, bit-exact, and error reporting (CPU); the bf16 forward, and the
per-tensor e4m3 quantization followed by the e4m3 forward, on the device from
C against the oracle (GPU)."""

import os
import subprocess

import numpy as np
import pytest

from oracle import skiparse_ref as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER = os.path.join(ROOT, "fixed_pattern_sparse_amd", "c_caller")


def caller(*args):
    if not os.path.exists(CALLER):
        pytest.fail(f"{CALLER} is missing: build the package first (python -m fixed_pattern_sparse_amd.build)")
    r = subprocess.run([CALLER, *map(str, args)], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout.splitlines()


@pytest.mark.parametrize("T,H,W,k,mode", [(2, 6, 10, 2, ref.GROUP), (1, 5, 7, 2, ref.TOKEN), (3, 9, 17, 3, ref.GROUP),
                                          (1, 4, 5, 2, ref.TOKEN_1D), (2, 3, 3, 1, ref.TOKEN)])
def test_c_plan_and_map(T, H, W, k, mode):
    out = caller("plan", 1, T, H, W, 2, 64, k, mode)
    plan = out[0].split()
    assert plan[0] == "plan"
    Hp, Wp, sub_h, sub_w, n_sub, sub_len, pairs = (int(x) for x in plan[1:])
    want = ref.gather_map(T, H, W, k, mode)
    assert (n_sub, sub_len) == want.shape
    got = np.array([int(x) for x in out[1].split()[1:]], np.int32).reshape(n_sub, sub_len)
    np.testing.assert_array_equal(got, want)
    n = (want >= 0).sum(axis=1).astype(np.int64)
    assert pairs == int((n * n).sum()) * 2          # two heads
    assert out[2] == f"bad {-1} message"


def hash_inputs(shape, t):
    i = np.arange(int(np.prod(shape)), dtype=np.uint64)
    h = ((i * np.uint64(2654435761) + np.uint64(t) * np.uint64(40503)) & np.uint64(0xFFFFFFFF)) >> np.uint64(8)
    return (h.astype(np.float64) / 16777216.0 - 0.5).astype(np.float32).reshape(shape)


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
def test_c_attention_on_device(mode, tmp_path):
    import torch
    shp = (1, 2, 6, 10, 2, 128)
    out_path = tmp_path / "o.bin"
    lines = caller("attn", *shp, 2, mode, out_path)
    assert lines[-1].startswith("attn ok")
    got = torch.from_numpy(np.fromfile(out_path, dtype=np.uint16).astype(np.int16)).view(torch.bfloat16)
    got = got.float().numpy().astype(np.float64).reshape(shp)
    q, k, v = (torch.from_numpy(hash_inputs(shp, t)).to(torch.bfloat16).float().numpy().astype(np.float64)
               for t in range(3))
    want = ref.skiparse_attention(q, k, v, 2, mode)
    assert np.max(np.abs(got - want)) <= 2e-2 * max(1.0, np.max(np.abs(want)))


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [ref.TOKEN, ref.GROUP])
def test_c_fp8_attention_on_device(mode, tmp_path):
    import torch
    from oracle import fp8_ref as f8
    shp = (1, 2, 6, 10, 2, 128)
    out_path = tmp_path / "o8.bin"
    lines = caller("attn8", *shp, 2, mode, out_path)
    assert lines[-1].startswith("attn ok")
    got = torch.from_numpy(np.fromfile(out_path, dtype=np.uint16).astype(np.int16)).view(torch.bfloat16)
    got = got.float().numpy().astype(np.float64).reshape(shp)
    deq = []
    for t in range(3):
        x = torch.from_numpy(hash_inputs(shp, t)).to(torch.bfloat16).float().numpy()
        codes, scale, _ = f8.quantize_per_tensor(x.reshape(-1))
        deq.append(f8.dequantize(codes, scale).reshape(shp))
    want = ref.skiparse_attention(*deq, 2, mode)
    assert np.max(np.abs(got - want)) <= 6e-2 * max(1.0, np.max(np.abs(want)))
