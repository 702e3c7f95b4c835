"""The matrix-core kernels fit their register budgets: each source is compiled
for gfx950 with the library's own flags, and no kernel of the attention
forwards, the backward passes or the projection GEMM may use scratch memory
(a spill would leave every parity test green while costing the kernel much of
its speed).  Host-only: hipcc cross-compiles without a GPU."""

import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fixed_pattern_sparse_amd import build as b

SOURCES = ["attn_bf16.hip", "attn_fp8.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "gemm_fp8.hip"]


def kernel_resources(src):
    cmd = [b.hipcc(), *b.FLAGS, *b.SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           f"{b.CSRC}/{src}", "-o", "-"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = r.stdout
    out = {}
    # one kernel descriptor per kernel: its private segment and VGPR count
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, re.S):
        blk = m.group(2)
        priv = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", blk).group(1))
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", blk).group(1))
        out[m.group(1)] = (vgpr, priv)
    assert len(out) == asm.count(".amdhsa_kernel "), "a kernel descriptor was not parsed"
    return out


@pytest.fixture(scope="module")
def resources():
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(kernel_resources, SOURCES)))


@pytest.mark.parametrize("src", SOURCES)
def test_kernels_use_no_scratch(resources, src):
    kernels = resources[src]
    assert kernels, f"no kernel metadata found for {src}"
    spilled = {k: v for k, v in kernels.items() if v[1] != 0}
    assert not spilled, f"kernels with scratch (vgprs, bytes): {spilled}"
    for name, (vgpr, _) in kernels.items():
        assert vgpr <= 512, (name, vgpr)
