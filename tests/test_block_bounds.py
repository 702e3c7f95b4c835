"""Host-side bounds of every launch the fp8 block makes (CPU only).

skiparse_block_fwd_fp8 runs 19 kernels on regions of one caller workspace.
For a plan, this test derives, from each launch's arguments and the index
bounds of its kernel, the byte range each launch can read or write in each
region, and checks that every range stays inside its own region and that the
regions are disjoint.  It runs at the 720P-5s shape with all 40 heads
(C = 5120), the shape at which the block's first version (projections on
hipBLASLt) faulted the GPU, and at smaller shapes.

The workspace layout and the launch grids are restated here from the library's
host code; they are pinned to the library itself through the sizes it
exports (skiparse_block_workspace_bytes, skiparse_quant_fp8_workspace_bytes,
skiparse_rope_fp8_workspace_bytes), which are built from the same quantities.

Kernel index bounds used (each read off the kernel source):
- amax / quantize (quant_fp8.hip): 16-byte vectors i < numel / vec, a scalar
  tail below numel, one partial per work-group, grid = blocks_for(numel);
- scale: partials [0, nb), writes {scale, 1/scale};
- GEMM (gemm_fp8.hip): the XCD-major tile remap is a bijection of [0, total)
  (checked exhaustively below); W rows n0 + lrow + 64 s < n0 + 256 <= N;
  X rows clamped to M - 1; Y stores masked to m < M and n < N; K steps of
  128 bytes below K;
- rotary table: entries i < tab_len; rotary amax / encode: 16-byte vectors
  i < nvec, one partial per work-group, grid = rope_blocks(nvec);
- e4m3 attention: rows of tokens < T*H*W at offset tok * heads * d + head * d
  (+ 128 bytes of codes, or 256 bytes of bf16 output);
- every grid-stride index is below 2^31 + grid size, inside 32 bits.
"""

import ctypes

import pytest

import fixed_pattern_sparse_amd as sk

R256 = lambda n: (n + 255) & ~255


def blocks_for(numel):
    return max(1, min(2048, (numel + 16383) // 16384))


def rope_blocks(nvec):
    return max(1, min(2048, (nvec + 2047) // 2048))


def layout(B, T, H, W, heads, d):
    mc = B * T * H * W * heads * d
    nvec = mc // 8
    part = max(blocks_for(mc) * 4, rope_blocks(nvec) * 4)
    L, at = {}, 0
    for name, size in [("x8", R256(mc)), ("qkv16", R256(3 * mc * 2)), ("qkv8", R256(3 * mc)), ("scales", 256),
                       ("part", R256(part)), ("tab", R256((T + H + W) * (d // 2) * 8))]:
        L[name] = (at, size)
        at += size
    return L, at


SHAPES = [(1, 21, 45, 80, 40, 128), (1, 21, 32, 52, 12, 128), (1, 21, 45, 80, 12, 128), (2, 3, 5, 7, 2, 128),
          (1, 1, 1, 1, 1, 128), (2, 21, 48, 80, 40, 128)]


@pytest.mark.parametrize("shape", SHAPES)
def test_layout_and_grids_match_the_library(shape):
    B, T, H, W, heads, d = shape
    plan = sk.skiparse_plan_init(B, T, H, W, heads, d, 2, 0)
    _, total = layout(*shape)
    assert sk.skiparse_block_workspace_bytes(plan) == total
    mc = B * T * H * W * heads * d
    assert sk.skiparse_quant_fp8_workspace_bytes(mc) == blocks_for(mc) * 4
    assert sk.skiparse_rope_fp8_workspace_bytes(plan) == R256((T + H + W) * (d // 2) * 8) + R256(rope_blocks(mc // 8) * 4)


def gemm_tile_ranges(M, N, K):
    """(x bytes, w bytes, y bytes) the 256 x 256 GEMM can touch, from its tile
    decode and loader/store bounds."""
    TN = TM = 256
    tiles_n = N // TN
    total = (M + TM - 1) // TM * tiles_n
    q, r = divmod(total, 8)
    seen = bytearray(total)
    x_hi = w_hi = y_hi = 0
    for bid in range(total):
        c = bid % 8
        tile = c * q + min(c, r) + bid // 8
        assert 0 <= tile < total
        seen[tile] += 1
        n0, m0 = (tile % tiles_n) * TN, (tile // tiles_n) * TM
        w_hi = max(w_hi, (n0 + 7 + 64 * 3 + 24) * K + 7 * 16 + 16)   # lrow < 32 per pass, 4 passes of 64 rows
        xr = min(m0 + 31 + 64 * 3 + 32, M - 1)                         # clamped row
        x_hi = max(x_hi, xr * K + 7 * 16 + 16)
        m_last = min(m0 + TM, M) - 1
        y_hi = max(y_hi, (m_last * N + n0 + TN) * 2)
    assert all(s == 1 for s in seen), "tile remap is not a bijection"
    # the row bound above: lrow = tid >> 3 < 64 for 512 threads, passes s < 4 of kRP = 64 rows
    assert x_hi <= M * K and w_hi <= N * K and y_hi <= M * N * 2
    return x_hi, w_hi, y_hi


@pytest.mark.parametrize("shape", SHAPES)
def test_every_launch_stays_in_its_region(shape):
    B, T, H, W, heads, d = shape
    C, M = heads * d, B * T * H * W
    mc = M * C
    L, total = layout(*shape)
    regions = sorted(L.values())
    for (a0, s0), (a1, _) in zip(regions, regions[1:]):
        assert a0 + s0 <= a1, "regions overlap"
    assert regions[-1][0] + regions[-1][1] == total

    launches = []   # (what, region, lo, hi) byte ranges relative to the region
    nb = blocks_for(mc)
    # q8(x): x (caller) -> x8, partials, scale of x
    launches += [("amax x", "part", 0, nb * 4), ("scale x", "scales", 0, 8), ("quant x", "x8", 0, mc)]
    # three projections: x8 . W^T -> bf16 Q, K, V
    if C % 256 == 0:
        x_hi, w_hi, y_hi = gemm_tile_ranges(M, C, C)
    else:
        x_hi, w_hi, y_hi = mc, C * C, mc * 2
    for i in range(3):
        launches += [(f"gemm {i} reads x8", "x8", 0, x_hi), (f"gemm {i} writes", "qkv16", i * mc * 2, i * mc * 2 + y_hi)]
    tab_len = (T + H + W) * (d // 2)
    launches.append(("rope table", "tab", 0, tab_len * 8))
    nvec = mc // 8
    assert nvec < 2 ** 31 and nvec + 2048 * 256 < 2 ** 32
    rb = rope_blocks(nvec)
    for i in range(2):
        launches += [(f"rope amax {i}", "qkv16", i * mc * 2, i * mc * 2 + nvec * 16), (f"rope part {i}", "part", 0, rb * 4),
                     (f"rope scale {i}", "scales", 8 + 8 * i, 16 + 8 * i),
                     (f"rope encode {i}", "qkv8", i * mc, i * mc + nvec * 8)]
    launches += [("amax V", "qkv16", 2 * mc * 2, 3 * mc * 2), ("part V", "part", 0, nb * 4),
                 ("scale V", "scales", 24, 32), ("quant V", "qkv8", 2 * mc, 3 * mc)]
    # attention: codes rows of tokens < T*H*W (per batch sample), O bf16 over the Q projection
    row_last = (B * T * H * W - 1) * C + (heads - 1) * d
    for i in range(3):
        launches.append((f"attn reads {i}", "qkv8", i * mc, i * mc + row_last + d))
    launches += [("attn descale", "scales", 8, 32), ("attn writes O", "qkv16", 0, (row_last + d) * 2)]
    launches += [("amax O", "qkv16", 0, mc * 2), ("part O", "part", 0, nb * 4), ("scale O", "scales", 32, 40),
                 ("quant O", "x8", 0, mc), ("gemm out reads", "x8", 0, x_hi)]
    for what, reg, lo, hi in launches:
        start, size = L[reg]
        assert 0 <= lo < hi <= size, (what, reg, lo, hi, size)
    # 32-bit row offsets of the attention kernels' fast paths
    assert T * H * W < 2 ** 24 and C < 2 ** 24 and T * H * W * C < 2 ** 32
    # the block at 720P-5s with 40 heads: about 3.9 GB of workspace
    if shape == (1, 21, 45, 80, 40, 128):
        assert 3.8e9 < total < 4.0e9
