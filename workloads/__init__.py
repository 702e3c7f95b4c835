"""Seeded synthetic inputs and named workload shapes.

This module only draws random numbers and names shapes: it holds none of the
attention arithmetic, so the HIP path's tests and the oracle can both take
their inputs from it.

Recipe (one per tensor, reproducible on any host):
* numpy ``Generator(PCG64)``; tensor ``i`` of a workload with seed ``S`` is cut
  into chunks of 2**22 elements and chunk ``c`` is drawn from
  ``SeedSequence(S, spawn_key=(i, c))`` as float32 standard normals (chunks run
  on a thread pool; the values do not depend on the thread count);
* optional outlier channels: round(0.05 * heads * d) distinct channel indices
  of the flattened (heads, d) axis, drawn from ``SeedSequence(S,
  spawn_key=(100 + i,))``, are multiplied by 8 for every token;
* the float32 values are rounded to bfloat16 (round to nearest even) for bf16
  and fp8 workloads, and kept as float32 for fp32 workloads.

Tensor ids: 0 = Q, 1 = K, 2 = V.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TOKEN = 0
GROUP = 1

_CHUNK = 1 << 22


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    W: int
    heads: int
    d: int
    k: int
    dtype: str          # "f32", "bf16" or "fp8" (fp8: bf16 inputs quantized per tensor)
    seed: int
    outliers: bool
    note: str = ""

    @property
    def shape(self):
        return (self.B, self.T, self.H, self.W, self.heads, self.d)

    @property
    def numel(self):
        return self.B * self.T * self.H * self.W * self.heads * self.d

    def with_(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 8, 8, 2, 64, 2, "f32", 1001, False,
                     "128 tokens, token-wise then group-wise layer"),
    "480p": Workload("480p", 1, 21, 32, 52, 12, 128, 2, "bf16", 1002, False,
                     "480P-like latent, no padding"),
    "720p_5s": Workload("720p_5s", 1, 21, 45, 80, 40, 128, 2, "bf16", 1003, True,
                        "720P 5 s latent, H padded 45->48, 5% outlier channels x8"),
    "768p_5s": Workload("768p_5s", 2, 21, 48, 80, 40, 128, 2, "bf16", 1004, False,
                        "768P 5 s latent, cond/uncond pair, no padding"),
    "720p_5s_fp8": Workload("720p_5s_fp8", 1, 21, 45, 80, 40, 128, 2, "fp8", 1005, True,
                            "720P 5 s shape quantized per tensor to e4m3; also k=4"),
}


def _fill(out: np.ndarray, seed: int, tensor_id: int, workers: int):
    flat = out.reshape(-1)
    n = flat.size
    chunks = [(c, c * _CHUNK, min(n, (c + 1) * _CHUNK)) for c in range((n + _CHUNK - 1) // _CHUNK)]

    def work(item):
        c, a, b = item
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, c))))
        rng.standard_normal(out=flat[a:b], dtype=np.float32)

    if len(chunks) <= 1 or workers <= 1:
        for it in chunks:
            work(it)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(work, chunks))


def outlier_channels(seed: int, tensor_id: int, heads: int, d: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(100 + tensor_id,))))
    count = int(round(0.05 * heads * d))
    return np.sort(rng.choice(heads * d, size=count, replace=False))


def normal_tensor(shape, seed: int, tensor_id: int, outliers: bool = False,
                  workers: int | None = None) -> np.ndarray:
    """float32 array of the given (B, T, H, W, heads, d) shape."""
    workers = workers or min(16, os.cpu_count() or 1)
    x = np.empty(shape, np.float32)
    _fill(x, seed, tensor_id, workers)
    if outliers:
        heads, d = shape[-2], shape[-1]
        ch = outlier_channels(seed, tensor_id, heads, d)
        xv = x.reshape(-1, heads * d)
        xv[:, ch] *= np.float32(8.0)
    return x


def make_inputs(w: Workload, workers: int | None = None):
    """Q, K, V as torch CPU tensors: float32 for "f32" workloads, bfloat16
    (RNE-rounded) otherwise."""
    import torch
    out = []
    for tid in range(3):
        x = normal_tensor(w.shape, w.seed, tid, w.outliers, workers)
        t = torch.from_numpy(x)
        if w.dtype != "f32":
            t = t.to(torch.bfloat16)
        out.append(t)
        del x
    return tuple(out)


# ---------------------------------------------------------------------------
# Counter-based values for tensors too large to draw on the host: element i of
# tensor t is ((i * 2654435761 + t * 40503) mod 2^32 >> 8) / 2^24 - 0.5, times
# a power-of-two gain, computed in fp32 (exact) and rounded to bf16 (nearest
# even).  Both generators below follow this definition, one in numpy for any
# set of indices, one with torch integer ops on the device for a whole tensor.
# ---------------------------------------------------------------------------

HASH_MUL = 2654435761
HASH_TENSOR = 40503


def hash_values(tensor_id: int, idx, gain: float = 1.0) -> np.ndarray:
    """float32 values (already on the bf16 grid) of the elements at flat
    indices ``idx`` (any integer array)."""
    import torch
    i = np.asarray(idx, np.uint64)
    h = (i * np.uint64(HASH_MUL) + np.uint64(tensor_id * HASH_TENSOR)) & np.uint64(0xFFFFFFFF)
    v = (h >> np.uint64(8)).astype(np.float32) / np.float32(16777216.0) - np.float32(0.5)
    v = v * np.float32(gain)
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).float().numpy()


def hash_fill_(t, tensor_id: int, gain: float = 1.0, chunk: int = 1 << 27):
    """Fill the bf16 device tensor ``t`` (contiguous) with the values of
    :func:`hash_values` for its flat indices, in chunks."""
    import torch
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        i = torch.arange(s, e, dtype=torch.int64, device=t.device)
        h = (i * HASH_MUL + tensor_id * HASH_TENSOR) & 0xFFFFFFFF
        v = (h >> 8).to(torch.float32) / 16777216.0 - 0.5
        flat[s:e] = (v * gain).to(torch.bfloat16)
    return t
