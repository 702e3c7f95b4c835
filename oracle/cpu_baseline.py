"""CPU baseline: the oracle's algorithm in fp32 numpy/BLAS, for timing only
(test infrastructure; not a fallback for anything).

Per (batch, head, subsequence) unit: gather the unit's real rows with the
closed-form map from :mod:`oracle.skiparse_ref`, then for each block of 1024
queries compute S = scale * Q K^T (sgemm), a max-subtracted softmax, O = P V
(sgemm), and scatter the rows back.  Nothing is tuned; BLAS uses whatever host
threads it is given.
"""

from __future__ import annotations

import os
import time

import numpy as np

from . import skiparse_ref as ref


def blas_threads() -> int:
    """Threads the BLAS behind numpy will use (best effort)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def run_units(q, k, v, T, H, W, kf, mode, units, out=None, scale=None, block=1024):
    """Run the listed units (b, head, s) in fp32.  q/k/v: float32 arrays shaped
    (B, N, heads, d).  Returns (out, computed pairs)."""
    B, N, nh, d = q.shape
    scale = np.float32(ref.default_scale(d) if scale is None else scale)
    members = ref.subsequence_members(T, H, W, kf, mode)
    if out is None:
        out = np.zeros_like(q)
    pairs = 0
    for (b, h, s) in units:
        mem = members[s]
        n = mem.size
        if n == 0:
            continue
        ks = np.ascontiguousarray(k[b, mem, h])
        vs = np.ascontiguousarray(v[b, mem, h])
        qs = np.ascontiguousarray(q[b, mem, h])
        for i0 in range(0, n, block):
            sc = (qs[i0:i0 + block] @ ks.T) * scale
            sc -= sc.max(axis=1, keepdims=True)
            np.exp(sc, out=sc)
            sc /= sc.sum(axis=1, keepdims=True)
            out[b, mem[i0:i0 + block], h] = sc @ vs
        pairs += n * n
    return out, pairs


def time_sample(q, k, v, T, H, W, kf, mode, units, repeats=1):
    """Seconds to run ``units`` once (best of ``repeats``) and their pair count."""
    best = float("inf")
    pairs = 0
    for _ in range(max(1, repeats)):
        t0 = time.perf_counter()
        _, pairs = run_units(q, k, v, T, H, W, kf, mode, units)
        best = min(best, time.perf_counter() - t0)
    return best, pairs
