"""Gradients of Skiparse-2D attention, written out plainly in float64 (test
infrastructure only).

The sparse model is fine-tuned and trained in 8 bits with this attention in
its layers (OSP-Next summary, 方法步骤详情 method steps: a separate quantization
maximum is set for backpropagation; 技术新颖性 novelty: joint 8-bit training
with the sparse model; 复现评估 reproduction: the fine-tuning configuration),
so the layer needs dQ, dK and dV for an upstream gradient dO.  The pages give
no formula for them: they are the derivative of the forward pass, i.e. of
dense softmax attention inside each subsequence (forward: see
``oracle.skiparse_ref``).  With S = scale * Q K^T, P = softmax(S) by rows and
O = P V, the chain rule gives, inside one subsequence,

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))        (the softmax Jacobian applied by rows)
    dQ = scale * dS K
    dK = scale * dS^T Q

Padded tokens are not keys, so they receive no gradient; padded queries are
discarded by the forward pass, so their upstream gradient never reaches
anything.  The log-sum-exp of a query row (natural log),
LSE_i = log sum_j exp(S_ij), is what a training forward pass keeps so that the
backward pass can form P without a second softmax.
"""

from __future__ import annotations

import numpy as np

from .skiparse_ref import TOKEN, _members_for, default_scale, from_subsequences, subsequence_real_mask, to_subsequences


def softmax_attention_bwd(q, k, v, do, scale, key_ok=None, o=None):
    """Gradients (dq, dk, dv) of O = softmax(scale * q k^T) v for upstream dO,
    in float64, the keys where ``key_ok`` is False excluded (they get zero
    gradient).  q, do: (Lq, d); k, v: (Lk, d).  With ``o`` given (Lq, d), the
    row term of dS is formed from it as rowsum(dO * o), the form a backward
    pass that receives the forward's output uses (equal to rowsum(P * dP)
    when o is the exact output); otherwise from the softmax Jacobian."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    s = (q @ k.T) * scale
    if key_ok is not None:
        s = np.where(key_ok[None, :], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    rowterm = (p * dp).sum(axis=1, keepdims=True) if o is None else (do * np.asarray(o, np.float64)).sum(axis=1, keepdims=True)
    ds = p * (dp - rowterm)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def skiparse_attention_bwd(q, k, v, do, kf: int, mode: int, scale=None, o=None):
    """(dq, dk, dv) of Skiparse-2D attention, all (B, T, H, W, heads, d), by the
    same steps as the forward oracle: pad -> rearrange -> per-subsequence
    gradients -> rearrange back -> crop.  ``o``: optional forward output of the
    same layout, as in :func:`softmax_attention_bwd`."""
    q = np.asarray(q, np.float64)
    B, T, H, W, nh, d = q.shape
    mode = TOKEN if kf == 1 else mode
    scale = default_scale(d) if scale is None else scale
    qs, ks, vs, dos = (to_subsequences(np.asarray(x, np.float64), kf, mode) for x in (q, k, v, do))
    os_ = None if o is None else to_subsequences(np.asarray(o, np.float64), kf, mode)
    ok = subsequence_real_mask(T, H, W, kf, mode)
    grads = [np.zeros_like(qs) for _ in range(3)]
    for b in range(B):
        for s in range(qs.shape[1]):
            real = ok[s]
            if not real.any():
                continue
            for h in range(nh):
                # only real queries exist; their gradients reach real keys only
                dq, dk, dv = softmax_attention_bwd(qs[b, s, h][real], ks[b, s, h][real], vs[b, s, h][real],
                                                   dos[b, s, h][real], scale,
                                                   o=None if os_ is None else os_[b, s, h][real])
                grads[0][b, s, h][real] = dq
                grads[1][b, s, h][real] = dk
                grads[2][b, s, h][real] = dv
    return tuple(from_subsequences(g, T, H, W, kf, mode) for g in grads)


def attention_lse(q, k, kf: int, mode: int, scale=None):
    """(B, T*H*W, heads) natural-log softmax denominators LSE_i = log sum_j
    exp(scale q_i . k_j) over the keys of each real query's subsequence."""
    q = np.asarray(q, np.float64)
    B, T, H, W, nh, d = q.shape
    N = T * H * W
    scale = default_scale(d) if scale is None else scale
    members, _ = _members_for((T, H, W, kf, TOKEN if kf == 1 else mode))
    qf = q.reshape(B, N, nh, d)
    kf_ = np.asarray(k, np.float64).reshape(B, N, nh, d)
    out = np.zeros((B, N, nh), np.float64)
    for b in range(B):
        for mem in members:
            if mem.size == 0:
                continue
            for h in range(nh):
                s = (qf[b, mem, h] @ kf_[b, mem, h].T) * scale
                m = s.max(axis=1)
                out[b, mem, h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


# ---------------------------------------------------------------------------
# 8-bit training
# ---------------------------------------------------------------------------

def quantized_inputs(q, k, v, do=None, fp8_max=448.0, fp8_max_grad=448.0, eps=1e-12):
    """The per-tensor 8-bit tensors of the training path (OSP-Next summary,
    方法步骤详情 method steps: every tensor quantized as a whole with
    scale = FP8max / (Amax + eps), the backward pass with its own maximum), by
    the oracle's own codec (oracle.fp8_ref).  Returns a dict with the codes,
    the fp32 scales and the dequantized float64 tensors code / scale, for Q, K,
    V (maximum fp8_max) and, if given, dO (maximum fp8_max_grad)."""
    from . import fp8_ref as f8
    out = {}
    named = [("q", q, fp8_max), ("k", k, fp8_max), ("v", v, fp8_max)]
    if do is not None:
        named.append(("do", do, fp8_max_grad))
    for name, x, mx in named:
        codes, scale, _ = f8.quantize_per_tensor(np.asarray(x, np.float32).ravel(), mx, eps)
        out[name + "8"] = codes.reshape(np.shape(x))
        out["s_" + name] = scale
        out[name] = f8.dequantize(codes, scale).reshape(np.shape(x))
    return out


def dequantized_part(part, amax, fp8_max=448.0, eps=1e-12):
    """Dequantized float64 values of a part of a tensor that is quantized as a
    whole: the scale comes from the whole tensor's amax (fp32), the codes from
    the part's own elements (per-element, so any part can be formed alone)."""
    from . import fp8_ref as f8
    scale = f8.per_tensor_scale(np.float32(amax), fp8_max, eps)
    codes = f8.e4m3_encode((np.asarray(part, np.float32) * scale).astype(np.float32))
    return f8.dequantize(codes, scale)


def skiparse_attention_bwd_fp8(q, k, v, do, kf: int, mode: int, scale=None, fp8_max=448.0, fp8_max_grad=448.0,
                               eps=1e-12, o=None):
    """Gradients of the 8-bit training path: Q, K, V and dO are quantized per
    tensor (:func:`quantized_inputs`) and the layer's gradients are those of
    the dequantized tensors, :func:`skiparse_attention_bwd` applied to them
    (``o`` passed through).  Returns (dq, dk, dv, the quantized-input dict)."""
    t = quantized_inputs(q, k, v, do, fp8_max, fp8_max_grad, eps)
    return (*skiparse_attention_bwd(t["q"], t["k"], t["v"], t["do"], kf, mode, scale, o=o), t)


# ---------------------------------------------------------------------------
# Sampled rows for full-size shapes
# ---------------------------------------------------------------------------

def _rows64(x, b, idx, h):
    return np.asarray(x[b, idx, h], np.float64)


def dq_rows(q, k, v, do, T, H, W, kf, mode, b, head, tokens, scale=None):
    """dQ[b, token, head, :] for real flat tokens, each row computed on its own
    from all keys of its subsequence.  Arrays are indexable as (B, N, heads, d)."""
    B, N, nh, d = q.shape
    scale = default_scale(d) if scale is None else scale
    members, sub_of = _members_for((T, H, W, kf, TOKEN if kf == 1 else mode))
    tokens = np.asarray(tokens, np.int64)
    out = np.zeros((tokens.size, d), np.float64)
    for s in np.unique(sub_of[tokens]):
        sel = np.nonzero(sub_of[tokens] == s)[0]
        mem = members[s]
        kk, vv = _rows64(k, b, mem, head), _rows64(v, b, mem, head)
        qq, dd = _rows64(q, b, tokens[sel], head), _rows64(do, b, tokens[sel], head)
        sc = (qq @ kk.T) * scale
        sc -= sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p /= p.sum(axis=1, keepdims=True)
        dp = dd @ vv.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        out[sel] = scale * (ds @ kk)
    return out


def dkv_rows(q, k, v, do, T, H, W, kf, mode, b, head, tokens, scale=None, chunk=2048):
    """(dK, dV)[b, token, head, :] for real flat key tokens.  A key's gradient
    sums over every query of its subsequence, so each touched subsequence's
    query rows are formed in chunks (their softmax over all keys, then the
    columns of the sampled keys)."""
    B, N, nh, d = q.shape
    scale = default_scale(d) if scale is None else scale
    members, sub_of = _members_for((T, H, W, kf, TOKEN if kf == 1 else mode))
    tokens = np.asarray(tokens, np.int64)
    dk = np.zeros((tokens.size, d), np.float64)
    dv = np.zeros((tokens.size, d), np.float64)
    for s in np.unique(sub_of[tokens]):
        sel = np.nonzero(sub_of[tokens] == s)[0]
        mem = members[s]
        kk, vv = _rows64(k, b, mem, head), _rows64(v, b, mem, head)
        ksel, vsel = _rows64(k, b, tokens[sel], head), _rows64(v, b, tokens[sel], head)
        for c0 in range(0, mem.size, chunk):
            rows = mem[c0:c0 + chunk]
            qq, dd = _rows64(q, b, rows, head), _rows64(do, b, rows, head)
            sc = (qq @ kk.T) * scale
            m = sc.max(axis=1, keepdims=True)
            z = np.exp(sc - m).sum(axis=1, keepdims=True)
            p_all = np.exp(sc - m) / z                       # (rows, n)
            dp_all = dd @ vv.T
            dsum = (p_all * dp_all).sum(axis=1, keepdims=True)
            p = np.exp((qq @ ksel.T) * scale - m) / z        # columns of the sampled keys
            dp = dd @ vsel.T
            ds = p * (dp - dsum)
            dv[sel] += p.T @ dd
            dk[sel] += scale * (ds.T @ qq)
    return dk, dv
