"""Skiparse-2D attention, written out plainly in float64 (test infrastructure only).

What the method computes (OSP-Next summary, 核心方法 core method, and
方法步骤详情 method steps; OSP-Next abstract):

* Video tokens of shape (B, T, H, W, C) -- here C is split into (heads, d) --
  are regrouped by a fixed rule into k*k subsequences, each 1/k^2 of the tokens.
* token-wise: like pixel unshuffle, the H x W map is cut into k x k sub-maps;
  token (h, w) joins subsequence (h mod k, w mod k).
* group-wise: like patch unshuffle, k x k blocks of tokens are grouped; the
  block (h // k, w // k) joins subsequence ((h // k) mod k, (w // k) mod k).
  The 2D pattern is the 1D skip pattern applied to each spatial axis on its own
  (OSP-Next summary, 技术新颖性 novelty).
* Dense softmax attention runs inside each subsequence; the result is put back
  in the original layout.
* Any resolution: when H or W is not a multiple of k^2 it is padded up to the
  nearest multiple and the padded tokens are masked, so that a position follows
  the same pattern at every resolution (方法步骤详情 method steps).

Readings taken where the pages leave a step open (each is listed in the design
notes): padding goes at the high end of each axis; every subsequence spans all
T frames; batch and heads are independent; padded tokens are never keys and
padded queries are discarded; the softmax scale is 1/sqrt(d); the canonical
order inside a subsequence is row-major in the original (t, h, w).

Two independent formulations are kept on purpose: ``gather_map`` builds the
index map from the per-axis closed form, while ``skiparse_attention`` pads and
rearranges with reshape/transpose exactly as the einops-style description
reads.  Tests check each against the other and against torch's pixel_unshuffle
and hand-derived maps.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TOKEN = 0     # token-wise pattern
GROUP = 1     # group-wise pattern
TOKEN_1D = 2  # Skiparse-1D, token-wise, on the flattened (h, w) of each frame
GROUP_1D = 3  # Skiparse-1D, group-wise


def is_1d(mode: int) -> bool:
    """Skiparse-1D: the skip pattern of one axis applied to the flattened
    spatial sequence (OSP-Next summary, 技术新颖性 novelty: the 2D pattern is
    the 1D one applied to each spatial axis, and the flattened 1D variant is
    what it is compared with).  Reading: each frame's (h, w) is flattened to
    l = h*W + w, the 1D rule runs along l with stride K = k*k (so the density
    1/k^2 matches the 2D pattern), l is padded at its end to a multiple of K^2,
    and every subsequence spans all T frames."""
    return mode in (TOKEN_1D, GROUP_1D)


def rule_of(mode: int) -> int:
    """The per-axis rule (TOKEN or GROUP) a mode applies."""
    return GROUP if mode in (GROUP, GROUP_1D) else TOKEN


# ---------------------------------------------------------------------------
# Per-axis index function
# ---------------------------------------------------------------------------

def padded_extent(n: int, k: int) -> int:
    """Round a spatial extent up to a multiple of k^2 (any-resolution rule,
    OSP-Next summary, 方法步骤详情 method steps)."""
    m = k * k
    return ((n + m - 1) // m) * m


def subsequence_coord(x, k: int, mode: int):
    """Subsequence coordinate of spatial index ``x`` along one axis.

    token-wise (pixel unshuffle): x mod k.
    group-wise (patch unshuffle of k x k blocks, block index mod k): (x // k) mod k.
    (OSP-Next summary, 核心方法 core method.)
    """
    if k == 1:
        return x * 0
    if mode == TOKEN:
        return x % k
    return (x // k) % k


def spatial_of_local(xl, p: int, k: int, mode: int):
    """The spatial index whose subsequence coordinate is ``p`` and whose
    position on that subsequence's local axis is ``xl``."""
    if k == 1:
        return xl
    if mode == TOKEN:
        return xl * k + p
    return (xl // k) * (k * k) + p * k + xl % k


def real_extent(n: int, k: int, mode: int, p: int) -> int:
    """Number of real (unpadded) indices x < n on axis coordinate ``p``, counted
    one by one."""
    return int(sum(1 for x in range(n) if subsequence_coord(x, k, mode) == p))


# ---------------------------------------------------------------------------
# Plan
# ---------------------------------------------------------------------------

@dataclass
class Plan:
    """Geometry of one Skiparse-2D attention call."""
    B: int
    T: int
    H: int
    W: int
    heads: int
    d: int
    k: int
    mode: int
    Hp: int = 0
    Wp: int = 0
    sub_h: int = 0          # local grid rows Hp / k
    sub_w: int = 0          # local grid cols Wp / k
    n_sub: int = 0          # k * k
    sub_len_padded: int = 0  # T * sub_h * sub_w
    real_h: list = field(default_factory=list)  # real local rows per p
    real_w: list = field(default_factory=list)  # real local cols per q
    sub_len: list = field(default_factory=list)  # real tokens per subsequence s = p*k+q
    pairs: int = 0          # computed (real x real, same subsequence) pairs

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs: 2*d for Q.K and 2*d for P.V per computed pair."""
        return 4 * self.d * self.pairs


def make_plan(B, T, H, W, heads, d, k, mode) -> Plan:
    mode = TOKEN if k == 1 else mode
    p = Plan(B, T, H, W, heads, d, k, mode)
    if is_1d(mode):
        # the flattened axis l = h*W + w of length L as the single row of a
        # (T, 1, Lp) grid, stride K along it
        K, L = k * k, H * W
        p.Hp, p.Wp = 1, padded_extent(L, K)
        p.sub_h, p.sub_w = 1, p.Wp // K
        p.n_sub = K
        p.sub_len_padded = T * p.sub_w
        p.real_h = [1]
        p.real_w = [real_extent(L, K, rule_of(mode), q) for q in range(K)]
        p.sub_len = [T * r for r in p.real_w]
        p.pairs = sum(n * n for n in p.sub_len) * B * heads
        return p
    p.Hp, p.Wp = padded_extent(H, k), padded_extent(W, k)
    p.sub_h, p.sub_w = p.Hp // k, p.Wp // k
    p.n_sub = k * k
    p.sub_len_padded = T * p.sub_h * p.sub_w
    p.real_h = [real_extent(H, k, mode, i) for i in range(k)]
    p.real_w = [real_extent(W, k, mode, i) for i in range(k)]
    p.sub_len = [T * p.real_h[a] * p.real_w[b] for a in range(k) for b in range(k)]
    p.pairs = sum(n * n for n in p.sub_len) * B * heads
    return p


# ---------------------------------------------------------------------------
# Gather map (closed form)
# ---------------------------------------------------------------------------

def gather_map(T: int, H: int, W: int, k: int, mode: int) -> np.ndarray:
    """Index map G of shape (k*k, T*(Hp/k)*(Wp/k)).

    G[s, j] is the flat token index (t*H + h)*W + w that slot j of subsequence
    s = p*k + q holds, or -1 for a padded slot.  Slot j enumerates the padded
    local grid (T, Hp/k, Wp/k) row-major.
    """
    mode = TOKEN if k == 1 else mode
    if is_1d(mode):
        # slot j = t * (Lp/K) + l' of subsequence q holds l = the l'-th index
        # of coordinate q along the flattened axis
        K, L = k * k, H * W
        sw = padded_extent(L, K) // K
        t = np.arange(T)[:, None]
        G = np.full((K, T * sw), -1, dtype=np.int64)
        for q in range(K):
            l = spatial_of_local(np.arange(sw), q, K, rule_of(mode))[None, :]
            G[q] = np.where((l < L) & (t >= 0), t * L + l, -1).reshape(-1)
        return G
    Hp, Wp = padded_extent(H, k), padded_extent(W, k)
    sh, sw = Hp // k, Wp // k
    G = np.full((k * k, T * sh * sw), -1, dtype=np.int64)
    t = np.arange(T)[:, None, None]
    for p in range(k):
        h = spatial_of_local(np.arange(sh), p, k, mode)[None, :, None]
        for q in range(k):
            w = spatial_of_local(np.arange(sw), q, k, mode)[None, None, :]
            tok = (t * H + h) * W + w
            ok = (h < H) & (w < W) & (t >= 0)
            G[p * k + q] = np.where(ok, tok, -1).reshape(-1)
    return G


def subsequence_members(T, H, W, k, mode) -> list:
    """Real token indices of each subsequence, in canonical order."""
    G = gather_map(T, H, W, k, mode)
    return [row[row >= 0] for row in G]


# ---------------------------------------------------------------------------
# Literal rearrange (pad -> reshape/transpose), and its inverse
# ---------------------------------------------------------------------------

def _rearrange_axes(k, mode):
    """Reshape factors and permutation for 't (...) (...) -> (p q) (t ...)'."""
    if mode == TOKEN:
        # t (h' p) (w' q) heads d -> p q heads (t h' w') d
        return "token", (0, 3, 5, 6, 1, 2, 4, 7)
    # t (hb p kh) (wb q kw) heads d -> p q heads (t hb kh wb kw) d
    return "group", (0, 3, 6, 8, 1, 2, 4, 5, 7, 9)


def rearrange_literal(x: np.ndarray, k: int, mode: int) -> np.ndarray:
    """(B, T, Hp, Wp, heads, d) -> (B, k*k, heads, T*(Hp/k)*(Wp/k), d)."""
    B, T, Hp, Wp, nh, d = x.shape
    if k == 1:
        return x.reshape(B, 1, T * Hp * Wp, nh, d).transpose(0, 1, 3, 2, 4)
    kind, perm = _rearrange_axes(k, mode)
    if kind == "token":
        y = x.reshape(B, T, Hp // k, k, Wp // k, k, nh, d)
    else:
        y = x.reshape(B, T, Hp // (k * k), k, k, Wp // (k * k), k, k, nh, d)
    y = y.transpose(perm)
    return y.reshape(B, k * k, nh, -1, d)


def inverse_rearrange_literal(y: np.ndarray, T, Hp, Wp, k, mode) -> np.ndarray:
    """Inverse of :func:`rearrange_literal`."""
    B, S, nh, L, d = y.shape
    if k == 1:
        return y.transpose(0, 1, 3, 2, 4).reshape(B, T, Hp, Wp, nh, d)
    kind, perm = _rearrange_axes(k, mode)
    inv = np.argsort(perm)
    if kind == "token":
        shp = (B, k, k, nh, T, Hp // k, Wp // k, d)
    else:
        shp = (B, k, k, nh, T, Hp // (k * k), k, Wp // (k * k), k, d)
    x = y.reshape(shp).transpose(inv)
    return x.reshape(B, T, Hp, Wp, nh, d)


def pad_tokens(x: np.ndarray, k: int) -> np.ndarray:
    """Zero-pad H and W at the high end up to multiples of k^2."""
    B, T, H, W, nh, d = x.shape
    Hp, Wp = padded_extent(H, k), padded_extent(W, k)
    out = np.zeros((B, T, Hp, Wp, nh, d), dtype=x.dtype)
    out[:, :, :H, :W] = x
    return out


# --- Skiparse-1D: flatten, pad, reshape/transpose --------------------------

def rearrange_1d_literal(x: np.ndarray, k: int, mode: int) -> np.ndarray:
    """(B, T, Lp, heads, d), the flattened and padded frames, ->
    (B, K, heads, T*Lp/K, d) with K = k*k:
    token-wise 't (l' q) -> q (t l')', group-wise 't (lb q kl) -> q (t lb kl)'."""
    B, T, Lp, nh, d = x.shape
    K = k * k
    if rule_of(mode) == TOKEN:
        y = x.reshape(B, T, Lp // K, K, nh, d).transpose(0, 3, 4, 1, 2, 5)
    else:
        y = x.reshape(B, T, Lp // (K * K), K, K, nh, d).transpose(0, 3, 5, 1, 2, 4, 6)
    return y.reshape(B, K, nh, -1, d)


def inverse_rearrange_1d_literal(y: np.ndarray, T: int, Lp: int, k: int, mode: int) -> np.ndarray:
    """Inverse of :func:`rearrange_1d_literal`."""
    B, K, nh, _, d = y.shape
    if rule_of(mode) == TOKEN:
        x = y.reshape(B, K, nh, T, Lp // K, d).transpose(0, 3, 4, 1, 2, 5)
    else:
        x = y.reshape(B, K, nh, T, Lp // (K * K), K, d).transpose(0, 3, 4, 1, 5, 2, 6)
    return x.reshape(B, T, Lp, nh, d)


# --- both patterns: pad -> rearrange, and back -----------------------------

def to_subsequences(x: np.ndarray, kf: int, mode: int) -> np.ndarray:
    """Pad and rearrange (B, T, H, W, heads, d) into (B, n_sub, heads, L_sub, d)."""
    mode = TOKEN if kf == 1 else mode
    if not is_1d(mode):
        return rearrange_literal(pad_tokens(x, kf), kf, mode)
    B, T, H, W, nh, d = x.shape
    Lp = padded_extent(H * W, kf * kf)
    flat = np.zeros((B, T, Lp, nh, d), dtype=x.dtype)
    flat[:, :, :H * W] = x.reshape(B, T, H * W, nh, d)
    return rearrange_1d_literal(flat, kf, mode)


def subsequence_real_mask(T: int, H: int, W: int, kf: int, mode: int) -> np.ndarray:
    """(n_sub, L_sub) bool: which slots of each rearranged subsequence are real."""
    m = np.ones((1, T, H, W, 1, 1), dtype=bool)
    return to_subsequences(m, kf, mode)[0, :, 0, :, 0]


def from_subsequences(y: np.ndarray, T: int, H: int, W: int, kf: int, mode: int) -> np.ndarray:
    """Rearrange back and crop: (B, n_sub, heads, L_sub, d) -> (B, T, H, W, heads, d)."""
    mode = TOKEN if kf == 1 else mode
    if not is_1d(mode):
        full = inverse_rearrange_literal(y, T, padded_extent(H, kf), padded_extent(W, kf), kf, mode)
        return full[:, :, :H, :W]
    B, nh, d = y.shape[0], y.shape[2], y.shape[4]
    Lp = padded_extent(H * W, kf * kf)
    flat = inverse_rearrange_1d_literal(y, T, Lp, kf, mode)
    return flat[:, :, :H * W].reshape(B, T, H, W, nh, d)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def softmax_attention(q, k, v, scale, key_ok=None):
    """Textbook softmax attention in float64: softmax(scale * q k^T) v, with the
    keys where ``key_ok`` is False excluded.  q: (Lq, d), k/v: (Lk, d)."""
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    if key_ok is not None:
        s = np.where(key_ok[None, :], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ np.asarray(v, np.float64)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def skiparse_attention(q, k, v, kf: int, mode: int, scale=None) -> np.ndarray:
    """Skiparse-2D attention forward, following the method steps in order:
    pad -> rearrange -> masked dense attention per subsequence -> rearrange back
    -> crop.  Inputs and output are (B, T, H, W, heads, d); computed in float64.
    """
    q = np.asarray(q, np.float64)
    k_ = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, W, nh, d = q.shape
    mode = TOKEN if kf == 1 else mode
    scale = default_scale(d) if scale is None else scale
    qs, ks, vs = (to_subsequences(x, kf, mode) for x in (q, k_, v))
    ok = subsequence_real_mask(T, H, W, kf, mode)
    out = np.zeros_like(qs)
    for b in range(B):
        for s in range(qs.shape[1]):
            if not ok[s].any():
                continue  # a subsequence made only of padding has nothing to attend
            for h in range(nh):
                o = softmax_attention(qs[b, s, h], ks[b, s, h], vs[b, s, h], scale, ok[s])
                o[~ok[s]] = 0.0  # padded queries are discarded
                out[b, s, h] = o
    return from_subsequences(out, T, H, W, kf, mode)


# ---------------------------------------------------------------------------
# Brute force: full attention under the equivalent block mask
# ---------------------------------------------------------------------------

def block_mask(T, H, W, k, mode) -> np.ndarray:
    """(N, N) bool over the unpadded tokens: True where two tokens fall in the
    same subsequence, decided token by token from the membership rule."""
    mode = TOKEN if k == 1 else mode
    N = T * H * W
    sub = np.empty(N, dtype=np.int64)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                x = (t * H + h) * W + w
                if is_1d(mode):   # the 1D rule on the flattened index, stride k*k
                    sub[x] = subsequence_coord(h * W + w, k * k, rule_of(mode))
                else:
                    sub[x] = subsequence_coord(h, k, mode) * k + subsequence_coord(w, k, mode)
    return sub[:, None] == sub[None, :]


def masked_full_attention(q, k, v, mask, scale=None) -> np.ndarray:
    """Full attention over all N tokens where query x may only see keys y with
    mask[x, y].  q/k/v: (B, T, H, W, heads, d); loops over batch and heads."""
    q = np.asarray(q, np.float64)
    B, T, H, W, nh, d = q.shape
    scale = default_scale(d) if scale is None else scale
    N = T * H * W
    qf = q.reshape(B, N, nh, d)
    kf = np.asarray(k, np.float64).reshape(B, N, nh, d)
    vf = np.asarray(v, np.float64).reshape(B, N, nh, d)
    out = np.zeros_like(qf)
    for b in range(B):
        for h in range(nh):
            s = (qf[b, :, h] @ kf[b, :, h].T) * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h] = p @ vf[b, :, h]
    return out.reshape(q.shape)


def probability_matrix(q, k, kf: int, mode: int, b: int, head: int, scale=None) -> np.ndarray:
    """(N, N) attention probabilities of one (batch, head): row x holds the
    softmax weights query x puts on every token (zero outside its subsequence)."""
    q = np.asarray(q, np.float64)
    B, T, H, W, nh, d = q.shape
    scale = default_scale(d) if scale is None else scale
    N = T * H * W
    mask = block_mask(T, H, W, kf, mode)
    s = (q.reshape(B, N, nh, d)[b, :, head] @ np.asarray(k, np.float64).reshape(B, N, nh, d)[b, :, head].T) * scale
    s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Sampled rows at full size
# ---------------------------------------------------------------------------

_MEMBERS_CACHE: dict = {}


def _members_for(shape_key):
    if shape_key not in _MEMBERS_CACHE:
        T, H, W, kf, mode = shape_key
        G = gather_map(T, H, W, kf, mode)
        sub_of = np.full(T * H * W, -1, np.int64)
        for s, row in enumerate(G):
            sub_of[row[row >= 0]] = s
        _MEMBERS_CACHE[shape_key] = ([row[row >= 0] for row in G], sub_of)
    return _MEMBERS_CACHE[shape_key]


def attention_rows(q, k, v, T, H, W, kf, mode, b, head, tokens, scale=None):
    """Output rows O[b, token, head, :] in float64 for real flat token indices
    ``tokens``, each computed on its own from all keys of its subsequence.

    q, k, v are indexable as (B, N, heads, d) with N = T*H*W (numpy arrays of
    any float dtype); only the rows that are needed are widened to float64.
    """
    B, N, nh, d = q.shape
    assert N == T * H * W
    scale = default_scale(d) if scale is None else scale
    members, sub_of = _members_for((T, H, W, kf, TOKEN if kf == 1 else mode))
    tokens = np.asarray(tokens, np.int64)
    if tokens.size and (tokens.min() < 0 or tokens.max() >= N):
        raise IndexError("token index out of range")
    out = np.zeros((tokens.size, d), np.float64)
    for s in np.unique(sub_of[tokens]):
        sel = np.nonzero(sub_of[tokens] == s)[0]
        mem = members[s]
        kk = np.asarray(k[b, mem, head], np.float64)
        vv = np.asarray(v[b, mem, head], np.float64)
        qq = np.asarray(q[b, tokens[sel], head], np.float64)
        out[sel] = softmax_attention(qq, kk, vv, scale)
    return out


def pair_count(B, T, H, W, heads, k, mode) -> int:
    """Computed (real x real, same subsequence) pairs, counted from the map."""
    members = subsequence_members(T, H, W, k, mode)
    return int(sum(len(m) ** 2 for m in members)) * B * heads
