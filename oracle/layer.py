"""A pre-norm decoder layer on shared-prompt micro-batches (oracle side, fp64).

"DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
the packed P+NR layout carries its token reduction from attention to the
whole model; the packed computation is exactly the replicated one on each
of the N sequences [prompt; response n].  The layer (the plainest one the
pages' models share; the abstract names none of its parts beyond
attention):

    h1 = RMSNorm(x; n1);  q, k, v = h1 Wq, h1 Wk, h1 Wv
    q, k = RoPE(q, k) at each token's position in its sequence
    o = causal attention (GQA, optional window) over the sequence
    x1 = x + o Wo;  h2 = RMSNorm(x1; n2);  y = x1 + (silu(h2 W1) * (h2 W3)) W2

RoPE rotates the pair (i, i + D/2) of every head by pos * base^(-2i/D).
RMSNorm: x / sqrt(mean(x^2) + eps) * w.  Weights are [in][out].

* ``sequence_layer``   forward and analytic backward on one sequence,
                       attention through ``replicated.causal_sequence``;
* ``layer_fold``       the packed outputs through the N replicated
                       sequences (prompt dY to copy 0 only, prompt dX and all
                       weight gradients summed over the copies), for every
                       group of a micro-batch;
* ``packed_dense_layer`` a second route: token-wise steps on the packed rows
                       (RoPE at logical positions: prompt t -> t, response
                       row r -> P + r) and dense masked attention over the
                       packed layout (tiny inputs).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import numpy as np

from . import dense, replicated
from .groups import layout, visibility as group_visibility

NAMES = ("norm1", "wq", "wk", "wv", "wo", "norm2", "w1", "w3", "w2")


def rmsnorm(x, w, eps):
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * w, r


def rmsnorm_bwd(x, w, r, dy):
    """dx and dw of y = x * r * w, r = (mean(x^2) + eps)^(-1/2)."""
    xh = x * r
    g = dy * w
    dx = r * (g - xh * np.mean(g * xh, axis=-1, keepdims=True))
    dw = (dy * xh).sum(axis=0)
    return dx, dw


def rope(x, pos, base, inverse=False):
    """x [S, H, D]: rotate pair (i, i + D/2) by pos * base^(-2i/D)."""
    S, H, D = x.shape
    half = D // 2
    inv = base ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [S, half]
    if inverse:
        ang = -ang
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(u):
    return u / (1.0 + np.exp(-u))


def swiglu_bwd(u, g, dm):
    s = 1.0 / (1.0 + np.exp(-u))
    return dm * g * s * (1.0 + u * (1.0 - s)), dm * u * s


def _heads(a, H):
    return a.reshape(a.shape[0], H, -1)


def _layer(x, W, dy, pos, Hq, Hkv, base, eps, attend):
    """Forward (and backward if dy is given) of the layer on rows x [S, Hm],
    attention by ``attend``.  Returns dict(y[, dx, grads])."""
    h1, r1 = rmsnorm(x, W["norm1"], eps)
    q = rope(_heads(h1 @ W["wq"], Hq), pos, base)
    k = rope(_heads(h1 @ W["wk"], Hkv), pos, base)
    v = _heads(h1 @ W["wv"], Hkv)
    att = attend(q, k, v, None)
    o = att["o"].reshape(x.shape[0], -1)
    x1 = x + o @ W["wo"]
    h2, r2 = rmsnorm(x1, W["norm2"], eps)
    u, g = h2 @ W["w1"], h2 @ W["w3"]
    m = silu(u) * g
    y = x1 + m @ W["w2"]
    out = dict(y=y)
    if dy is None:
        return out
    G = {}
    dm = dy @ W["w2"].T
    G["w2"] = m.T @ dy
    du, dg = swiglu_bwd(u, g, dm)
    dh2 = du @ W["w1"].T + dg @ W["w3"].T
    G["w1"], G["w3"] = h2.T @ du, h2.T @ dg
    dx1n, G["norm2"] = rmsnorm_bwd(x1, W["norm2"], r2, dh2)
    dx1 = dy + dx1n
    do = _heads(dx1 @ W["wo"].T, Hq)
    G["wo"] = o.T @ dx1
    att = attend(q, k, v, do)
    dq = rope(att["dq"], pos, base, inverse=True).reshape(x.shape[0], -1)
    dk = rope(att["dk"], pos, base, inverse=True).reshape(x.shape[0], -1)
    dv = att["dv"].reshape(x.shape[0], -1)
    dh1 = dq @ W["wq"].T + dk @ W["wk"].T + dv @ W["wv"].T
    G["wq"], G["wk"], G["wv"] = h1.T @ dq, h1.T @ dk, h1.T @ dv
    dxn, G["norm1"] = rmsnorm_bwd(x, W["norm1"], r1, dh1)
    out.update(dx=dx1 + dxn, grads=G)
    return out


def sequence_layer(x, W, dy, n_valid, Hq, Hkv, window, base, eps):
    """The layer on one sequence of S rows (rows >= n_valid are padding:
    masked in attention as queries and keys)."""
    x = np.asarray(x, dtype=np.float64)
    W = {n: np.asarray(W[n], dtype=np.float64) for n in NAMES}

    def attend(q, k, v, do):
        if do is None:
            return replicated.causal_sequence(q, k, v, None, n_valid, window, backward=False)
        return replicated.causal_sequence(q, k, v, do, n_valid, window)

    return _layer(x, W, None if dy is None else np.asarray(dy, dtype=np.float64),
                  np.arange(x.shape[0]), Hq, Hkv, base, eps, attend)


def layer_fold(x, W, dy, groups, Hq, Hkv, window=0, base=1e4, eps=1e-6, valid_len=None):
    """Packed-layout outputs of every group through its replicated sequences.
    Returns dict(y, dx, grads) (dx, grads only if dy is given)."""
    x = np.asarray(x, dtype=np.float64)
    T, Hm = x.shape
    y = np.zeros((T, Hm))
    dx = np.zeros((T, Hm)) if dy is not None else None
    grads = {n: np.zeros(np.shape(W[n])) for n in NAMES} if dy is not None else None
    for (N, P, R), (r0, Tg, vl0) in zip(groups, layout(groups)):
        L = [R] * N if valid_len is None else [int(a) for a in valid_len[vl0:vl0 + N]]
        for n in range(N):
            idx = r0 + replicated.sequence_rows(n, N, P, R)
            dyn = None
            if dy is not None:
                dyn = np.asarray(dy, dtype=np.float64)[idx].copy()
                if n != 0:
                    dyn[:P] = 0.0                  # prompt dY belongs to copy 0 only
            res = sequence_layer(x[idx], W, dyn, P + L[n], Hq, Hkv, window, base, eps)
            rs = slice(r0 + P + n * R, r0 + P + (n + 1) * R)
            if n == 0:
                y[r0:r0 + P] = res["y"][:P]
            y[rs] = res["y"][P:]
            if dy is not None:
                dx[r0:r0 + P] += res["dx"][:P]
                dx[rs] = res["dx"][P:]
                for name in NAMES:
                    grads[name] += res["grads"][name]
    out = dict(y=y)
    if dy is not None:
        out.update(dx=dx, grads=grads)
    return out


def packed_positions(groups):
    """Logical position of every packed row: t for prompt row t of a group,
    P + r for row r of a response."""
    pos = []
    for N, P, R in groups:
        pos.append(np.arange(P))
        for _ in range(N):
            pos.append(P + np.arange(R))
    return np.concatenate(pos) if pos else np.zeros(0, dtype=np.int64)


def packed_dense_layer(x, W, dy, groups, Hq, Hkv, window=0, base=1e4, eps=1e-6, valid_len=None):
    """The layer on the packed rows directly: token-wise steps once per
    packed row, dense masked attention with the micro-batch's visibility."""
    x = np.asarray(x, dtype=np.float64)
    W = {n: np.asarray(W[n], dtype=np.float64) for n in NAMES}
    vis = group_visibility(groups, window, valid_len)

    def attend(q, k, v, do):
        o, lse = dense.forward_masked(q, k, v, vis)
        if do is None:
            return dict(o=o)
        dq, dk, dv = dense.backward_masked(q, k, v, o, lse, do, vis)
        return dict(o=o, dq=dq, dk=dk, dv=dv)

    return _layer(x, W, None if dy is None else np.asarray(dy, dtype=np.float64),
                  packed_positions(groups), Hq, Hkv, base, eps, attend)
