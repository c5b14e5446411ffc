"""O1: dense attention over the packed P+NR layout (tiny inputs only).

This is the definition written out: for every query head, the scaled
scores against every key row, the visibility mask of ``oracle.mask``,
softmax, and the analytic backward of softmax attention.  The method is
exactly equal to standard attention ("DualKV: Shared-Prompt Flash
Attention ...", arXiv 2605.15422, Abstract), so no approximation appears.

Conventions (readings where the abstract is silent):
* GQA: query head h uses KV head h // (Hq / Hkv);
* LSE is the natural-log log-sum-exp of the *scaled* scores, [Hq, T];
* a query row with no visible key has O = 0, LSE = -inf, dQ = 0;
* dK/dV of a KV head sum over all query heads of its group.

All arithmetic is fp64.  TEST INFRASTRUCTURE ONLY.
"""
from __future__ import annotations

import numpy as np

from .mask import visibility


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(q, k, v, N, P, R, window=0, scale=None, valid_len=None):
    """Return (O [T,Hq,D], LSE [Hq,T]) in fp64."""
    return forward_masked(q, k, v, visibility(N, P, R, window, valid_len), scale)


def forward_masked(q, k, v, vis, scale=None):
    """Dense attention with an explicit [T, T] visibility mask (query row,
    key row); returns (O [T,Hq,D], LSE [Hq,T]) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    has = vis.any(axis=1)
    o = np.zeros((T, Hq, D))
    lse = np.full((Hq, T), -np.inf)
    for h in range(Hq):
        c = h // g
        s = scale * (q[:, h, :] @ k[:, c, :].T)
        s = np.where(vis, s, -np.inf)[has]
        m = s.max(axis=1)
        l = np.exp(s - m[:, None]).sum(axis=1)
        lse_h = m + np.log(l)
        p = np.exp(s - lse_h[:, None])
        o[has, h, :] = p @ v[:, c, :]
        lse[h, has] = lse_h
    return o, lse


def backward(q, k, v, o, lse, do, N, P, R, window=0, scale=None, valid_len=None):
    """Analytic backward of ``forward``; returns (dQ, dK, dV) in fp64."""
    return backward_masked(q, k, v, o, lse, do, visibility(N, P, R, window, valid_len), scale)


def backward_masked(q, k, v, o, lse, do, vis, scale=None):
    """Analytic backward of ``forward_masked``; returns (dQ, dK, dV)."""
    q, k, v, o, lse, do = map(_f64, (q, k, v, o, lse, do))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        c = h // g
        s = scale * (q[:, h, :] @ k[:, c, :].T)
        lh = lse[h]
        ok = np.isfinite(lh)              # rows with at least one visible key
        p = np.zeros((T, T))
        p[ok] = np.exp(np.where(vis[ok], s[ok] - lh[ok][:, None], -np.inf))
        delta = (do[:, h, :] * o[:, h, :]).sum(axis=1)
        dp = do[:, h, :] @ v[:, c, :].T
        ds = p * (dp - delta[:, None])
        dq[:, h, :] = scale * (ds @ k[:, c, :])
        dk[:, c, :] += scale * (ds.T @ q[:, h, :])
        dv[:, c, :] += p.T @ do[:, h, :]
    return dq, dk, dv
