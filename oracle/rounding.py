"""Per-element error envelope of a bf16 backward (a tolerance model, fp64).

"DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
the method is exact, so a bf16 implementation differs from the fp64
definition only by its roundings.  The reading of where a bf16 kernel
rounds: inputs are bf16; P is rounded to bf16 before the P.V product; the
forward output O is stored in bf16 and the backward forms Delta = dO . O
from that stored O; dS is rounded to bf16 before the dQ and dK products; P
is rounded to bf16 before the dV product.  On inputs whose softmax is close
to one-hot, dS = P (dP - Delta) cancels and those roundings move single
gradient elements by far more than the usual 2e-2 * max(1, |y|).  This
module bounds that movement from the fp64 oracle's own quantities, so that
a parity test of such inputs can keep an element-by-element gate.

With u = 2^-8 (bf16 unit roundoff) and a rounding modelled as an
independent error of standard deviation u |x| / sqrt(3):

* the stored O of a bf16 forward and the oracle's O rounded to bf16 are at
  most one bf16 step apart, so |dDelta_i| <= e_i = 2u sum_d |dO_id O_id|
  and, as a random quantity, var(dDelta_i) = (2u)^2/3 sum_d (dO_id O_id)^2;
* dQ_i moves by scale * dDelta_i * (sum_j p_ij k_j) (one quantity per row:
  the bound e_i is used) plus the dS roundings, sum over j of independent
  terms: var = scale^2 u^2/3 sum_j ds_ij^2 k_j^2;
* dK_j: scale^2 sum_i p_ij^2 q_i^2 var(dDelta_i) + scale^2 u^2/3 sum_i
  ds_ij^2 q_i^2;  dV_j: u^2/3 sum_i p_ij^2 dO_i^2;
* the envelope is e-term + 6 sigma (dQ), 6 sigma (dK, dV).

Terms are computed per replicated sequence exactly as ``oracle.replicated``
does (prompt dO to copy 0 only) and folded over the copies (bounds add,
variances add).  Pinned in tests/test_oracle_rounding.py against a plain
fp64 emulation of those roundings.

TEST INFRASTRUCTURE ONLY.
"""
from __future__ import annotations

import numpy as np

from .replicated import round_bf16, sequence_rows

U = 2.0 ** -8


def _sequence_terms(q, k, v, do, n_valid, window, scale):
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    eq = np.zeros((S, Hq, D))
    vk = np.zeros((S, Hkv, D))
    vv = np.zeros((S, Hkv, D))
    var1 = U * U / 3.0
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    vis = (j <= i) & (i < n_valid) & (j < n_valid)
    if window > 0:
        vis &= (i - j) < window
    has = vis.any(axis=1)
    for h in range(Hq):
        c = h // g
        s = np.where(vis, scale * (q[:, h] @ k[:, c].T), -np.inf)
        m = np.where(has, s.max(axis=1), 0.0)
        lse = np.where(has, m + np.log(np.where(has, np.exp(s - m[:, None]).sum(axis=1), 1.0)), 0.0)
        p = np.where(vis, np.exp(s - lse[:, None]), 0.0)
        o = p @ v[:, c]
        dd = do[:, h]
        delta = (dd * round_bf16(o)).sum(axis=1)
        ds = p * (dd @ v[:, c].T - delta[:, None])
        e = 2.0 * U * np.abs(dd * o).sum(axis=1)
        var_delta = 4.0 * var1 * ((dd * o) ** 2).sum(axis=1)
        eq[:, h] = scale * (e[:, None] * np.abs(p @ k[:, c])
                            + 6.0 * np.sqrt(var1 * ((ds ** 2) @ (k[:, c] ** 2))))
        vk[:, c] += scale ** 2 * ((p ** 2 * var_delta[:, None]).T @ (q[:, h] ** 2)
                                  + var1 * ((ds ** 2).T @ (q[:, h] ** 2)))
        vv[:, c] += var1 * ((p ** 2).T @ (dd ** 2))
    return eq, vk, vv


def backward_envelope(q, k, v, do, N, P, R, window=0, scale=None, valid_len=None):
    """Envelopes dict(dq, dk, dv) on the packed rows (same shapes as the
    gradients) for the roundings listed in the module docstring."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    eq = np.zeros((T, Hq, D))
    vk = np.zeros((T, Hkv, D))
    vv = np.zeros((T, Hkv, D))
    for n in range(N):
        idx = sequence_rows(n, N, P, R)
        don = do[idx].copy()
        if n != 0:
            don[:P] = 0.0
        a, b, c = _sequence_terms(q[idx], k[idx], v[idx], don, P + L[n], window, scale)
        rs = slice(P + n * R, P + (n + 1) * R)
        eq[:P] += a[:P]
        vk[:P] += b[:P]
        vv[:P] += c[:P]
        eq[rs], vk[rs], vv[rs] = a[P:], b[P:], c[P:]
    return dict(dq=eq, dk=6.0 * np.sqrt(vk), dv=6.0 * np.sqrt(vv))
