"""Work accounting for shared-prompt attention (measurement only).

Useful work counts visible (query, key) pairs of a head.  Every visible key
set of a query at logical position p is the contiguous position range
[max(0, p-W+1), p] (the shared prompt followed by the query's own
response), so a valid row sees min(p+1, W) keys (W = infinity without a
window).  Padded response rows see none.

FLOPs per visible pair and query head (two per multiply-add):
  forward  4*D  (S = QK^T, O = PV),
  backward 10*D (S recompute, dV, dP, dK, dQ),
and per kernel of this library: dq kernel 6*D (S, dP, dQ), dkdv kernel 8*D
(S, dP, dV, dK).  Softmax exponentials are not counted.
"""
from __future__ import annotations

import numpy as np


def _row_counts(positions: np.ndarray, window: int) -> int:
    c = positions + 1
    if window > 0:
        c = np.minimum(c, window)
    return int(c.sum())


def visible_pairs(N, P, R, window=0, valid_len=None) -> int:
    """Visible pairs per head of the packed P+NR layout."""
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    a = _row_counts(np.arange(P, dtype=np.int64), window)
    for n in range(N):
        a += _row_counts(P + np.arange(L[n], dtype=np.int64), window)
    return a


def replicated_pairs(N, P, R, window=0, valid_len=None) -> int:
    """Visible pairs per head of the N replicated (P+R)-token sequences."""
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    a = 0
    for n in range(N):
        a += _row_counts(np.arange(P + L[n], dtype=np.int64), window)
    return a


def flops(pairs: int, n_q_heads: int, head_dim: int) -> dict:
    u = pairs * n_q_heads * head_dim
    return {"fwd": 4 * u, "bwd": 10 * u, "fwd_bwd": 14 * u, "kernel_fwd": 4 * u,
            "kernel_bwd_dq": 6 * u, "kernel_bwd_dkdv": 8 * u}


def token_ratio(N, P, R) -> float:
    """rho = N(P+R) / (P+NR)."""
    return N * (P + R) / (P + N * R)
