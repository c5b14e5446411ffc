"""The N(P+R) <-> P+NR row maps (oracle side).

Source: "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422),
Abstract: the data pipeline repacks the N(P+R) tokens of a micro-batch
into P+NR tokens, keeping one copy of the shared prompt.

Readings: the replicated layout is N sequences [prompt; response n], each
P+R rows; the packed layout is [prompt; response 0; ...; response N-1].
GATHER (replicated -> packed) takes the prompt from copy 0.  SCATTER
(packed -> replicated) broadcasts the prompt to every copy.  Both are
pure row copies, so they are bit exact for any row content.

TEST INFRASTRUCTURE ONLY.
"""
from __future__ import annotations

import numpy as np


def gather_rows(N: int, P: int, R: int) -> np.ndarray:
    """Replicated row index that packed row t copies from."""
    idx = []
    for t in range(P):
        idx.append(t)                       # prompt, copy 0
    for n in range(N):
        for r in range(R):
            idx.append(n * (P + R) + P + r)  # response n, token r
    return np.asarray(idx, dtype=np.int64)


def scatter_rows(N: int, P: int, R: int) -> np.ndarray:
    """Packed row index that replicated row u copies from."""
    idx = []
    for n in range(N):
        for i in range(P):
            idx.append(i)                    # prompt broadcast
        for r in range(R):
            idx.append(P + n * R + r)
    return np.asarray(idx, dtype=np.int64)


def gather(replicated: np.ndarray, N: int, P: int, R: int) -> np.ndarray:
    return replicated[gather_rows(N, P, R)]


def scatter(packed: np.ndarray, N: int, P: int, R: int) -> np.ndarray:
    return packed[scatter_rows(N, P, R)]
