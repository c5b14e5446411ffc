"""Packed-layout bookkeeping and the visibility definition (oracle side).

Source: "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422),
Abstract.  The micro-batch of N sequences that share a prompt is repacked
from N(P+R) rows into P+NR rows; attention for a response query runs over
two disjoint key regions, the shared prompt and that response's own
tokens, and prompt queries see the prompt only (causal masking).

Readings where the abstract is silent:
* packed row order: prompt rows 0..P-1, then response n at rows
  P+nR .. P+nR+R-1 for n = 0..N-1;
* a response token r has logical position P+r; causal order and the
  sliding window use logical positions;
* causal is inclusive (a token sees itself);
* window W > 0 keeps keys with 0 <= pos_q - pos_k < W (W positions
  including self); W <= 0 means no window;
* padded response rows (r >= L_n) are masked both as queries and as keys.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import numpy as np


def row_layout(N: int, P: int, R: int):
    """Return (seg, pos, r) for every packed row.

    seg = -1 for prompt rows, n for rows of response n; pos = logical
    position; r = index inside the response (-1 for prompt rows).
    """
    T = P + N * R
    t = np.arange(T, dtype=np.int64)
    is_prompt = t < P
    rel = t - P
    if R > 0:
        seg = np.where(is_prompt, -1, rel // R)
        r = np.where(is_prompt, -1, rel % R)
    else:
        seg = np.full(T, -1, dtype=np.int64)
        r = np.full(T, -1, dtype=np.int64)
    pos = np.where(is_prompt, t, P + r)
    return seg, pos, r


def row_valid(N: int, P: int, R: int, valid_len=None) -> np.ndarray:
    """True for prompt rows and for response rows with r < L_n."""
    seg, pos, r = row_layout(N, P, R)
    if valid_len is None:
        return np.ones(P + N * R, dtype=bool)
    L = np.asarray(valid_len, dtype=np.int64)
    Lrow = np.where(seg >= 0, L[np.maximum(seg, 0)], 0)
    return (seg < 0) | (r < Lrow)


def visibility(N: int, P: int, R: int, window: int = 0, valid_len=None) -> np.ndarray:
    """Dense [T, T] boolean: entry (i, j) is True iff key row j is visible
    to query row i in the packed layout.

    j is visible to i iff both rows are valid, pos_j <= pos_i, j lies in
    the shared prompt or in i's own response, and (with a window W > 0)
    pos_i - pos_j < W.
    """
    seg, pos, _ = row_layout(N, P, R)
    ok = row_valid(N, P, R, valid_len)
    qi = (slice(None), None)
    kj = (None, slice(None))
    same_region = (seg[kj] == -1) | (seg[kj] == seg[qi])
    vis = ok[qi] & ok[kj] & (pos[kj] <= pos[qi]) & same_region
    if window > 0:
        vis &= (pos[qi] - pos[kj]) < window
    return vis


def count_visible_pairs(N: int, P: int, R: int, window: int = 0, valid_len=None) -> int:
    """Number of visible (query, key) pairs per head, by enumeration."""
    return int(visibility(N, P, R, window, valid_len).sum())
