"""Several prompt groups in one packed micro-batch (oracle side, fp64).

"DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
a micro-batch of responses that share one prompt is packed as P+NR rows.
A micro-batch holding several prompts is read here as several such packed
groups laid one after the other (row offsets like the cumulative sequence
offsets of variable-length attention); attention never crosses a group,
so every group is its own shared-prompt problem.

* ``layout``          row offsets of the groups;
* ``grouped_fold``    the definition: each group's rows through
                      ``replicated.replicated_fold`` (its N replicated
                      causal sequences), the results placed at its rows;
* ``visibility``      the dense [Tld, Tld] mask of the whole micro-batch,
                      from every row's group, segment and position;
* ``grouped_dense``   dense masked attention with that mask (tiny inputs),
                      a second, independent route to the same numbers.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import numpy as np

from . import dense, replicated
from .mask import row_layout


def layout(groups):
    """[(row0, T_g, vl0), ...]: first packed row, rows and first valid-length
    entry of every group."""
    out, row, vl = [], 0, 0
    for N, P, R in groups:
        out.append((row, P + N * R, vl))
        row += P + N * R
        vl += N
    return out


def grouped_fold(q, k, v, do, groups, window=0, scale=None, valid_len=None, backward=True,
                 delta_o=None):
    """dict(o, lse, dq, dk, dv) over all packed rows of the groups."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = np.shape(k)[1]
    out = dict(o=np.zeros((T, Hq, D)), lse=np.full((Hq, T), -np.inf))
    if backward:
        out.update(dq=np.zeros((T, Hq, D)), dk=np.zeros((T, Hkv, D)), dv=np.zeros((T, Hkv, D)))
    for (N, P, R), (r0, Tg, vl0) in zip(groups, layout(groups)):
        if Tg == 0:
            continue
        rows = slice(r0, r0 + Tg)
        vl = None if valid_len is None else np.asarray(valid_len)[vl0:vl0 + N]
        res = replicated.replicated_fold(q[rows], k[rows], v[rows], None if do is None else do[rows],
                                         N, P, R, window, scale, vl, backward=backward, delta_o=delta_o)
        out["o"][rows] = res["o"]
        out["lse"][:, rows] = res["lse"]
        if backward:
            for name in ("dq", "dk", "dv"):
                out[name][rows] = res[name]
    return out


def visibility(groups, window=0, valid_len=None):
    """Dense [Tld, Tld] boolean: key row j visible to query row i.

    Both rows in the same group, both valid, pos_j <= pos_i, j in the
    group's prompt or in i's own response, and pos_i - pos_j < W with a
    window W > 0 (positions counted inside the group)."""
    gid, seg, pos, ok = [], [], [], []
    for gi, ((N, P, R), (_, Tg, vl0)) in enumerate(zip(groups, layout(groups))):
        s, p, r = row_layout(N, P, R)
        L = np.full(N, R) if valid_len is None else np.asarray(valid_len, dtype=np.int64)[vl0:vl0 + N]
        valid = (s < 0) | (r < np.where(s >= 0, L[np.maximum(s, 0)], 0))
        gid.append(np.full(Tg, gi))
        seg.append(s)
        pos.append(p)
        ok.append(valid)
    gid, seg, pos, ok = (np.concatenate(a) if a else np.zeros(0, dtype=np.int64) for a in (gid, seg, pos, ok))
    ok = ok.astype(bool)
    qi, kj = (slice(None), None), (None, slice(None))
    vis = (gid[qi] == gid[kj]) & ok[qi] & ok[kj] & (pos[kj] <= pos[qi])
    vis &= (seg[kj] == -1) | (seg[kj] == seg[qi])
    if window > 0:
        vis &= (pos[qi] - pos[kj]) < window
    return vis


def grouped_dense(q, k, v, do, groups, window=0, scale=None, valid_len=None):
    """Dense masked forward and analytic backward over the whole micro-batch."""
    vis = visibility(groups, window, valid_len)
    o, lse = dense.forward_masked(q, k, v, vis, scale)
    dq, dk, dv = dense.backward_masked(q, k, v, o, lse, do, vis, scale)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
