"""Outputs of selected rows, for checks at full layer size (fp64).

Same definition as ``oracle.replicated`` ("DualKV: Shared-Prompt Flash
Attention ...", arXiv 2605.15422, Abstract: exactly standard attention on
the N sequences [prompt; response n]), evaluated only where asked:

* ``query_rows``: O, LSE and dQ of chosen packed query rows.  A prompt row
  belongs to copy 0 (it gets the prompt dO); response row r of response n
  sees sequence n up to its own position.
* ``key_rows``: dK and dV of chosen packed key rows of one KV head.  A key
  row is seen by every query row whose visible range holds it; each such
  query's softmax statistics (LSE, O, Delta) are computed from its full
  visible key range, in query chunks, so no value comes from elsewhere.

Visible key range of a query (logical position p, window W): positions
[max(0, p-W+1), p] of its sequence; padded rows (r >= L_n) see nothing and
are seen by nothing.

TEST INFRASTRUCTURE ONLY.
"""
from __future__ import annotations

import numpy as np


def _seq_keys(t, N, P, R, window, L):
    """Packed key rows visible to packed query row t (ascending position),
    and the query's logical position; None if the row is padding."""
    if t < P:
        pos = t
        rows = np.arange(t + 1)
    else:
        n, r = divmod(t - P, R)
        if r >= L[n]:
            return None, None
        pos = P + r
        rows = np.concatenate([np.arange(P), P + n * R + np.arange(r + 1)])
    if window > 0:
        rows = rows[max(0, pos - window + 1):]
    return rows, pos


def query_rows(q, k, v, do, rows, N, P, R, window=0, scale=None, valid_len=None, heads=None):
    """Return dict(o [n,Hq,D], lse [Hq,n], dq [n,Hq,D]) for packed rows `rows`."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    heads = range(Hq) if heads is None else heads
    out_o = np.zeros((len(rows), Hq, D))
    out_l = np.full((Hq, len(rows)), -np.inf)
    out_dq = np.zeros((len(rows), Hq, D))
    for a, t in enumerate(rows):
        keys, _ = _seq_keys(int(t), N, P, R, window, L)
        if keys is None:
            continue
        c_loaded = None
        for h in heads:
            c = h // g
            if c != c_loaded:
                kk = k[keys, c, :].astype(np.float64)
                vv = v[keys, c, :].astype(np.float64)
                c_loaded = c
            qi = q[t, h, :].astype(np.float64)
            di = do[t, h, :].astype(np.float64)
            s = scale * (kk @ qi)
            m = s.max()
            lse = m + np.log(np.exp(s - m).sum())
            p = np.exp(s - lse)
            o = p @ vv
            delta = di @ o
            ds = p * (vv @ di - delta)
            out_o[a, h] = o
            out_l[h, a] = lse
            out_dq[a, h] = scale * (ds @ kk)
    return dict(o=out_o, lse=out_l, dq=out_dq)


def key_rows(q, k, v, do, rows, kv_head, N, P, R, window=0, scale=None, valid_len=None,
             chunk=1024):
    """Return dict(dk [n,D], dv [n,D]) of packed key rows `rows` of one KV head."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    rows = [int(x) for x in rows]
    dk = np.zeros((len(rows), D))
    dv = np.zeros((len(rows), D))
    # Queries that can see any of the key rows, grouped by sequence.
    # Sequence -1 is the prompt (copy 0), n >= 0 the responses.
    def seq_of(j):
        return -1 if j < P else (j - P) // R

    wanted = set(seq_of(j) for j in rows)
    if -1 in wanted:
        wanted |= set(range(N))          # every response sees the prompt
    c = kv_head
    for seq in sorted(wanted):
        if seq < 0:
            qrows = np.arange(P)
            seq_rows = np.arange(P)
            nvalid = P
        else:
            # queries before the earliest wanted key of this sequence see none
            # of them (unless prompt keys are wanted: every query sees those)
            r_first = 0
            if not any(j < P for j in rows):
                r_first = min(j - P - seq * R for j in rows if seq_of(j) == seq)
            qrows = P + seq * R + np.arange(r_first, L[seq])
            seq_rows = np.concatenate([np.arange(P), P + seq * R + np.arange(R)])
            nvalid = P + L[seq]
        if len(qrows) == 0:
            continue
        kk = k[seq_rows, c, :].astype(np.float64)
        vv = v[seq_rows, c, :].astype(np.float64)
        # logical positions of this sequence's key rows and of the queries
        kpos = np.arange(len(seq_rows))
        qpos = qrows if seq < 0 else P + (qrows - P - seq * R)
        # which of the wanted key rows live in this sequence, at which index
        local = [(a, int(np.searchsorted(seq_rows, j))) for a, j in enumerate(rows)
                 if (j < P) or (seq >= 0 and seq_of(j) == seq)]
        if not local:
            continue
        sel = np.array([li for _, li in local])
        for h in range(c * g, (c + 1) * g):
            for a0 in range(0, len(qrows), chunk):
                qi = qrows[a0:a0 + chunk]
                pi = qpos[a0:a0 + chunk]
                s = scale * (q[qi, h, :].astype(np.float64) @ kk.T)
                vis = (kpos[None, :] <= pi[:, None]) & (kpos[None, :] < nvalid)
                if window > 0:
                    vis &= (pi[:, None] - kpos[None, :]) < window
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)
                lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
                p = np.exp(s - lse[:, None])
                o = p @ vv
                dd = do[qi, h, :].astype(np.float64)
                delta = (dd * o).sum(axis=1)
                psel = p[:, sel]
                dpsel = dd @ vv[sel].T
                dssel = psel * (dpsel - delta[:, None])
                qq = q[qi, h, :].astype(np.float64)
                dk[[a for a, _ in local]] += scale * (dssel.T @ qq)
                dv[[a for a, _ in local]] += psel.T @ dd
    return dict(dk=dk, dv=dv)
