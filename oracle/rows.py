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
  Queries that cannot see a wanted key, or whose dO is zero, add nothing
  and are left out.

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
    """Return dict(dk [n,D], dv [n,D]) of packed key rows `rows` of one KV head.

    Work is limited to what can reach the wanted keys, which leaves the
    result unchanged:
     * per sequence, only queries whose visible range [p-W+1, p] holds one
       of the wanted key positions;
     * a query whose dO row (of that head) is all zero adds exactly zero to
       dK and dV (dp = 0 and Delta = dO . O = 0, so ds = 0), and is skipped;
     * each chunk of queries scores only the key positions any of them can
       see, [min p - W + 1, max p]; every query's softmax still covers its
       whole visible range.
    The arithmetic is fp64 (torch CPU ops, which use every host thread).
    """
    import torch

    T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    rows = [int(x) for x in rows]
    dk = np.zeros((len(rows), D))
    dv = np.zeros((len(rows), D))
    c = kv_head

    def seq_of(j):
        return -1 if j < P else (j - P) // R

    # Sequence -1 is the prompt's own queries (copy 0), n >= 0 response n;
    # every response sees the prompt keys.
    wanted = set(seq_of(j) for j in rows)
    if -1 in wanted:
        wanted |= set(range(N))
    for seq in sorted(wanted):
        if seq < 0:
            seq_rows = np.arange(P)
            nvalid = P
            qrows_all = np.arange(P)
            qpos_all = np.arange(P)
            local = [(a, j) for a, j in enumerate(rows) if j < P]
        else:
            seq_rows = np.concatenate([np.arange(P), P + seq * R + np.arange(R)])
            nvalid = P + L[seq]
            qrows_all = P + seq * R + np.arange(L[seq])
            qpos_all = P + np.arange(L[seq])
            local = [(a, j if j < P else P + (j - P - seq * R)) for a, j in enumerate(rows)
                     if j < P or seq_of(j) == seq]
        # wanted keys past the sequence's valid range are seen by nothing
        local = [(a, kp) for a, kp in local if kp < nvalid]
        if not local:
            continue
        out_idx = np.array([a for a, _ in local])
        kps = np.array([kp for _, kp in local])
        see = np.zeros(len(qpos_all), dtype=bool)
        for kp in np.unique(kps):                # queries at [kp, kp + W) see key kp
            band = qpos_all >= kp
            if window > 0:
                band &= qpos_all < kp + window
            see |= band
        qrows_s, qpos_s = qrows_all[see], qpos_all[see]
        if len(qrows_s) == 0:
            continue
        kk_all = torch.from_numpy(np.ascontiguousarray(k[seq_rows, c, :], dtype=np.float64))
        vv_all = torch.from_numpy(np.ascontiguousarray(v[seq_rows, c, :], dtype=np.float64))
        for h in range(c * g, (c + 1) * g):
            live = np.any(do[qrows_s, h, :] != 0, axis=1)
            qr, qp = qrows_s[live], qpos_s[live]
            # chunks of at most `chunk` queries inside runs of consecutive
            # positions (a chunk's key range stays one query's range + chunk)
            cuts = np.flatnonzero(np.diff(qp) != 1) + 1
            starts = []
            for r0, r1 in zip(np.r_[0, cuts], np.r_[cuts, len(qp)]):
                starts += [(a, min(a + chunk, r1)) for a in range(r0, r1, chunk)]
            for a0, a1 in starts:
                qi, pi = qr[a0:a1], qp[a0:a1]
                lo = max(0, int(pi.min()) - window + 1) if window > 0 else 0
                hi = int(pi.max()) + 1                       # key positions [lo, hi)
                kk, vv = kk_all[lo:hi], vv_all[lo:hi]
                kpos = torch.arange(lo, hi, dtype=torch.int64)
                pt = torch.from_numpy(pi.astype(np.int64))
                qq = torch.from_numpy(np.ascontiguousarray(q[qi, h, :], dtype=np.float64))
                dd = torch.from_numpy(np.ascontiguousarray(do[qi, h, :], dtype=np.float64))
                s = (qq @ kk.T) * scale
                vis = (kpos[None, :] <= pt[:, None]) & (kpos[None, :] < nvalid)
                if window > 0:
                    vis &= (pt[:, None] - kpos[None, :]) < window
                s.masked_fill_(~vis, float("-inf"))
                m = s.max(dim=1).values
                s.sub_(m[:, None]).exp_()                    # unnormalised p
                s.div_(s.sum(dim=1, keepdim=True))           # p
                o = s @ vv
                delta = (dd * o).sum(dim=1)
                inr = (kps >= lo) & (kps < hi)
                if not inr.any():
                    continue
                sel = torch.from_numpy(kps[inr] - lo)
                psel = s[:, sel]
                dssel = psel * (dd @ vv[sel].T - delta[:, None])
                dk[out_idx[inr]] += scale * (dssel.T @ qq).numpy()
                dv[out_idx[inr]] += (psel.T @ dd).numpy()
    return dict(dk=dk, dv=dv)
