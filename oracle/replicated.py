"""O2: replicated sequences + fold (the graded oracle).

Source: "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422),
Abstract.  Standard attention on N sequences [prompt; response n] repeats
the shared prompt N times; the method removes that repetition and is
exactly equal to it.  So the oracle materialises the N replicated causal
sequences, runs plain softmax attention and its analytic backward on each
in fp64, and maps the result back onto the packed P+NR rows:

* forward outputs of prompt rows come from copy 0 (prompt rows do not see
  any response, so all copies agree; ``prompt_spread`` reports the largest
  difference seen, the invariance the abstract relies on);
* the packed map is  packed -> broadcast prompt -> N sequences -> select
  rows, so its vector-Jacobian product gives the prompt rows of dO to
  copy 0 only and sums the prompt rows of dQ, dK, dV over the N copies
  (ascending n).  Handing the prompt dO to every copy would count the
  prompt-query term N times.

Query rows are processed in chunks of ``chunk`` rows only to bound
memory; each row's softmax is independent, and dK/dV accumulate over
chunks in ascending row order.  Every chunk scores against all keys
[0, end of chunk) under the mask.

Conventions as in ``oracle.dense`` (GQA h // g, natural-log LSE of scaled
scores, empty rows O = 0 / LSE = -inf, padded rows masked as queries and
keys, window W keeps 0 <= i - j < W).

``delta_o="bf16"`` evaluates the backward as a function of a forward output
stored in bfloat16: Delta = rowsum(dO * O) takes O rounded to bf16 (round
to nearest, ties to even, via fp32), the value a bf16 forward hands to the
backward; everything else stays fp64.  Used only to separate that rounding
from kernel error on inputs where a near one-hot softmax amplifies it.

TEST INFRASTRUCTURE ONLY.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x):
    """fp64 -> fp32 -> bfloat16 (nearest, ties to even), returned as fp64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def causal_sequence(q, k, v, do, n_valid, window=0, scale=None, chunk=1024,
                    kv_heads=None, backward=True, delta_o=None):
    """Standard causal attention on one sequence, forward and backward.

    q, do: [S, Hq, D]; k, v: [S, Hkv, D] (fp64).  Rows >= n_valid are
    padding.  Returns dict(o, lse, dq, dk, dv); heads outside ``kv_heads``
    (a subset of KV heads, default all) are left at zero / -inf.
    """
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if kv_heads is None:
        kv_heads = range(Hkv)
    o = np.zeros((S, Hq, D))
    lse = np.full((Hq, S), -np.inf)
    dq = np.zeros((S, Hq, D)) if backward else None
    dk = np.zeros((S, Hkv, D)) if backward else None
    dv = np.zeros((S, Hkv, D)) if backward else None
    for c in kv_heads:
        for h in range(c * g, (c + 1) * g):
            for a in range(0, S, chunk):
                b = min(S, a + chunk)
                i = np.arange(a, b)[:, None]
                j = np.arange(b)[None, :]
                vis = (j <= i) & (i < n_valid) & (j < n_valid)
                if window > 0:
                    vis &= (i - j) < window
                s = scale * (q[a:b, h, :] @ k[:b, c, :].T)
                s = np.where(vis, s, -np.inf)
                has = vis.any(axis=1)
                m = np.where(has, s.max(axis=1), 0.0)
                lsum = np.exp(s - m[:, None]).sum(axis=1)
                lse_c = np.where(has, m + np.log(np.where(has, lsum, 1.0)), -np.inf)
                p = np.exp(s - np.where(has, lse_c, 0.0)[:, None])   # masked -> 0
                o_c = p @ v[:b, c, :]
                o[a:b, h, :] = o_c
                lse[h, a:b] = lse_c
                if backward:
                    o_d = round_bf16(o_c) if delta_o == "bf16" else o_c
                    delta = (do[a:b, h, :] * o_d).sum(axis=1)
                    dp = do[a:b, h, :] @ v[:b, c, :].T
                    ds = p * (dp - delta[:, None])
                    dq[a:b, h, :] = scale * (ds @ k[:b, c, :])
                    dk[:b, c, :] += scale * (ds.T @ q[a:b, h, :])
                    dv[:b, c, :] += p.T @ do[a:b, h, :]
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def sequence_rows(n: int, N: int, P: int, R: int) -> np.ndarray:
    """Packed rows that make up replicated sequence n: [prompt; response n]."""
    return np.concatenate([np.arange(P), P + n * R + np.arange(R)]).astype(np.int64)


def replicated_fold(q, k, v, do, N, P, R, window=0, scale=None, valid_len=None,
                    kv_heads=None, responses=None, chunk=1024, backward=True, delta_o=None):
    """Packed-layout outputs computed through the N replicated sequences.

    q, do: packed [T, Hq, D]; k, v: packed [T, Hkv, D].  Returns dict(o,
    lse, dq, dk, dv, prompt_spread) in fp64 on the packed rows.
    ``responses`` (default all) restricts the run to a subset of the
    sequences; then prompt rows are complete only if that subset is all N
    (used for bounded timing samples).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if backward:
        do = np.asarray(do, dtype=np.float64)
    L = [R] * N if valid_len is None else [int(x) for x in valid_len]
    if responses is None:
        responses = range(N)
    out = dict(o=np.zeros((T, Hq, D)), lse=np.full((Hq, T), -np.inf))
    if backward:
        out.update(dq=np.zeros((T, Hq, D)), dk=np.zeros((T, Hkv, D)), dv=np.zeros((T, Hkv, D)))
    spread = 0.0
    first = True
    for n in responses:
        idx = sequence_rows(n, N, P, R)
        don = None
        if backward:
            don = do[idx].copy()
            if n != 0:
                don[:P] = 0.0          # prompt dO belongs to copy 0 only
        res = causal_sequence(q[idx], k[idx], v[idx], don, P + L[n], window, scale,
                              chunk, kv_heads, backward, delta_o)
        rs = slice(P + n * R, P + (n + 1) * R)
        if first:
            out["o"][:P] = res["o"][:P]
            out["lse"][:, :P] = res["lse"][:, :P]
            first = False
        else:
            d = np.abs(res["o"][:P] - out["o"][:P])
            spread = max(spread, float(d.max()) if d.size else 0.0)
        out["o"][rs] = res["o"][P:]
        out["lse"][:, rs] = res["lse"][:, P:]
        if backward:
            for name in ("dq", "dk", "dv"):
                out[name][:P] += res[name][:P]     # fold, ascending n
                out[name][rs] = res[name][P:]
    out["prompt_spread"] = spread
    return out
