"""Parity at the full layer sizes, in the launch configuration bench.py times.

The oracle cannot afford whole tensors at these sizes, so each case checks
 * sampled query rows (prompt start/middle/end, response starts and ends,
   padded rows): O, LSE and dQ against the oracle's definition of those rows;
 * sampled response key rows of two KV heads: dK, dV;
 * sampled prompt key rows (start, middle, around P - W under a window, end):
   dK, dV summed over the prompt's own queries and every response.  Where
   the oracle can afford every query head of the group, against the main
   run; otherwise a second backward with dO kept on one query head only
   (dO zero elsewhere, so every other head and KV head must come out
   exactly zero) is checked against the oracle on that same dO;
 * identities over every row: sum_j dK_j = 0 and sum_j dV_j = sum of dO over
   the group's valid query rows, per KV head and dim; <Q,dQ> = <K,dK> and
   <V,dV> = <O,dO>.
Inputs are the seeded workloads themselves (value scale 0.5), so the
elementwise gate is the localised-fault detector of parity_utils.
"""
import time

import numpy as np
import pytest
import torch

import shared_prompt_exact_amd as dk
import workloads
from oracle import rows as orows

import parity_utils
from parity_utils import check, inputs_on_device

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]

NAMES = ["qwen3_8b", "dapo_long", "moe_30b", "gemma_global", "gemma_swa"]
PROMPT_KEY_BUDGET = 2.5e9    # oracle score elements for the prompt-key check (all heads of a group)


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, flush=True)


def sample_query_rows(w, L):
    N, P, R = w.n_resp, w.prompt_len, w.resp_len
    rows = {0, 1, P // 2, P - 1} if P else set()
    for n in sorted({0, N // 2, N - 1}):
        base = P + n * R
        for r in {0, 1, max(0, L[n] - 1), min(R - 1, L[n]), R - 1}:
            rows.add(base + r)
    return sorted(x for x in rows if 0 <= x < P + N * R)


KEY_ROW_BUDGET = 4e10        # oracle multiply-adds for sampled response key rows


def sample_key_rows(w, L, n):
    """Key rows of response n: early ones only while the oracle can afford
    every later query of the response seeing them."""
    P, R, D = w.prompt_len, w.resp_len, w.head_dim
    g = w.n_q_heads // w.n_kv_heads
    base = P + n * R
    out = []
    for r in (0, L[n] // 2, L[n] - 64, L[n] - 1):
        if r < 0 or r >= L[n]:
            continue
        cost = (L[n] - r) * (P + L[n]) * g * D * 4
        if cost <= KEY_ROW_BUDGET:
            out.append(base + r)
    return sorted(set(out))


def prompt_key_rows(w):
    P, W = w.prompt_len, w.window
    cand = {0, 1, P // 2, P - 64, P - 2, P - 1}
    if W > 0:
        cand |= {P - W - 1, P - W, P - W + 1, P - W // 2}
    return sorted(j for j in cand if 0 <= j < P)


def score_elements(w, L, keys):
    """(query, key) scores the row oracle evaluates for prompt key rows
    `keys`, per query head: each query that sees one of them scores its
    whole visible range."""
    P, W = w.prompt_len, w.window
    pos = np.arange(P + max(L, default=0))
    see = np.zeros(len(pos), dtype=bool)
    for kp in keys:
        see |= (pos >= kp) & ((pos < kp + W) if W > 0 else True)
    span = np.minimum(pos + 1, W) if W > 0 else pos + 1
    prompt = int(span[:P][see[:P]].sum())
    resp = sum(int(span[P:P + l][see[P:P + l]].sum()) for l in L)
    return prompt + resp


def dot64(a, b, rows=4096):
    """sum(a * b) in fp64, in row chunks (a, b: float32 arrays)."""
    t = 0.0
    for i in range(0, a.shape[0], rows):
        t += float(np.einsum("thd,thd->", a[i:i + rows].astype(np.float64), b[i:i + rows].astype(np.float64)))
    return t


def host32(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("name", NAMES)
def test_full_size_layer(name):
    w = workloads.WORKLOADS[name]
    N, P, R = w.n_resp, w.prompt_len, w.resp_len
    log(f"{name}: generating inputs")
    x = workloads.generate(w)
    L = [R] * N if x.valid_len is None else [int(a) for a in x.valid_len]
    d = inputs_on_device(w, x)
    kw = dict(window=w.window, valid_len=d["valid"])
    log(f"{name}: forward + backward on the GPU")
    o, lse = dk.dualkv_fwd(d["q"], d["k"], d["v"], N, P, R, **kw)
    dq, dkk, dv = dk.dualkv_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], N, P, R, **kw)
    torch.cuda.synchronize()
    O, LSE, DQ, DK, DV = (host32(t) for t in (o, lse, dq, dkk, dv))
    del dq, dkk, dv
    torch.cuda.empty_cache()

    # sampled query rows
    qr = sample_query_rows(w, L)
    log(f"{name}: oracle on {len(qr)} query rows")
    ref = orows.query_rows(x.q, x.k, x.v, x.do, qr, N, P, R, w.window, None, x.valid_len)
    for nm, got, want in (("o", O[qr], ref["o"]), ("lse", LSE[:, qr], ref["lse"]),
                          ("dq", DQ[qr], ref["dq"])):
        log(f"  {nm}: rel-L2 %.2e max-abs %.2e" % check(nm, got, want, w.dtype, False, local_fault=parity_utils.FULL_SIZE_LOCAL_FAULT.get(nm, parity_utils.LOCAL_FAULT)) + " local %.2e" % parity_utils.LAST_LOCAL[0])

    # sampled response key rows, first and last KV head
    kr = sorted(set(sample_key_rows(w, L, 0) + sample_key_rows(w, L, N - 1)))
    for c in sorted({0, w.n_kv_heads - 1}):
        log(f"{name}: oracle on response key rows {kr}, KV head {c}")
        ref = orows.key_rows(x.q, x.k, x.v, x.do, kr, c, N, P, R, w.window, None, x.valid_len)
        for nm, got, want in (("dk", DK[kr, c], ref["dk"]), ("dv", DV[kr, c], ref["dv"])):
            log(f"  {nm}: rel-L2 %.2e max-abs %.2e" % check(nm, got, want, w.dtype, False, local_fault=parity_utils.FULL_SIZE_LOCAL_FAULT.get(nm, parity_utils.LOCAL_FAULT)) + " local %.2e" % parity_utils.LAST_LOCAL[0])

    # sampled prompt key rows: the sum over the prompt's queries and all N
    # responses
    pk = prompt_key_rows(w)
    g = w.n_q_heads // w.n_kv_heads
    if pk:
        cost = score_elements(w, L, pk)
        if cost * g <= PROMPT_KEY_BUDGET:
            c = w.n_kv_heads - 1
            log(f"{name}: oracle on prompt key rows {pk}, KV head {c}, all {g} query heads ({cost * g:.2e} scores)")
            ref = orows.key_rows(x.q, x.k, x.v, x.do, pk, c, N, P, R, w.window, None, x.valid_len)
            for nm, got, want in (("dk", DK[pk, c], ref["dk"]), ("dv", DV[pk, c], ref["dv"])):
                log(f"  {nm}: rel-L2 %.2e max-abs %.2e" % check(nm, got, want, w.dtype, False, local_fault=parity_utils.FULL_SIZE_LOCAL_FAULT.get(nm, parity_utils.LOCAL_FAULT)) + " local %.2e" % parity_utils.LAST_LOCAL[0])
        else:
            h1 = w.n_q_heads - 1
            c = h1 // g
            log(f"{name}: backward with dO on query head {h1} only")
            do1 = torch.zeros_like(d["do"])
            do1[:, h1] = d["do"][:, h1]
            dq1, dk1, dv1 = dk.dualkv_bwd(d["q"], d["k"], d["v"], o, lse, do1, N, P, R, **kw)
            torch.cuda.synchronize()
            others = [h for h in range(w.n_q_heads) if h != h1]
            assert bool((dq1[:, others] == 0).all()), "dQ of heads without dO must be exactly 0"
            assert bool((dk1[:, :c] == 0).all()) and bool((dv1[:, :c] == 0).all()), \
                "dK/dV of KV heads without dO must be exactly 0"
            DK1, DV1 = host32(dk1[pk, c]), host32(dv1[pk, c])
            del do1, dq1, dk1, dv1
            xdo = np.zeros_like(x.do)
            xdo[:, h1] = x.do[:, h1]
            log(f"{name}: oracle on prompt key rows {pk}, KV head {c}, query head {h1} ({cost:.2e} scores)")
            ref = orows.key_rows(x.q, x.k, x.v, xdo, pk, c, N, P, R, w.window, None, x.valid_len)
            del xdo
            for nm, got, want in (("dk", DK1, ref["dk"]), ("dv", DV1, ref["dv"])):
                log(f"  {nm}: rel-L2 %.2e max-abs %.2e" % check(nm, got, want, w.dtype, False, local_fault=parity_utils.FULL_SIZE_LOCAL_FAULT.get(nm, parity_utils.LOCAL_FAULT)) + " local %.2e" % parity_utils.LAST_LOCAL[0])
    del d, o, lse
    torch.cuda.empty_cache()

    # identities over all rows (fp64 sums of the GPU outputs)
    log(f"{name}: identities")
    T = P + N * R
    live = np.isfinite(LSE)                                  # [Hq, T]
    for c in range(w.n_kv_heads):
        dkc = DK[:, c].astype(np.float64)
        sk = dkc.sum(0)
        scale_k = np.sqrt(T) * np.sqrt(np.mean(dkc ** 2))
        assert np.abs(sk).max() <= 0.02 * scale_k, (c, np.abs(sk).max(), scale_k)
        want = sum(x.do[live[h], h].astype(np.float64).sum(0) for h in range(c * g, (c + 1) * g))
        dvc = DV[:, c].astype(np.float64)
        sv = dvc.sum(0)
        scale_v = np.sqrt(T) * np.sqrt(np.mean(dvc ** 2))
        assert np.abs(sv - want).max() <= 0.02 * scale_v, (c, np.abs(sv - want).max(), scale_v)
    qdq, kdk = dot64(x.q, DQ), dot64(x.k, DK)
    vdv, odo = dot64(x.v, DV), dot64(O, x.do)
    assert abs(qdq - kdk) <= 1e-2 * max(abs(qdq), abs(kdk), 1e-6), (qdq, kdk)
    assert abs(vdv - odo) <= 1e-2 * max(abs(vdv), abs(odo), 1e-6), (vdv, odo)
    log(f"{name}: ok")
