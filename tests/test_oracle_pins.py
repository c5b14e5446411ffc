"""Pins of the fp64 oracle against facts that do not come from the oracle.

The method ("DualKV: Shared-Prompt Flash Attention ...", arXiv 2605.15422,
Abstract) is exactly equal to standard causal softmax attention over the
N replicated sequences.  Each test below pins one part of the oracle to
something independent of it: a hand-worked example, closed forms, torch's
own attention routine (fp64, CPU), finite differences, or identities that
hold for any softmax attention.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dense, replicated
from oracle.mask import count_visible_pairs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, T, Hq, Hkv, D):
    return (rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)),
            rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hq, D)))


def _expr(s):
    """Evaluate a fixture expression made of fractions, + - * and log()."""
    return float(eval(s, {"__builtins__": {}}, {"log": math.log, "F": Fraction}))


# ---------------------------------------------------------------- hand example

def test_hand_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    N, P, R, scale = fx["N"], fx["P"], fx["R"], fx["scale"]
    arr = lambda key: np.array([_expr(s) for s in fx[key]]).reshape(-1, 1, 1)
    q, k, v, do = arr("q"), arr("k"), arr("v"), arr("do")
    for run in ("dense", "replicated"):
        if run == "dense":
            o, lse = dense.forward(q, k, v, N, P, R, 0, scale)
            dq, dk, dv = dense.backward(q, k, v, o, lse, do, N, P, R, 0, scale)
        else:
            r = replicated.replicated_fold(q, k, v, do, N, P, R, 0, scale)
            o, lse, dq, dk, dv = r["o"], r["lse"], r["dq"], r["dk"], r["dv"]
        np.testing.assert_allclose(o.ravel(), arr("o").ravel(), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse.ravel(), arr("lse").ravel(), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dq.ravel(), arr("dq").ravel(), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk.ravel(), arr("dk").ravel(), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dv.ravel(), arr("dv").ravel(), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- closed form, Q = 0

CASES = [
    # N, P, R, window, valid lengths
    (3, 7, 5, 0, None),
    (2, 9, 6, 4, None),          # window reaches across the prompt/response boundary
    (4, 5, 6, 3, [6, 0, 2, 5]),  # window + valid lengths, one empty response
    (3, 0, 4, 0, [4, 1, 3]),     # no prompt: independent causal sequences
    (2, 6, 0, 0, None),          # no responses: causal attention on the prompt
    (1, 4, 3, 1, None),          # window 1: each token sees only itself
]


@pytest.mark.parametrize("N,P,R,W,L", CASES)
def test_zero_query_closed_form(N, P, R, W, L):
    """With Q = 0 every visible score is 0: LSE_i = ln(c_i), O_i is the mean
    of the visible V rows and dK = 0.  Every visible key set is the
    contiguous range of logical positions [max(0, pos-W+1), pos], so
    c_i = min(pos_i + 1, W) for valid rows and 0 for padded rows."""
    rng = np.random.default_rng(1)
    T, Hq, Hkv, D = P + N * R, 2, 1, 3
    _, k, v, do = _rand(rng, T, Hq, Hkv, D)
    q = np.zeros((T, Hq, D))
    Ls = [R] * N if L is None else L
    # Expected values built from the logical-position ranges.
    exp_lse = np.full(T, -np.inf)
    exp_o = np.zeros((T, D))
    Wp = W if W > 0 else 10 ** 9
    for t in range(T):
        if t < P:
            pos, rows = t, list(range(t + 1))
        else:
            n, r = divmod(t - P, R)
            if r >= Ls[n]:
                continue
            pos = P + r
            rows = list(range(P)) + [P + n * R + x for x in range(r + 1)]
        lo = max(0, pos - Wp + 1)
        keep = [j for j, p in zip(rows, list(range(len(rows)))) if p >= lo]
        c = min(pos + 1, Wp)
        assert len(keep) == c
        exp_lse[t] = math.log(c)
        exp_o[t] = v[keep, 0, :].mean(axis=0)
    r = replicated.replicated_fold(q, k, v, do, N, P, R, W, 0.37, L, chunk=4)
    o1, l1 = dense.forward(q, k, v, N, P, R, W, 0.37, L)
    for o, lse in ((r["o"], r["lse"]), (o1, l1)):
        for h in range(Hq):
            np.testing.assert_array_equal(np.isinf(lse[h]), np.isinf(exp_lse))
            fin = np.isfinite(exp_lse)
            np.testing.assert_allclose(lse[h][fin], exp_lse[fin], rtol=0, atol=1e-14)
            np.testing.assert_allclose(o[:, h, :], exp_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-14)
    expected_pairs = sum(min(p + 1, Wp) for p in range(P))
    for n in range(N):
        expected_pairs += sum(min(P + x + 1, Wp) for x in range(Ls[n]))
    assert count_visible_pairs(N, P, R, W, L) == expected_pairs


# ---------------------------------------------------------------- torch SDPA (library routine)

def _sdpa(q, k, v, mask=None, causal=False, grads_of=None):
    """torch's fp64 CPU attention on [S, H, D] arrays (GQA via enable_gqa)."""
    t = lambda a: torch.tensor(a, dtype=torch.float64).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    tq, tk, tv = t(q), t(k), t(v)
    m = None if mask is None else torch.tensor(mask)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                         enable_gqa=q.shape[1] != k.shape[1])
    res = out[0].permute(1, 0, 2).detach().numpy()
    if grads_of is None:
        return res
    do = torch.tensor(grads_of, dtype=torch.float64).permute(1, 0, 2).unsqueeze(0)
    out.backward(do)
    g = lambda a: a.grad[0].permute(1, 0, 2).numpy()
    return res, g(tq), g(tk), g(tv)


@pytest.mark.parametrize("P,R,Hq,Hkv", [(7, 5, 4, 2), (0, 9, 2, 2), (6, 0, 3, 1), (16, 16, 8, 2)])
def test_single_response_is_causal_attention(P, R, Hq, Hkv):
    """N = 1: packed and replicated layouts coincide; the result is plain
    causal attention (forward and gradients from torch autograd)."""
    rng = np.random.default_rng(2)
    T, D = P + R, 8
    q, k, v, do = _rand(rng, T, Hq, Hkv, D)
    o_ref, dq_ref, dk_ref, dv_ref = _sdpa(q, k, v, causal=True, grads_of=do)
    r = replicated.replicated_fold(q, k, v, do, 1, P, R, chunk=5)
    o1, l1 = dense.forward(q, k, v, 1, P, R)
    g1 = dense.backward(q, k, v, o1, l1, do, 1, P, R)
    for o, dq, dk, dv in ((r["o"], r["dq"], r["dk"], r["dv"]), (o1,) + g1):
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dq, dq_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, dk_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, dv_ref, rtol=0, atol=1e-12)


def test_no_prompt_is_independent_sequences():
    """P = 0: every response is an independent causal sequence."""
    rng = np.random.default_rng(3)
    N, R, Hq, Hkv, D = 3, 6, 2, 1, 4
    T = N * R
    q, k, v, do = _rand(rng, T, Hq, Hkv, D)
    r = replicated.replicated_fold(q, k, v, do, N, 0, R)
    o1, _ = dense.forward(q, k, v, N, 0, R)
    for n in range(N):
        s = slice(n * R, (n + 1) * R)
        o_ref, dq_ref, dk_ref, dv_ref = _sdpa(q[s], k[s], v[s], causal=True, grads_of=do[s])
        np.testing.assert_allclose(r["o"][s], o_ref, atol=1e-13)
        np.testing.assert_allclose(o1[s], o_ref, atol=1e-13)
        np.testing.assert_allclose(r["dq"][s], dq_ref, atol=1e-12)
        np.testing.assert_allclose(r["dk"][s], dk_ref, atol=1e-12)
        np.testing.assert_allclose(r["dv"][s], dv_ref, atol=1e-12)


@pytest.mark.parametrize("W", [1, 3, 8])
def test_window_matches_banded_sdpa(W):
    """Sliding window of W positions, built for torch as a band of tril/triu."""
    rng = np.random.default_rng(4)
    N, P, R, Hq, Hkv, D = 2, 6, 5, 2, 1, 4
    q, k, v, do = _rand(rng, P + N * R, Hq, Hkv, D)
    r = replicated.replicated_fold(q, k, v, do, N, P, R, W)
    S = P + R
    ones = torch.ones(S, S, dtype=torch.bool)
    band = (torch.tril(ones) & ~torch.tril(ones, diagonal=-W)).numpy()
    for n in range(N):
        idx = replicated.sequence_rows(n, N, P, R)
        dsq = do[idx].copy()
        if n:
            dsq[:P] = 0
        o_ref, dq_ref, dk_ref, dv_ref = _sdpa(q[idx], k[idx], v[idx], mask=band, grads_of=dsq)
        np.testing.assert_allclose(r["o"][P + n * R:P + (n + 1) * R], o_ref[P:], atol=1e-13)
        np.testing.assert_allclose(r["dq"][P + n * R:P + (n + 1) * R], dq_ref[P:], atol=1e-12)
        if n == 0:
            np.testing.assert_allclose(r["o"][:P], o_ref[:P], atol=1e-13)


def test_gqa_equals_repeated_kv_heads():
    """GQA (query head h uses KV head h // g) equals MHA on KV heads repeated
    g times; the GQA dK/dV are the group sums of the MHA ones."""
    rng = np.random.default_rng(5)
    N, P, R, Hq, Hkv, D, W = 3, 5, 4, 6, 2, 4, 4
    g = Hq // Hkv
    q, k, v, do = _rand(rng, P + N * R, Hq, Hkv, D)
    a = replicated.replicated_fold(q, k, v, do, N, P, R, W)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    b = replicated.replicated_fold(q, kr, vr, do, N, P, R, W)
    np.testing.assert_allclose(a["o"], b["o"], atol=1e-14)
    np.testing.assert_allclose(a["dq"], b["dq"], atol=1e-13)
    T = P + N * R
    np.testing.assert_allclose(a["dk"], b["dk"].reshape(T, Hkv, g, D).sum(2), atol=1e-13)
    np.testing.assert_allclose(a["dv"], b["dv"].reshape(T, Hkv, g, D).sum(2), atol=1e-13)


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("N,P,R,W,L", [(3, 5, 4, 0, None), (2, 6, 5, 4, [5, 2]), (2, 0, 5, 0, [3, 5])])
def test_backward_finite_differences(N, P, R, W, L):
    """Directional derivatives of L(Q,K,V) = <dO, O> (fp64 central
    differences) equal <grad, E> for random directions E."""
    rng = np.random.default_rng(6)
    Hq, Hkv, D = 4, 2, 3
    T = P + N * R
    q, k, v, do = _rand(rng, T, Hq, Hkv, D)
    r = replicated.replicated_fold(q, k, v, do, N, P, R, W, None, L)

    def loss(qq, kk, vv):
        o = replicated.replicated_fold(qq, kk, vv, None, N, P, R, W, None, L, backward=False)["o"]
        return float((o * do).sum())

    h = 1e-6
    for _ in range(3):
        for name, grad in (("q", r["dq"]), ("k", r["dk"]), ("v", r["dv"])):
            base = {"q": q, "k": k, "v": v}
            E = rng.standard_normal(base[name].shape)
            plus = dict(base); plus[name] = base[name] + h * E
            minus = dict(base); minus[name] = base[name] - h * E
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
            an = float((grad * E).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_lse_gradient_is_attention_over_keys():
    """d LSE_i / d q_i = scale * sum_j p_ij k_j, i.e. attention output with V
    replaced by K (torch SDPA).  Pins LSE away from the Q = 0 case."""
    rng = np.random.default_rng(7)
    P, R, H, D = 5, 4, 1, 3
    T = P + R
    q, k, _, _ = _rand(rng, T, H, H, D)
    scale = 1 / math.sqrt(D)
    ref = _sdpa(q, k, k, causal=True)
    h = 1e-6
    for i in (0, P - 1, P, T - 1):
        grad = np.zeros(D)
        for d in range(D):
            qp = q.copy(); qp[i, 0, d] += h
            qm = q.copy(); qm[i, 0, d] -= h
            lp = replicated.replicated_fold(qp, k, k, None, 1, P, R, backward=False)["lse"][0, i]
            lm = replicated.replicated_fold(qm, k, k, None, 1, P, R, backward=False)["lse"][0, i]
            grad[d] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, scale * ref[i, 0], atol=1e-8)


# ---------------------------------------------------------------- identities

SWEEP = [
    (3, 5, 4, 4, 2, 8, 0, None), (2, 7, 5, 2, 1, 4, 3, [2, 5]), (1, 6, 0, 2, 2, 4, 0, None),
    (3, 0, 4, 2, 1, 4, 0, [0, 4, 1]), (4, 9, 3, 6, 3, 5, 1, None), (2, 4, 6, 4, 1, 6, 20, [6, 3]),
    (5, 3, 2, 2, 2, 3, 2, [1, 2, 0, 2, 2]),
]


@pytest.mark.parametrize("N,P,R,Hq,Hkv,D,W,L", SWEEP)
def test_sum_rules(N, P, R, Hq, Hkv, D, W, L):
    """Identities of any softmax attention, needing no reference:
    sum_j dK_j = 0 (rows of dS sum to zero); sum_j dV_j = sum of dO over
    query rows that see a key; <Q,dQ> = <K,dK> (scores depend on q.k only);
    <V,dV> = <O,dO> (O is linear in V)."""
    rng = np.random.default_rng(8)
    T = P + N * R
    q, k, v, do = _rand(rng, T, Hq, Hkv, D)
    r = replicated.replicated_fold(q, k, v, do, N, P, R, W, None, L, chunk=3)
    g = Hq // Hkv
    live = np.isfinite(r["lse"])            # [Hq, T]
    for c in range(Hkv):
        np.testing.assert_allclose(r["dk"][:, c].sum(0), 0.0, atol=1e-12)
        want = sum((do[:, h] * live[h][:, None]).sum(0) for h in range(c * g, (c + 1) * g))
        np.testing.assert_allclose(r["dv"][:, c].sum(0), want, atol=1e-12)
    assert abs((q * r["dq"]).sum() - (k * r["dk"]).sum()) < 1e-11
    assert abs((v * r["dv"]).sum() - (r["o"] * do).sum()) < 1e-11


@pytest.mark.parametrize("N,P,R,Hq,Hkv,D,W,L", SWEEP)
def test_dense_definition_equals_replicated_fold(N, P, R, Hq, Hkv, D, W, L):
    """O1 (dense packed mask) and O2 (replicated + fold) are two independent
    routes to the same numbers."""
    rng = np.random.default_rng(9)
    q, k, v, do = _rand(rng, P + N * R, Hq, Hkv, D)
    o1, l1 = dense.forward(q, k, v, N, P, R, W, None, L)
    g1 = dense.backward(q, k, v, o1, l1, do, N, P, R, W, None, L)
    r = replicated.replicated_fold(q, k, v, do, N, P, R, W, None, L, chunk=2)
    np.testing.assert_allclose(o1, r["o"], atol=1e-13)
    np.testing.assert_array_equal(np.isinf(l1), np.isinf(r["lse"]))
    np.testing.assert_allclose(l1[np.isfinite(l1)], r["lse"][np.isfinite(l1)], atol=1e-13)
    for a, name in zip(g1, ("dq", "dk", "dv")):
        np.testing.assert_allclose(a, r[name], atol=1e-12)


def test_prompt_rows_invariant_to_responses_and_N():
    """Prompt outputs (O, LSE, dQ) do not depend on the responses or on N,
    and every replicated copy computes the same prompt outputs."""
    rng = np.random.default_rng(10)
    P, R, Hq, Hkv, D = 6, 4, 2, 1, 4
    q, k, v, do = _rand(rng, P + 4 * R, Hq, Hkv, D)
    a = replicated.replicated_fold(q, k, v, do, 4, P, R)
    assert a["prompt_spread"] < 1e-15
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[P:] = rng.standard_normal(x[P:].shape)
    b = replicated.replicated_fold(q2, k2, v2, do2, 4, P, R)
    c = replicated.replicated_fold(q[:P + R], k[:P + R], v[:P + R], do[:P + R], 1, P, R)
    for other in (b, c):
        np.testing.assert_allclose(other["o"][:P], a["o"][:P], atol=1e-15)
        np.testing.assert_allclose(other["lse"][:, :P], a["lse"][:, :P], atol=1e-15)
        np.testing.assert_allclose(other["dq"][:P], a["dq"][:P], atol=1e-15)


def test_permuting_responses_permutes_rows():
    rng = np.random.default_rng(11)
    N, P, R, Hq, Hkv, D = 4, 5, 3, 2, 1, 4
    q, k, v, do = _rand(rng, P + N * R, Hq, Hkv, D)
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(P)] + [P + n * R + np.arange(R) for n in perm])
    a = replicated.replicated_fold(q, k, v, do, N, P, R)
    b = replicated.replicated_fold(q[rows], k[rows], v[rows], do[rows], N, P, R)
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(b[name], a[name][rows], atol=1e-14)
    np.testing.assert_allclose(b["lse"], a["lse"][:, rows], atol=1e-14)


def test_value_and_key_shifts():
    """V = constant row c gives O = c; K + 1c^T leaves O unchanged and adds
    scale*<q_i, c> to LSE_i; V + 1c^T adds c to O."""
    rng = np.random.default_rng(12)
    N, P, R, Hq, Hkv, D, W = 3, 5, 4, 2, 1, 4, 5
    T = P + N * R
    q, k, v, _ = _rand(rng, T, Hq, Hkv, D)
    c = rng.standard_normal(D)
    scale = 1 / math.sqrt(D)
    base = replicated.replicated_fold(q, k, v, None, N, P, R, W, backward=False)
    const = replicated.replicated_fold(q, k, np.broadcast_to(c, v.shape).copy(), None, N, P, R, W, backward=False)
    np.testing.assert_allclose(const["o"], np.broadcast_to(c, (T, Hq, D)), atol=1e-14)
    ks = replicated.replicated_fold(q, k + c, v, None, N, P, R, W, backward=False)
    np.testing.assert_allclose(ks["o"], base["o"], atol=1e-13)
    np.testing.assert_allclose(ks["lse"], base["lse"] + scale * np.einsum("thd,d->ht", q, c), atol=1e-13)
    vs = replicated.replicated_fold(q, k, v + c, None, N, P, R, W, backward=False)
    np.testing.assert_allclose(vs["o"], base["o"] + c, atol=1e-13)


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistake_dO_to_every_copy_is_caught(monkeypatch):
    """Give the prompt dO to every replicated copy (a plausible misreading of
    the fold) inside the oracle: the dV sum rule must fail."""
    rng = np.random.default_rng(13)
    N, P, R, Hq, Hkv, D = 3, 5, 4, 2, 1, 4
    q, k, v, do = _rand(rng, P + N * R, Hq, Hkv, D)
    orig = replicated.causal_sequence
    calls = []

    def mutated(qq, kk, vv, dd, *a, **kw):
        calls.append(1)
        if dd is not None and len(calls) > 1:
            dd = dd.copy()
            dd[:P] = do[:P]
        return orig(qq, kk, vv, dd, *a, **kw)

    monkeypatch.setattr(replicated, "causal_sequence", mutated)
    r = replicated.replicated_fold(q, k, v, do, N, P, R)
    want = sum(do[:, h].sum(0) for h in range(Hq))
    assert np.abs(r["dv"][:, 0].sum(0) - want).max() > 1e-3


def test_planted_mistake_window_off_by_one_is_caught(monkeypatch):
    """A window that keeps W+1 positions inside the oracle breaks the Q = 0
    closed form."""
    orig = replicated.causal_sequence

    def mutated(q, k, v, do, n_valid, window=0, *a, **kw):
        return orig(q, k, v, do, n_valid, window + 1 if window > 0 else 0, *a, **kw)

    monkeypatch.setattr(replicated, "causal_sequence", mutated)
    with pytest.raises(AssertionError):
        test_zero_query_closed_form(2, 9, 6, 4, None)


# ---------------------------------------------------------------- bf16 Delta variant

def test_round_bf16_matches_torch():
    """The oracle's own bf16 rounding equals torch's fp32 -> bfloat16 cast
    (a library routine), ties and subnormals included."""
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 1e-40, -3e-39, 0.0, 65504.0])])
    want = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(replicated.round_bf16(x), want)


def test_bf16_delta_variant():
    """delta_o='bf16' changes only Delta: the forward is identical; where O
    is exact in bf16 (V rows all equal to a bf16 constant, so O = that row)
    the backward is identical too; otherwise dQ moves by the predicted
    amount scale * sum_j p_ij (Delta_i - Delta'_i) k_j."""
    rng = np.random.default_rng(22)
    N, P, R, Hq, Hkv, D = 2, 5, 4, 2, 1, 8
    q, k, v, do = _rand(rng, P + N * R, Hq, Hkv, D)
    a = replicated.replicated_fold(q, k, v, do, N, P, R)
    b = replicated.replicated_fold(q, k, v, do, N, P, R, delta_o="bf16")
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["lse"], b["lse"])
    assert np.abs(a["dq"] - b["dq"]).max() > 0
    c = replicated.round_bf16(rng.standard_normal(D))
    vc = np.broadcast_to(c, v.shape).copy()
    a = replicated.replicated_fold(q, k, vc, do, N, P, R)
    b = replicated.replicated_fold(q, k, vc, do, N, P, R, delta_o="bf16")
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(b[name], a[name], rtol=0, atol=1e-14)
    # N = 1: dQ_i(bf16 Delta) - dQ_i = scale * (Delta_i - Delta'_i) * sum_j p_ij k_j
    q1, k1, v1, do1 = q[:P + R], k[:P + R], v[:P + R], do[:P + R]
    a = replicated.replicated_fold(q1, k1, v1, do1, 1, P, R)
    b = replicated.replicated_fold(q1, k1, v1, do1, 1, P, R, delta_o="bf16")
    ok = replicated.replicated_fold(q1, k1, k1, None, 1, P, R, backward=False)["o"]   # sum_j p_ij k_j
    d_ex = (do1 * a["o"]).sum(-1)
    d_bf = (do1 * replicated.round_bf16(a["o"])).sum(-1)
    pred = (1 / np.sqrt(D)) * (d_ex - d_bf)[..., None] * ok
    np.testing.assert_allclose(b["dq"] - a["dq"], pred, rtol=0, atol=1e-13)
