"""Pins of the rounding envelope (oracle.rounding), CPU only.

The envelope must hold the error that the documented bf16 rounding points
cause, and must stay small where the inputs are well conditioned (else the
elementwise gate that uses it would detect nothing).  Both are checked
against a plain fp64 emulation written here independently: per replicated
sequence, P = exp(s - m - a) with a random reference offset a (the running
max of a streaming kernel is not the row max), P rounded to bf16 before the
P.V product, O normalised and stored in bf16, Delta from that stored O,
dS rounded to bf16 before the dQ and dK products, P rounded to bf16 before
the dV product; everything else fp64.
"""
import numpy as np
import pytest

import workloads
from oracle import replicated, rounding

from parity_utils import MAX_ERR_BF16, STRESS, stress_modifier

rb = replicated.round_bf16


def emulate(q, k, v, do, N, P, R, rng):
    T, Hq, D = q.shape
    g = Hq // k.shape[1]
    sc = 1.0 / np.sqrt(D)
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v))}
    for n in range(N):
        idx = replicated.sequence_rows(n, N, P, R)
        qs, ks, vs, ds_ = q[idx], k[idx], v[idx], do[idx].copy()
        if n:
            ds_[:P] = 0.0
        S = len(idx)
        causal = np.tril(np.ones((S, S), dtype=bool))
        acc = {nm: np.zeros((S,) + a.shape[1:]) for nm, a in (("dq", qs), ("dk", ks), ("dv", vs))}
        for h in range(Hq):
            c = h // g
            s = np.where(causal, sc * qs[:, h] @ ks[:, c].T, -np.inf)
            m = s.max(axis=1, keepdims=True)
            a = rng.uniform(0.0, 8.0, size=(S, 1))
            e = np.exp(s - m - a)
            o = rb(rb(e) @ vs[:, c] / e.sum(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            dlt = (ds_[:, h] * o).sum(axis=1, keepdims=True)
            dsm = rb(p * (ds_[:, h] @ vs[:, c].T - dlt))
            acc["dq"][:, h] = sc * dsm @ ks[:, c]
            acc["dk"][:, c] += sc * dsm.T @ qs[:, h]
            acc["dv"][:, c] += rb(p).T @ ds_[:, h]
        rs = slice(P + n * R, P + (n + 1) * R)
        for nm in out:
            out[nm][:P] += acc[nm][:P]
            out[nm][rs] = acc[nm][P:]
    return out


def inputs(kind):
    w = STRESS
    x = workloads.generate(w)
    if kind != "plain":
        stress_modifier(kind)(w, x)
    return w, [a.astype(np.float64) for a in (x.q, x.k, x.v, x.do)]


@pytest.mark.parametrize("kind", ["peaked", "early_max", "late_max", "plain"])
def test_envelope_holds_emulated_roundings(kind):
    w, (q, k, v, do) = inputs(kind)
    N, P, R = w.n_resp, w.prompt_len, w.resp_len
    ref = replicated.replicated_fold(q, k, v, do, N, P, R, delta_o="bf16")
    env = rounding.backward_envelope(q, k, v, do, N, P, R)
    got = emulate(q, k, v, do, N, P, R, np.random.default_rng(5))
    for nm in ("dq", "dk", "dv"):
        y = ref[nm]
        d = np.abs(rb(got[nm]) - y)
        worst = (d / (MAX_ERR_BF16 * np.maximum(1.0, np.abs(y)) + env[nm])).max()
        # the tests gate at 2 * env; the emulation must fit within half of that
        assert worst <= 1.0, (kind, nm, worst)


def test_envelope_is_small_on_plain_inputs():
    """On i.i.d. inputs the envelope stays below a tenth of the RMS for all
    but a few percent of the elements (the gate still detects faults)."""
    w, (q, k, v, do) = inputs("plain")
    ref = replicated.replicated_fold(q, k, v, do, w.n_resp, w.prompt_len, w.resp_len)
    env = rounding.backward_envelope(q, k, v, do, w.n_resp, w.prompt_len, w.resp_len)
    for nm in ("dq", "dk", "dv"):
        rms = np.sqrt(np.mean(ref[nm] ** 2))
        assert np.mean(env[nm] > 0.1 * rms) < 0.05, nm


@pytest.mark.parametrize("kind", ["peaked", "early_max", "late_max"])
def test_gate_still_detects_local_faults(kind):
    """On the stress inputs the widened gate (2e-2 max(1,|y|) + 2 env) stays
    below half the RMS on most elements, so a wrong row or tile (errors of
    order RMS or |y|) is still caught.  The exception is dQ on the
    early-max input: there dQ itself (RMS 0.06) is smaller than what the
    rounding of O into Delta can move it by (one key of score 40 * 3 * 0.125
    dominates every row), so only the rel-L2 gate is informative."""
    w, (q, k, v, do) = inputs(kind)
    N, P, R = w.n_resp, w.prompt_len, w.resp_len
    ref = replicated.replicated_fold(q, k, v, do, N, P, R, delta_o="bf16")
    env = rounding.backward_envelope(q, k, v, do, N, P, R)
    for nm in ("dq", "dk", "dv"):
        if kind == "early_max" and nm == "dq":
            continue
        y = ref[nm]
        budget = MAX_ERR_BF16 * np.maximum(1.0, np.abs(y)) + 2.0 * env[nm]
        assert np.mean(budget < 0.5 * np.sqrt(np.mean(y ** 2))) > 0.8, (kind, nm)
