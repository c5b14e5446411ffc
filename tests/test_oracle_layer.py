"""Pins of the layer oracle (oracle.layer), CPU only.

 * the replicated fold equals the packed route (token-wise steps once per
   packed row, RoPE at logical positions, dense masked attention): two
   computations that share only the token-wise formulas;
 * finite differences of <Y, dY> for dX (prompt and response rows) and for
   one entry of every weight;
 * RoPE and SiLU: hand-worked values (tests/golden/rope_silu_example.json)
   that fix the frequency exponent, the (i, i + D/2) pairing and the sense
   of rotation;
 * RoPE: position 0 is the identity, the inverse undoes it, pair norms are
   kept, and rotated scores depend only on the difference of positions;
 * RMSNorm: invariant to scaling a row (eps -> 0); a constant row maps to
   the weights;
 * SwiGLU backward against finite differences.
"""
import json
import os

import numpy as np
import pytest

from oracle import layer as ol

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_silu_example.json")

Hq, Hkv, D, Hm, F = 4, 2, 8, 16, 24


def weights(seed):
    rng = np.random.default_rng(seed)
    s = lambda *sh: rng.standard_normal(sh) / np.sqrt(sh[0])
    return {"norm1": 1 + 0.1 * rng.standard_normal(Hm), "wq": s(Hm, Hq * D), "wk": s(Hm, Hkv * D),
            "wv": s(Hm, Hkv * D), "wo": s(Hq * D, Hm), "norm2": 1 + 0.1 * rng.standard_normal(Hm),
            "w1": s(Hm, F), "w3": s(Hm, F), "w2": s(F, Hm)}


CASES = [
    (((2, 3, 2),), 0, None),
    (((2, 4, 3), (3, 0, 2), (1, 2, 0)), 3, None),
    (((3, 3, 3),), 0, [3, 1, 0]),
]


def data(groups, seed):
    rng = np.random.default_rng(seed)
    T = sum(P + N * R for N, P, R in groups)
    return rng.standard_normal((T, Hm)), rng.standard_normal((T, Hm))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fold_equals_packed_route(case):
    groups, W_, vl = CASES[case]
    W = weights(case)
    x, dy = data(groups, 10 + case)
    a = ol.layer_fold(x, W, dy, groups, Hq, Hkv, W_, 1e4, 1e-6, vl)
    b = ol.packed_dense_layer(x, W, dy, groups, Hq, Hkv, W_, 1e4, 1e-6, vl)
    np.testing.assert_allclose(a["y"], b["y"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(a["dx"], b["dx"], rtol=0, atol=1e-10)
    for n in ol.NAMES:
        np.testing.assert_allclose(a["grads"][n], b["grads"][n], rtol=0, atol=1e-10, err_msg=n)


def test_finite_differences():
    groups, W_, vl = CASES[1]
    W = weights(5)
    x, dy = data(groups, 6)
    res = ol.packed_dense_layer(x, W, dy, groups, Hq, Hkv, W_, 1e4, 1e-6, vl)

    def loss(x_, W2):
        return float((ol.packed_dense_layer(x_, W2, None, groups, Hq, Hkv, W_, 1e4, 1e-6, vl)["y"] * dy).sum())

    eps = 1e-6
    for t in (0, 4, x.shape[0] - 1):          # a prompt row, a response row, the last row
        for i in (0, Hm - 1):
            xp, xm = x.copy(), x.copy()
            xp[t, i] += eps
            xm[t, i] -= eps
            fd = (loss(xp, W) - loss(xm, W)) / (2 * eps)
            assert abs(fd - res["dx"][t, i]) <= 1e-6 * max(1, abs(fd)), (t, i, fd, res["dx"][t, i])
    for n in ol.NAMES:
        idx = (1,) if W[n].ndim == 1 else (1, 2)
        Wp = {k: v.copy() for k, v in W.items()}
        Wm = {k: v.copy() for k, v in W.items()}
        Wp[n][idx] += eps
        Wm[n][idx] -= eps
        fd = (loss(x, Wp) - loss(x, Wm)) / (2 * eps)
        assert abs(fd - res["grads"][n][idx]) <= 1e-6 * max(1, abs(fd)), (n, fd, res["grads"][n][idx])


def test_rope_properties():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 2, 8))
    np.testing.assert_allclose(ol.rope(x, np.zeros(5), 1e4), x, atol=0)
    pos = np.array([0, 3, 17, 1000, 65535])
    y = ol.rope(x, pos, 1e4)
    np.testing.assert_allclose(ol.rope(y, pos, 1e4, inverse=True), x, atol=1e-12)
    nx = x[..., :4] ** 2 + x[..., 4:] ** 2
    ny = y[..., :4] ** 2 + y[..., 4:] ** 2
    np.testing.assert_allclose(ny, nx, atol=1e-12)
    q, k = rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 1, 8))
    def score(pq, pk):
        return float((ol.rope(q, [pq], 1e4) * ol.rope(k, [pk], 1e4)).sum())
    for shift in (1, 50, 4000):
        assert abs(score(10 + shift, 4 + shift) - score(10, 4)) < 1e-9
    assert abs(score(10, 4) - score(10, 5)) > 1e-3


def test_rmsnorm_properties():
    rng = np.random.default_rng(4)
    x, w = rng.standard_normal((3, 16)), rng.standard_normal(16)
    a, _ = ol.rmsnorm(x, w, 1e-12)
    b, _ = ol.rmsnorm(7.5 * x, w, 1e-12)
    np.testing.assert_allclose(a, b, atol=1e-9)
    c, _ = ol.rmsnorm(np.full((1, 16), -2.0), w, 0.0)
    np.testing.assert_allclose(c[0], -w, atol=1e-12)


def test_swiglu_backward_by_finite_differences():
    rng = np.random.default_rng(5)
    u, g, dm = rng.standard_normal(6), rng.standard_normal(6), rng.standard_normal(6)
    du, dg = ol.swiglu_bwd(u, g, dm)
    e = 1e-6
    fu = ((ol.silu(u + e) * g - ol.silu(u - e) * g) / (2 * e)) * dm
    fg = ((ol.silu(u) * (g + e) - ol.silu(u) * (g - e)) / (2 * e)) * dm
    np.testing.assert_allclose(du, fu, atol=1e-8)
    np.testing.assert_allclose(dg, fg, atol=1e-8)


def test_rope_and_silu_golden_values():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    for case in g["rope"]:
        x = np.asarray(case["x"], dtype=np.float64)[None]          # [1, H, D]
        y = ol.rope(x, [case["pos"]], case["base"])
        np.testing.assert_allclose(y[0], np.asarray(case["y"]), rtol=0, atol=1e-14)
    u = np.asarray(g["silu"]["u"])
    np.testing.assert_allclose(ol.silu(u), np.asarray(g["silu"]["y"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("mistake", ["interleaved", "exponent", "sense"])
def test_rope_golden_catches_planted_mistakes(mistake):
    """Each plausible misreading of the rotation, planted in a copy of the
    oracle's formula, misses the golden values."""
    with open(GOLDEN) as fh:
        case = json.load(fh)["rope"][0]
    x = np.asarray(case["x"], dtype=np.float64)
    D = x.shape[1]
    half = D // 2
    i = np.arange(half)
    inv = case["base"] ** (-(i if mistake == "exponent" else 2.0 * i) / D)
    ang = case["pos"] * inv
    c, s = np.cos(ang), np.sin(ang)
    if mistake == "sense":
        s = -s
    if mistake == "interleaved":
        a, b = x[:, 0::2], x[:, 1::2]
        y = np.empty_like(x)
        y[:, 0::2], y[:, 1::2] = a * c - b * s, a * s + b * c
    else:
        a, b = x[:, :half], x[:, half:]
        y = np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    assert np.abs(y - np.asarray(case["y"])).max() > 1e-3
