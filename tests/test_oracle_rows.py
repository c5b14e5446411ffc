"""The sampled-row oracle equals the full replicated oracle on the rows it
evaluates (it is the same definition restricted to those rows)."""
import numpy as np
import pytest

from oracle import replicated, rows


@pytest.mark.parametrize("N,P,R,Hq,Hkv,D,W,L", [
    (3, 11, 7, 4, 2, 8, 0, None), (2, 9, 6, 2, 1, 4, 5, [6, 2]), (4, 0, 5, 2, 2, 4, 0, [5, 0, 3, 1]),
    (2, 13, 0, 2, 1, 4, 0, None), (3, 6, 6, 6, 3, 4, 4, None),
])
def test_rows_match_full_oracle(N, P, R, Hq, Hkv, D, W, L):
    rng = np.random.default_rng(42)
    T = P + N * R
    q, do = rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hq, D))
    k, v = rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    full = replicated.replicated_fold(q, k, v, do, N, P, R, W, None, L)
    sample = sorted(set(rng.integers(0, T, size=min(T, 9)).tolist() + [0, T - 1]))
    got = rows.query_rows(q, k, v, do, sample, N, P, R, W, None, L)
    np.testing.assert_allclose(got["o"], full["o"][sample], atol=1e-13)
    np.testing.assert_array_equal(np.isinf(got["lse"]), np.isinf(full["lse"][:, sample]))
    fin = np.isfinite(got["lse"])
    np.testing.assert_allclose(got["lse"][fin], full["lse"][:, sample][fin], atol=1e-13)
    np.testing.assert_allclose(got["dq"], full["dq"][sample], atol=1e-12)
    for c in range(Hkv):
        kr = rows.key_rows(q, k, v, do, sample, c, N, P, R, W, None, L, chunk=5)
        np.testing.assert_allclose(kr["dk"], full["dk"][sample, c], atol=1e-12)
        np.testing.assert_allclose(kr["dv"], full["dv"][sample, c], atol=1e-12)


@pytest.mark.parametrize("N,P,R,Hq,Hkv,D,W,L", [
    (3, 40, 12, 4, 2, 8, 9, None), (2, 30, 20, 2, 1, 4, 25, [20, 7]), (4, 17, 9, 2, 2, 4, 1, None),
    (2, 64, 16, 4, 1, 8, 70, [16, 3]),
])
def test_windowed_key_rows_near_the_boundary(N, P, R, Hq, Hkv, D, W, L):
    """Prompt keys around P - W and P - 1 (seen by the prompt's own queries
    and by the first W - 1 - (P - 1 - j) queries of each response) and the
    first response keys: the restricted evaluation equals the full oracle."""
    rng = np.random.default_rng(7)
    T = P + N * R
    q, do = rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hq, D))
    k, v = rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    full = replicated.replicated_fold(q, k, v, do, N, P, R, W, None, L)
    want = sorted({j for j in (0, P // 2, P - W - 1, P - W, P - W + 1, P - 2, P - 1, P, P + 1, P + R,
                               T - 1) if 0 <= j < T})
    for c in range(Hkv):
        kr = rows.key_rows(q, k, v, do, want, c, N, P, R, W, None, L, chunk=7)
        np.testing.assert_allclose(kr["dk"], full["dk"][want, c], atol=1e-12)
        np.testing.assert_allclose(kr["dv"], full["dv"][want, c], atol=1e-12)


def test_zero_do_rows_are_skipped_exactly():
    """With dO zero outside one query head and a subset of responses (the
    input of the masked full-size check), the restricted evaluation equals
    the full oracle on the same dO, and the other KV head's gradients are
    exactly zero in the full oracle."""
    N, P, R, Hq, Hkv, D = 5, 23, 11, 4, 2, 8
    rng = np.random.default_rng(8)
    T = P + N * R
    q, do = rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hq, D))
    k, v = rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    keep_h = 3
    do[:, [h for h in range(Hq) if h != keep_h]] = 0.0
    for n in (1, 3):
        do[P + n * R:P + (n + 1) * R] = 0.0
    full = replicated.replicated_fold(q, k, v, do, N, P, R)
    assert np.all(full["dk"][:, 0] == 0.0) and np.all(full["dv"][:, 0] == 0.0)
    want = [0, 5, P - 1, P, P + 2 * R + 4, T - 1]
    kr = rows.key_rows(q, k, v, do, want, 1, N, P, R, chunk=6)
    np.testing.assert_allclose(kr["dk"], full["dk"][want, 1], atol=1e-12)
    np.testing.assert_allclose(kr["dv"], full["dv"][want, 1], atol=1e-12)
