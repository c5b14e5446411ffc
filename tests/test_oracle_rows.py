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
