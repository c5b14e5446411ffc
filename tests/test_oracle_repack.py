"""Pins of the oracle's repack row maps (N(P+R) <-> P+NR)."""
import json
import os

import numpy as np
import pytest

from oracle import repack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_written_row_maps():
    fx = json.load(open(os.path.join(GOLDEN, "repack_example.json")))
    N, P, R = fx["N"], fx["P"], fx["R"]
    assert repack.gather_rows(N, P, R).tolist() == fx["gather_rows"]
    assert repack.scatter_rows(N, P, R).tolist() == fx["scatter_rows"]


@pytest.mark.parametrize("N,P,R", [(1, 5, 3), (4, 7, 2), (3, 0, 4), (2, 6, 0), (5, 1, 1)])
def test_round_trips(N, P, R):
    rng = np.random.default_rng(0)
    packed = rng.integers(0, 2 ** 31, size=(P + N * R, 3), dtype=np.int64)
    rep = repack.scatter(packed, N, P, R)
    assert rep.shape[0] == N * (P + R)
    # Every copy holds the same prompt, followed by its own response.
    for n in range(N):
        seq = rep[n * (P + R):(n + 1) * (P + R)]
        np.testing.assert_array_equal(seq[:P], packed[:P])
        np.testing.assert_array_equal(seq[P:], packed[P + n * R:P + (n + 1) * R])
    np.testing.assert_array_equal(repack.gather(rep, N, P, R), packed)
    np.testing.assert_array_equal(repack.scatter(repack.gather(rep, N, P, R), N, P, R), rep)
    # The token ratio rho = N(P+R)/(P+NR).
    if P + N * R:
        assert rep.shape[0] / packed.shape[0] == pytest.approx(N * (P + R) / (P + N * R))
