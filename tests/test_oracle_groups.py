"""Pins of the grouped oracle (oracle.groups), CPU only.

The grouped definition (every group its own shared-prompt problem, groups
laid one after the other) is checked against what does not depend on it:
 * dense masked attention over the whole micro-batch with the block-
   diagonal mask built from row attributes (a second route: one softmax
   over packed rows, not N replicated sequences per group);
 * finite differences of sum(O * dO) for the dense route's gradients,
   at entries of different groups;
 * no leak: changing one group's inputs leaves the other groups' outputs
   bit for bit unchanged;
 * permuting the groups permutes the rows of every output;
 * the mask's pair count equals the closed form of the visible pairs
   summed over groups.
"""
import numpy as np
import pytest

from oracle import groups as og
from oracle import replicated
from shared_prompt_exact_amd import workcount

MIXES = [
    # (groups, window, valid lengths or None, Hq, Hkv, D)
    (((2, 5, 4), (3, 0, 3), (1, 6, 0), (2, 3, 5)), 0, None, 4, 2, 8),
    (((3, 4, 5), (2, 7, 3)), 4, None, 2, 1, 8),
    (((2, 6, 4), (3, 2, 3)), 0, [4, 1, 0, 3, 2], 2, 2, 4),
    (((1, 0, 0), (2, 3, 2), (1, 0, 0)), 3, [0, 2, 0, 0], 3, 1, 4),
]


def inputs(groups, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    T = sum(P + N * R for N, P, R in groups)
    return (rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)),
            rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hq, D)))


@pytest.mark.parametrize("case", range(len(MIXES)))
def test_grouped_fold_equals_dense_block_diagonal(case):
    groups, W, vl, Hq, Hkv, D = MIXES[case]
    q, k, v, do = inputs(groups, Hq, Hkv, D, 100 + case)
    a = og.grouped_fold(q, k, v, do, groups, W, None, vl)
    b = og.grouped_dense(q, k, v, do, groups, W, None, vl)
    np.testing.assert_array_equal(np.isfinite(a["lse"]), np.isfinite(b["lse"]))
    fin = np.isfinite(a["lse"])
    np.testing.assert_allclose(a["lse"][fin], b["lse"][fin], rtol=0, atol=1e-12)
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(a[name], b[name], rtol=0, atol=1e-11, err_msg=name)


def test_dense_gradients_by_finite_differences():
    groups, W, vl, Hq, Hkv, D = MIXES[0]
    q, k, v, do = inputs(groups, Hq, Hkv, D, 7)
    res = og.grouped_dense(q, k, v, do, groups, W, None, vl)
    lay = og.layout(groups)

    def loss(q_, k_, v_):
        o, _ = og.dense.forward_masked(q_, k_, v_, og.visibility(groups, W, vl))
        return float((o * do).sum())

    eps = 1e-6
    for gi in (0, 3):                      # a row inside two different groups
        t = lay[gi][0] + lay[gi][1] - 1
        for arr, grad, h in ((q, res["dq"], 1), (k, res["dk"], 0), (v, res["dv"], 1)):
            for d in (0, D - 1):
                a1, a2 = arr.copy(), arr.copy()
                a1[t, h, d] += eps
                a2[t, h, d] -= eps
                args1 = [a1 if x is arr else x for x in (q, k, v)]
                args2 = [a2 if x is arr else x for x in (q, k, v)]
                fd = (loss(*args1) - loss(*args2)) / (2 * eps)
                assert abs(fd - grad[t, h, d]) <= 1e-6 * max(1.0, abs(fd)), (gi, t, h, d, fd, grad[t, h, d])


def test_groups_do_not_leak():
    groups, W, vl, Hq, Hkv, D = MIXES[1]
    q, k, v, do = inputs(groups, Hq, Hkv, D, 8)
    a = og.grouped_fold(q, k, v, do, groups, W)
    r0, T0, _ = og.layout(groups)[0]
    r1, T1, _ = og.layout(groups)[1]
    for arr in (q, k, v, do):
        arr[r1:r1 + T1] *= -3.0             # change group 1 only
    b = og.grouped_fold(q, k, v, do, groups, W)
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[name][r0:r0 + T0], b[name][r0:r0 + T0])
        assert not np.allclose(a[name][r1:r1 + T1], b[name][r1:r1 + T1])
    np.testing.assert_array_equal(a["lse"][:, r0:r0 + T0], b["lse"][:, r0:r0 + T0])


def test_each_group_is_the_single_group_problem():
    groups, W, vl, Hq, Hkv, D = MIXES[2]
    q, k, v, do = inputs(groups, Hq, Hkv, D, 9)
    a = og.grouped_fold(q, k, v, do, groups, W, None, vl)
    for (N, P, R), (r0, Tg, vl0) in zip(groups, og.layout(groups)):
        rows = slice(r0, r0 + Tg)
        s = replicated.replicated_fold(q[rows], k[rows], v[rows], do[rows], N, P, R, W, None,
                                       vl[vl0:vl0 + N])
        for name in ("o", "dq", "dk", "dv"):
            np.testing.assert_array_equal(a[name][rows], s[name])


def test_permuting_groups_permutes_rows():
    groups, W, vl, Hq, Hkv, D = MIXES[0]
    q, k, v, do = inputs(groups, Hq, Hkv, D, 10)
    order = [2, 0, 3, 1]
    lay = og.layout(groups)
    perm = np.concatenate([np.arange(lay[i][0], lay[i][0] + lay[i][1]) for i in order])
    pg = [groups[i] for i in order]
    a = og.grouped_dense(q, k, v, do, groups, W)
    b = og.grouped_dense(q[perm], k[perm], v[perm], do[perm], pg, W)
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(b[name], a[name][perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["lse"], a["lse"][:, perm], rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", range(len(MIXES)))
def test_mask_pair_count_closed_form(case):
    groups, W, vl, *_ = MIXES[case]
    want = 0
    for (N, P, R), (_, _, vl0) in zip(groups, og.layout(groups)):
        want += workcount.visible_pairs(N, P, R, W, None if vl is None else vl[vl0:vl0 + N])
    assert int(og.visibility(groups, W, vl).sum()) == want
