"""Several prompt groups in one call: HIP path vs the fp64 grouped oracle.

Each case lays out groups of different (N, P, R) one after the other and
runs the grouped entry points once.  Checks:
 * O, LSE, dQ, dK, dV against ``oracle.groups.grouped_fold`` at the
   tolerances of the single-group parity tests;
 * bit-for-bit equality with one single-group call per group on the same
   rows (the grouped launches do the same arithmetic per group);
 * the grouped repack against the oracle's row maps, bit exact.
"""
import numpy as np
import pytest
import torch

import shared_prompt_exact_amd as dk
import workloads
from oracle import groups as og
from oracle import repack

from parity_utils import check, host, inputs_on_device

pytestmark = pytest.mark.gpu

GW = workloads.GroupedWorkload


def _many_groups(n, seed):
    rng = np.random.default_rng(seed)
    gs = []
    for _ in range(n):
        gs.append((int(rng.integers(1, 5)), int(rng.integers(0, 120)), int(rng.integers(0, 70))))
    return tuple(gs)


CASES = [
    # ragged tails, GQA 4, valid lengths, a group without a prompt
    GW("grp_mix", "bf16", ((3, 200, 150), (2, 0, 100), (4, 130, 96)), 8, 2, 128, seed=51, value_scale=1.0,
       len_ranges=((1, 150), (100, 100), (0, 96))),
    # window across each group's prompt/response boundary, far shorter than one prompt
    GW("grp_window", "bf16", ((2, 300, 140), (3, 90, 60), (2, 700, 100)), 4, 1, 128, 100, seed=52,
       value_scale=1.0),
    # head dim 64, a group without responses, an empty group in the middle
    GW("grp_d64", "bf16", ((1, 77, 65), (2, 170, 0), (1, 0, 0), (3, 50, 40)), 2, 2, 64, seed=53,
       value_scale=1.0),
    # head dims 256 (window) and 512
    GW("grp_d256", "bf16", ((2, 90, 70), (2, 150, 40)), 4, 2, 256, 40, seed=54, value_scale=1.0),
    GW("grp_d512", "bf16", ((2, 70, 45), (1, 40, 30)), 4, 1, 512, seed=55, value_scale=1.0),
    # groups whose cost ranges interleave (a long-prompt group, a long-response
    # group, many short responses), so the launch order mixes their chunks
    GW("grp_order", "bf16", ((12, 520, 64), (2, 64, 900), (5, 300, 33)), 4, 1, 128, seed=59,
       value_scale=1.0, len_ranges=((1, 64), (500, 900), (1, 33))),
    # the maximum number of groups, small and ragged
    GW("grp_max", "bf16", _many_groups(dk.MAX_GROUPS, 56), 4, 2, 128, seed=56, value_scale=1.0),
    # the scalar fp32 path
    GW("grp_f32", "f32", ((2, 40, 24), (3, 0, 17), (1, 33, 9)), 4, 2, 64, 20, seed=57, value_scale=1.0),
]


def run_grouped(w, x, d):
    kw = dict(window=w.window, valid_len=d["valid"])
    o, lse = dk.dualkv_fwd_groups(d["q"], d["k"], d["v"], w.groups, **kw)
    grads = dk.dualkv_bwd_groups(d["q"], d["k"], d["v"], o, lse, d["do"], w.groups, **kw)
    torch.cuda.synchronize()
    return o, lse, grads


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_groups_match_oracle(w):
    print(f"case {w.name} groups={w.groups}", flush=True)
    x = workloads.generate_groups(w)
    d = inputs_on_device(w, x)
    o, lse, (dq, dkk, dv) = run_grouped(w, x, d)
    ref = og.grouped_fold(x.q, x.k, x.v, x.do, w.groups, w.window, None, x.valid_len)
    out = {"o": check("o", host(o), ref["o"], w.dtype),
           "lse": check("lse", host(lse), ref["lse"], w.dtype)}
    for name, g in (("dq", dq), ("dk", dkk), ("dv", dv)):
        out[name] = check(name, host(g), ref[name], w.dtype)
    print({k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in out.items()}, flush=True)


def _case(name):
    return next(c for c in CASES if c.name == name)


@pytest.mark.parametrize("name", ["grp_mix", "grp_order", "grp_d512", "grp_max", "grp_window"])
def test_groups_write_every_output(name):
    """Every output element is written exactly by the grouped launches
    (outputs and workspace start as NaN): the launch order that interleaves
    the groups' work items reaches every item."""
    w = _case(name)
    print(f"case {w.name} groups={w.groups}", flush=True)
    x = workloads.generate_groups(w)
    d = inputs_on_device(w, x)
    kw = dict(window=w.window, valid_len=d["valid"])
    nan = float("nan")
    o = torch.full_like(d["q"], nan)
    lse = torch.full((d["q"].shape[1], d["q"].shape[0]), nan, dtype=torch.float32, device=d["q"].device)
    dk.dualkv_fwd_groups(d["q"], d["k"], d["v"], w.groups, out=o, lse=lse, **kw)
    need = dk.dualkv_bwd_groups_workspace_bytes(d["q"], d["k"], w.groups, **kw)
    ws = torch.full((max(need, 256),), 255, dtype=torch.uint8, device=d["q"].device)
    grads = [torch.full_like(d[n], nan) for n in ("q", "k", "v")]
    dk.dualkv_bwd_groups(d["q"], d["k"], d["v"], o, lse, d["do"], w.groups, workspace=ws, dq=grads[0],
                         dk=grads[1], dv=grads[2], **kw)
    torch.cuda.synchronize()
    assert not torch.isnan(lse).any()
    for name_, t in zip(("o", "dq", "dk", "dv"), [o] + grads):
        assert torch.isfinite(t).all(), name_


@pytest.mark.parametrize("w", [_case(n) for n in ("grp_mix", "grp_window", "grp_order", "grp_d512", "grp_max",
                                                  "grp_f32")],
                         ids=["grp_mix", "grp_window", "grp_order", "grp_d512", "grp_max", "grp_f32"])
def test_groups_bitwise_equal_single_calls(w):
    print(f"case {w.name} groups={w.groups}", flush=True)
    x = workloads.generate_groups(w)
    d = inputs_on_device(w, x)
    o, lse, grads = run_grouped(w, x, d)
    for (N, P, R), (r0, Tg, vl0) in zip(w.groups, og.layout(w.groups)):
        if Tg == 0:
            continue
        rows = slice(r0, r0 + Tg)
        sl = {n: d[n][rows].contiguous() for n in ("q", "k", "v", "do")}
        vl = None if d["valid"] is None else d["valid"][vl0:vl0 + N].contiguous()
        kw = dict(window=w.window, valid_len=vl)
        o1, l1 = dk.dualkv_fwd(sl["q"], sl["k"], sl["v"], N, P, R, **kw)
        g1 = dk.dualkv_bwd(sl["q"], sl["k"], sl["v"], o1, l1, sl["do"], N, P, R, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o[rows], o1), (N, P, R, "o")
        assert torch.equal(lse[:, rows], l1), (N, P, R, "lse")
        for name, a, b in zip(("dq", "dk", "dv"), grads, g1):
            assert torch.equal(a[rows], b), (N, P, R, name)


@pytest.mark.parametrize("groups,row_shape,dtype", [
    (((4, 64, 32), (2, 0, 11), (3, 13, 0), (1, 5, 7)), (2, 64), torch.bfloat16),
    (((3, 17, 5), (1, 0, 0), (5, 9, 7)), (3,), torch.int32),
    (_many_groups(dk.MAX_GROUPS, 58), (5,), torch.uint8),
])
def test_repack_groups_bit_exact(groups, row_shape, dtype):
    print(f"repack groups={groups} row={row_shape} {dtype}", flush=True)
    g = torch.Generator().manual_seed(len(groups))
    rows_rep = sum(N * (P + R) for N, P, R in groups)
    esz = torch.tensor([], dtype=dtype).element_size()
    raw = torch.randint(0, 256, (rows_rep,) + row_shape + (esz,), generator=g, dtype=torch.uint8)
    rep_host = raw.view(dtype).reshape((rows_rep,) + row_shape)
    packed = dk.dualkv_repack_groups(rep_host.cuda(), groups, dk.DUALKV_GATHER)
    back = dk.dualkv_repack_groups(packed, groups, dk.DUALKV_SCATTER)
    torch.cuda.synchronize()
    rep_u8 = rep_host.view(torch.uint8).numpy()
    exp_packed, exp_back, r = [], [], 0
    for N, P, R in groups:
        part = rep_u8[r:r + N * (P + R)]
        r += N * (P + R)
        pk = repack.gather(part, N, P, R)
        exp_packed.append(pk)
        exp_back.append(repack.scatter(pk, N, P, R))
    assert np.array_equal(packed.cpu().view(torch.uint8).numpy(), np.concatenate(exp_packed))
    assert np.array_equal(back.cpu().view(torch.uint8).numpy(), np.concatenate(exp_back))
