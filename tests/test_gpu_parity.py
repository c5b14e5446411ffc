"""Parity of the HIP path with the fp64 oracle (element by element).

Every case draws its inputs with the seeded generator, runs the library
through the C ABI (Python binding), and compares O, LSE, dQ, dK, dV with
the oracle's replicated-and-folded attention on the same inputs.
"""
import numpy as np
import pytest
import torch

import shared_prompt_exact_amd as dk
import workloads
from oracle import replicated, rounding

from parity_utils import STRESS, check, host, inputs_on_device, stress_modifier

pytestmark = pytest.mark.gpu

W = workloads.Workload


def run_case(w, impl=dk.IMPL_AUTO, backward=True, modify=None, delta_o=None, envelope=None):
    print(f"case {w}", flush=True)
    x = workloads.generate(w)
    if modify is not None:
        modify(w, x)
    d = inputs_on_device(w, x)
    kw = dict(window=w.window, valid_len=d["valid"], impl=impl)
    o, lse = dk.dualkv_fwd(d["q"], d["k"], d["v"], w.n_resp, w.prompt_len, w.resp_len, **kw)
    grads = None
    if backward:
        grads = dk.dualkv_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], w.n_resp, w.prompt_len,
                              w.resp_len, **kw)
    torch.cuda.synchronize()
    ref = replicated.replicated_fold(x.q, x.k, x.v, x.do, w.n_resp, w.prompt_len, w.resp_len,
                                     w.window, None, x.valid_len, backward=backward, delta_o=delta_o)
    uv = w.value_scale == 1.0
    out = {"o": check("o", host(o), ref["o"], w.dtype, uv),
           "lse": check("lse", host(lse), ref["lse"], w.dtype, uv)}
    if backward:
        for name, g in zip(("dq", "dk", "dv"), grads):
            out[name] = check(name, host(g), ref[name], w.dtype, uv,
                              envelope=None if envelope is None else envelope[name])
    print({k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in out.items()}, flush=True)
    return o, lse, grads


def test_tiny_f32_config():
    run_case(workloads.WORKLOADS["tiny_f32"])


def test_tiny_bf16_config():
    run_case(workloads.WORKLOADS["tiny_bf16"])


MID = [
    # ragged prompt and response tails, GQA 4, several 64-row blocks
    W("mid_gqa", "bf16", 3, 200, 150, 8, 2, 128, 0, seed=21, value_scale=1.0),
    # window across the prompt/response boundary
    W("mid_window", "bf16", 3, 300, 140, 4, 1, 128, 100, seed=22, value_scale=1.0),
    # per-response valid lengths incl. an empty and a full response
    W("mid_valid", "bf16", 4, 130, 96, 4, 2, 64, 0, seed=23, value_scale=1.0, len_range=(0, 96)),
    # no prompt (independent causal sequences) and no response
    W("mid_noprompt", "bf16", 3, 0, 100, 2, 2, 64, 0, seed=24, value_scale=1.0),
    W("mid_noresp", "bf16", 2, 170, 0, 4, 4, 128, 0, seed=25, value_scale=1.0),
    # one response: plain causal attention
    W("mid_single", "bf16", 1, 77, 65, 2, 1, 128, 0, seed=26, value_scale=1.0),
    # GQA 8 (one 32-row slice per head in a block), head dim 256
    W("mid_gqa8", "bf16", 2, 100, 70, 8, 1, 128, 0, seed=27, value_scale=1.0),
    W("mid_d256", "bf16", 2, 90, 70, 4, 2, 256, 40, seed=28, value_scale=1.0),
    # head dim 512 (head dim split over four waves) with GQA 4 and a ragged tail
    W("mid_d512", "bf16", 3, 70, 45, 4, 1, 512, 0, seed=31, value_scale=1.0),
    # head dim 256 without a window, valid lengths
    W("mid_d256_valid", "bf16", 3, 100, 64, 8, 2, 256, 0, seed=32, value_scale=1.0, len_range=(1, 64)),
    # the benchmark value scale (0.5) at a reduced size
    W("mid_half", "bf16", 4, 256, 128, 8, 2, 128, 0, seed=29, value_scale=0.5),
    # windows far shorter than the prompt: leading prompt key tiles get no
    # response term (no slot partials there), head dims 128 and 256
    W("mid_window_long", "bf16", 2, 700, 120, 4, 2, 128, 100, seed=33, value_scale=1.0),
    W("mid_window_d256", "bf16", 3, 400, 90, 4, 1, 256, 64, seed=34, value_scale=1.0),
]


@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_mid_cases_auto(w):
    run_case(w)


@pytest.mark.parametrize("w", MID[:4], ids=lambda w: w.name)
def test_mid_cases_scalar_path(w):
    run_case(w, impl=dk.IMPL_SCALAR)


@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_mid_cases_mfma_path(w):
    run_case(w, impl=dk.IMPL_MFMA)


def test_mid_f32_window_valid():
    w = W("mid_f32", "f32", 3, 70, 50, 4, 2, 64, 30, seed=30, value_scale=1.0, len_range=(10, 50))
    run_case(w)


@pytest.mark.parametrize("w", [m for m in MID if m.name in ("mid_gqa", "mid_d256", "mid_d512")],
                         ids=lambda w: w.name)
def test_forward_is_deterministic(w):
    """Two runs are bitwise equal, also where waves split the head dim and
    exchange partial scores (head dims 256 and 512)."""
    o1, l1, g1 = run_case(w)
    o2, l2, g2 = run_case(w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_prompt_rows_invariant_to_responses():
    """Prompt outputs are bitwise independent of the responses and of N."""
    w = MID[0]
    x = workloads.generate(w)
    d = inputs_on_device(w, x)
    o1, l1 = dk.dualkv_fwd(d["q"], d["k"], d["v"], w.n_resp, w.prompt_len, w.resp_len)
    P, R = w.prompt_len, w.resp_len
    q2, k2, v2 = (t[:P + R].contiguous() for t in (d["q"], d["k"], d["v"]))
    o2, l2 = dk.dualkv_fwd(q2, k2, v2, 1, P, R)
    torch.cuda.synchronize()
    assert torch.equal(o1[:P], o2[:P])
    assert torch.equal(l1[:, :P], l2[:, :P])


# Online-softmax stress (parity_utils.STRESS).  With a near one-hot softmax,
# dS = P (dP - Delta) cancels, and the backward takes Delta = rowsum(dO * O)
# from the bf16 O the forward returned: that rounding alone moves dQ by
# about 9% (rel-L2) on the early-max input.  So the backward is compared
# with the oracle's backward evaluated at its own O rounded to bf16 (the
# forward's output contract), under the rel-L2 gate and an elementwise gate
# widened by the rounding envelope of oracle.rounding (the kernel's own
# bf16 roundings of P, O and dS propagated through the fp64 oracle's
# quantities); the forward is compared with the exact oracle under the full
# gates.
@pytest.mark.parametrize("kind", ["peaked", "early_max", "late_max"])
def test_online_softmax_stress(kind):
    w = STRESS
    modify = stress_modifier(kind)
    x = workloads.generate(w)
    modify(w, x)
    env = rounding.backward_envelope(x.q, x.k, x.v, x.do, w.n_resp, w.prompt_len, w.resp_len)
    run_case(w, modify=modify, delta_o="bf16", envelope=env)
