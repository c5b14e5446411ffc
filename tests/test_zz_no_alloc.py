"""dualkv_bwd_noalloc (static per-device workspace) against dualkv_bwd.

Two calls in a row on the same GPU, the second on a smaller problem, so the
second runs on a buffer that still holds the first call's contents; each
call's gradients must equal dualkv_bwd's on the same inputs bit for bit
(the kernels and their order are the same; only the workspace differs).
The result is also checked against the fp64 oracle under the parity gates.
A problem whose workspace exceeds the static buffer is rejected.
"""
import ctypes

import pytest
import torch

import shared_prompt_exact_amd as dk
import workloads
from oracle import replicated

from parity_utils import check, host, inputs_on_device

pytestmark = pytest.mark.gpu

W = workloads.Workload
CASES = [
    # slot partials (several response slots), GQA 4, ragged tails
    W("noalloc_big", "bf16", 6, 300, 140, 8, 2, 128, 0, seed=51, value_scale=1.0),
    # smaller, with a window and valid lengths: reuses the dirty buffer
    W("noalloc_small", "bf16", 3, 130, 70, 4, 2, 64, 50, seed=52, value_scale=1.0, len_range=(1, 70)),
]


def run(w):
    print(f"case {w}", flush=True)
    x = workloads.generate(w)
    d = inputs_on_device(w, x)
    kw = dict(window=w.window, valid_len=d["valid"])
    o, lse = dk.dualkv_fwd(d["q"], d["k"], d["v"], w.n_resp, w.prompt_len, w.resp_len, **kw)
    ref = dk.dualkv_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], w.n_resp, w.prompt_len, w.resp_len, **kw)
    got = dk.dualkv_bwd_noalloc(d["q"], d["k"], d["v"], o, lse, d["do"], w.n_resp, w.prompt_len,
                                w.resp_len, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{w.name} {name}: noalloc differs from dualkv_bwd"
    ora = replicated.replicated_fold(x.q, x.k, x.v, x.do, w.n_resp, w.prompt_len, w.resp_len, w.window,
                                     None, x.valid_len)
    for name, a in zip(("dq", "dk", "dv"), got):
        print(name, "rel-L2 %.2e max-abs %.2e" % check(name, host(a), ora[name], w.dtype), flush=True)


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    for w in CASES:
        run(w)


def test_too_large_problem_is_rejected():
    # the Qwen3-8B-shaped layer's workspace (about 179 MB) fits; four times
    # its prompt does not.  Validation happens before anything is launched
    # or touched, so the pointers are never dereferenced.
    lib = dk.load_library()
    dummy = torch.empty(256, dtype=torch.uint8, device="cuda")
    ptr = ctypes.c_void_p(dummy.data_ptr())
    p = dk.Params(n_resp=32, prompt_len=4 * 8192, resp_len=1024, n_q_heads=32, n_kv_heads=8, head_dim=128,
                  window=0, softmax_scale=0.0, dtype=dk.DUALKV_BF16, impl=0, resp_valid_len=None)
    need = lib.dualkv_bwd_workspace_bytes(ctypes.byref(p))
    assert need > (256 << 20)
    st = lib.dualkv_bwd_noalloc(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None)
    assert st == 5, st
    assert b"static scratch" in lib.dualkv_strerror(st)
