"""The packed transformer layer and its token-wise kernels: HIP vs fp64 oracle.

 * GEMM (the three forms of a linear layer, both tile heights, ragged rows,
   a ragged k for the weight-gradient form, a residual) against fp64 products of the same bf16
   inputs: the only differences are the fp32 accumulation order and the
   final bf16 rounding (at most 2^-9 relative), so rel-L2 <= 2e-3;
 * RMSNorm, RoPE at logical positions, SwiGLU, forward and backward,
   against ``oracle.layer``'s formulas, at the same bar;
 * the whole layer, forward and backward, against ``oracle.layer.layer_fold``
   (the N replicated sequences of each group, folded): the HIP path stores
   every activation in bf16 between its steps, so errors of a few 2^-9
   roundings accumulate; the bar is the bf16 attention tolerance, rel-L2 <=
   1e-2 for y, dx and every weight gradient, with the local-fault gate;
 * two runs of the layer are bitwise equal.
"""
import numpy as np
import pytest
import torch

import shared_prompt_exact_amd as dk
from oracle import layer as ol
from oracle.replicated import round_bf16

from parity_utils import check, host

pytestmark = pytest.mark.gpu


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def rounded(rng, *shape, scale=1.0):
    return round_bf16(rng.standard_normal(shape) * scale)


def tight(name, got, want, rel=2e-3):
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    rms = np.sqrt(np.mean(want ** 2))
    worst = np.max(np.abs(got - want) - (2.0 ** -8) * np.abs(want) - 2e-3 * rms)
    print(f"  {name}: rel-L2 {err:.2e}", flush=True)
    assert err <= rel, (name, err)
    assert worst <= 0, (name, worst)


@pytest.mark.parametrize("ta,tb,M,N,K,res", [
    (0, 0, 300, 256, 192, False), (0, 0, 1000, 512, 1024, True), (0, 1, 300, 384, 256, False),
    (1, 0, 256, 384, 200, False), (1, 0, 128, 128, 64, True), (1, 0, 384, 256, 1001, False),
    # enough 256-row blocks for the eight-wave tile in the row-major forms
    (0, 0, 4000, 4096, 256, True), (0, 1, 4000, 4096, 128, False),
    # 256 x 256 tiles (256-wide column blocks, at least one block per CU), a ragged last row block
    # and, in the weight-gradient form, a ragged k
    (0, 0, 4000, 4096, 192, True), (0, 1, 4096, 4096, 128, False), (1, 0, 4096, 4096, 1001, False),
    # rows of C not 8-byte aligned (element-wise epilogue) and a ragged last column block
    (0, 1, 300, 383, 256, True), (0, 1, 4096, 4096, 256, True),
])
def test_gemm(ta, tb, M, N, K, res):
    print(f"gemm ta={ta} tb={tb} M={M} N={N} K={K} residual={res}", flush=True)
    rng = np.random.default_rng(M + N + K)
    a = rounded(rng, *((K, M) if ta else (M, K)))
    b = rounded(rng, *((N, K) if tb else (K, N)))
    r = rounded(rng, M, N) if res else None
    c = dk.dualkv_gemm_bf16(bf(a), bf(b), bool(ta), bool(tb), None if r is None else bf(r))
    want = (a.T if ta else a) @ (b.T if tb else b) + (0 if r is None else r)
    tight("C", host(c), want)


def test_rmsnorm():
    rng = np.random.default_rng(1)
    T, H = 333, 256
    x, w, dy, dres = rounded(rng, T, H), round_bf16(1 + 0.1 * rng.standard_normal(H)), rounded(rng, T, H), rounded(rng, T, H)
    y, rstd = dk.dualkv_rmsnorm_fwd(bf(x), bf(w), 1e-6)
    wy, wr = ol.rmsnorm(x, w, 1e-6)
    tight("y", host(y), wy)
    tight("rstd", host(rstd), wr[:, 0], 1e-5)
    dx, dw = dk.dualkv_rmsnorm_bwd(bf(x), bf(w), rstd, bf(dy), bf(dres))
    wdx, wdw = ol.rmsnorm_bwd(x, w, wr, dy)
    tight("dx", host(dx), wdx + dres)
    tight("dw", host(dw), wdw)


@pytest.mark.parametrize("head_dim", [64, 24])   # 16-byte vector path; scalar path
def test_rope_logical_positions(head_dim):
    rng = np.random.default_rng(2)
    groups = [(3, 50, 40), (2, 0, 30), (1, 7, 0)]
    T = sum(P + N * R for N, P, R in groups)
    x = rounded(rng, T, 2, head_dim)
    t = bf(x)
    dk.dualkv_rope(t, groups, 1e4)
    pos = ol.packed_positions(groups)
    tight("rope", host(t), ol.rope(x, pos, 1e4))
    y = host(t)                          # the rotated bf16 rows, input of the inverse
    dk.dualkv_rope(t, groups, 1e4, inverse=True)
    tight("rope^-1", host(t), ol.rope(y, pos, 1e4, inverse=True))


def test_swiglu():
    rng = np.random.default_rng(3)
    u, g, dm = rounded(rng, 64, 96, scale=2.0), rounded(rng, 64, 96), rounded(rng, 64, 96)
    m = dk.dualkv_swiglu_fwd(bf(u), bf(g))
    tight("m", host(m), ol.silu(u) * g)
    du, dg = dk.dualkv_swiglu_bwd(bf(u), bf(g), bf(dm))
    wdu, wdg = ol.swiglu_bwd(u, g, dm)
    tight("du", host(du), wdu)
    tight("dg", host(dg), wdg)


Hm, Hq, Hkv, D, F = 256, 4, 2, 64, 384
LAYER_CASES = [
    ([(2, 70, 45), (3, 40, 30)], 0, [45, 20, 30, 0, 17]),
    ([(3, 100, 60)], 48, None),
    # K/V projection widths of whole 256-column tiles: x Wk and x Wv (and
    # their weight gradients) run as one two-part launch
    ([(2, 90, 50)], 0, None, (8, 4, 64)),
]


def case_shape(case):
    """(Hq, Hkv, D) of a layer case; the module defaults unless it names its own."""
    return LAYER_CASES[case][3] if len(LAYER_CASES[case]) > 3 else (Hq, Hkv, D)


def layer_inputs(groups, seed, Hq=Hq, Hkv=Hkv, D=D):
    rng = np.random.default_rng(seed)
    T = sum(P + N * R for N, P, R in groups)
    sh = {"norm1": (Hm,), "wq": (Hm, Hq * D), "wk": (Hm, Hkv * D), "wv": (Hm, Hkv * D), "wo": (Hq * D, Hm),
          "norm2": (Hm,), "w1": (Hm, F), "w3": (Hm, F), "w2": (F, Hm)}
    W = {}
    for n in dk.LAYER_WEIGHTS:
        W[n] = round_bf16(1 + 0.1 * rng.standard_normal(sh[n])) if n.startswith("norm") else \
            rounded(rng, *sh[n], scale=1 / np.sqrt(sh[n][0]))
    return rounded(rng, T, Hm), rounded(rng, T, Hm), W


def run_layer(groups, window, vl, x, dy, W, Hq=Hq, Hkv=Hkv, D=D):
    valid = None if vl is None else torch.tensor(vl, dtype=torch.int32, device="cuda")
    p = dk.make_layer_params(Hm, Hq, Hkv, D, F, window, 1e4, 1e-6, valid)
    Wd = {n: bf(W[n]) for n in dk.LAYER_WEIGHTS}
    xd = bf(x)
    y, saved = dk.dualkv_layer_fwd(xd, Wd, groups, p)
    dx, grads = dk.dualkv_layer_bwd(xd, saved, bf(dy), Wd, groups, p)
    torch.cuda.synchronize()
    return y, dx, grads


@pytest.mark.parametrize("case", range(len(LAYER_CASES)))
def test_layer_matches_oracle(case):
    groups, window, vl = LAYER_CASES[case][:3]
    hq, hkv, d = case_shape(case)
    print(f"layer groups={groups} window={window} valid={vl} heads={hq}/{hkv} D={d}", flush=True)
    x, dy, W = layer_inputs(groups, 20 + case, hq, hkv, d)
    y, dx, grads = run_layer(groups, window, vl, x, dy, W, hq, hkv, d)
    ref = ol.layer_fold(x, W, dy, groups, hq, hkv, window, 1e4, 1e-6, vl)
    out = {"y": check("y", host(y), ref["y"], "bf16", False), "dx": check("dx", host(dx), ref["dx"], "bf16", False)}
    for n in dk.LAYER_WEIGHTS:
        out[n] = check(n, host(grads[n]), ref["grads"][n], "bf16", False)
    print({k: f"{v[0]:.2e}" for k, v in out.items()}, flush=True)


@pytest.mark.parametrize("case", [0, 2])
def test_layer_bitwise_reproducible(case):
    groups, window, vl = LAYER_CASES[case][:3]
    hq, hkv, d = case_shape(case)
    x, dy, W = layer_inputs(groups, 30, hq, hkv, d)
    a = run_layer(groups, window, vl, x, dy, W, hq, hkv, d)
    b = run_layer(groups, window, vl, x, dy, W, hq, hkv, d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for n in dk.LAYER_WEIGHTS:
        assert torch.equal(a[2][n], b[2][n]), n
