"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function declared in
include/dualkv.h, and reject invalid arguments on the host before any HIP
call, with the documented status codes.
"""
import ctypes
import os
import re

import pytest

import shared_prompt_exact_amd as dk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dualkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dk.LIB_PATH), reason="libdualkv.so not built")


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0      # counts devices without initialising HIP


# Tests that hand the library a fake device address (0x1000) rely on the
# host-side validation rejecting the call before any launch.  They run only
# where no GPU is visible: should a validation check ever move after a
# launch, the call then returns an error instead of starting a kernel that
# dereferences the fake address.
fake_ptr = pytest.mark.skipif(_gpu_visible(), reason="passes a fake device address; run only without a visible GPU")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dualkv_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = dk.load_library()
    names = declared_functions()
    assert set(names) >= {"dualkv_repack", "dualkv_fwd", "dualkv_bwd",
                          "dualkv_bwd_workspace_bytes", "dualkv_strerror"}
    for n in names:
        assert hasattr(lib, n), n


def params(**kw):
    base = dict(n_resp=4, prompt_len=64, resp_len=32, n_q_heads=4, n_kv_heads=2, head_dim=128,
                window=0, softmax_scale=0.0, dtype=dk.DUALKV_BF16, impl=0, resp_valid_len=None)
    base.update(kw)
    return dk.Params(**base)


def fwd_status(p):
    dummy = ctypes.c_void_p(0x1000)
    return dk.load_library().dualkv_fwd(ctypes.byref(p) if p is not None else None,
                                        dummy, dummy, dummy, dummy, dummy, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_resp=0), 1), (dict(prompt_len=-1), 1), (dict(resp_len=-2), 1),
    (dict(n_q_heads=6, n_kv_heads=4), 1), (dict(n_kv_heads=0), 1), (dict(head_dim=0), 1),
    (dict(head_dim=513), 2), (dict(dtype=7), 1), (dict(impl=9), 1),
    (dict(softmax_scale=-1.0), 1), (dict(softmax_scale=float("nan")), 1),
    (dict(dtype=dk.DUALKV_F32, impl=dk.IMPL_MFMA), 2),
    (dict(head_dim=96, impl=dk.IMPL_MFMA), 2),
])
@fake_ptr
def test_invalid_parameters_rejected(kw, code):
    assert fwd_status(params(**kw)) == code


@fake_ptr
def test_null_params_and_pointers():
    lib = dk.load_library()
    assert fwd_status(None) == 1
    p = params()
    assert lib.dualkv_fwd(ctypes.byref(p), None, None, None, None, None, None) == 1
    assert lib.dualkv_bwd_workspace_bytes(None) == 0
    assert lib.dualkv_bwd_workspace_bytes(ctypes.byref(params(n_resp=0))) == 0


def test_empty_problem_is_a_no_op():
    # P = R = 0: nothing to compute, success without touching the device
    p = params(prompt_len=0, resp_len=0)
    lib = dk.load_library()
    assert lib.dualkv_fwd(ctypes.byref(p), None, None, None, None, None, None) == 0


@fake_ptr
def test_workspace_too_small():
    lib = dk.load_library()
    p = params()
    need = lib.dualkv_bwd_workspace_bytes(ctypes.byref(p))
    assert need > 0 and need % 256 == 0
    d = ctypes.c_void_p(0x1000)
    st = lib.dualkv_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, need - 1, None)
    assert st == 3


@fake_ptr
def test_repack_argument_checks():
    lib = dk.load_library()
    d = ctypes.c_void_p(0x1000)
    assert lib.dualkv_repack(d, d, 0, 2, 3, 4, 0, None) == 1       # row_bytes < 1
    assert lib.dualkv_repack(d, d, 16, 0, 3, 4, 0, None) == 1      # N < 1
    assert lib.dualkv_repack(d, d, 16, 2, -1, 4, 0, None) == 1     # P < 0
    assert lib.dualkv_repack(d, d, 16, 2, 3, 4, 5, None) == 1      # direction
    assert lib.dualkv_repack(None, d, 16, 2, 3, 4, 0, None) == 1   # null with rows
    assert lib.dualkv_repack(None, None, 16, 2, 0, 0, 0, None) == 0  # nothing to copy


def test_strerror():
    lib = dk.load_library()
    assert lib.dualkv_strerror(0) == b"success"
    assert lib.dualkv_strerror(3) == b"workspace too small"
    assert lib.dualkv_strerror(99) == b"unknown status"


def group_array(*gs):
    return (dk.Group * max(1, len(gs)))(*[dk.Group(*g) for g in gs]), len(gs)


def fwd_groups_status(p, arr, n):
    d = ctypes.c_void_p(0x1000)
    return dk.load_library().dualkv_fwd_groups(ctypes.byref(p), arr, n, d, d, d, d, d, None)


@fake_ptr
def test_group_argument_checks():
    lib = dk.load_library()
    p = params()
    arr, _ = group_array((2, 16, 8))
    assert fwd_groups_status(p, arr, 0) == 1                           # no group
    assert lib.dualkv_fwd_groups(ctypes.byref(p), None, 1, *[None] * 6) == 1
    many, n = group_array(*[(1, 4, 4)] * (dk.MAX_GROUPS + 1))
    assert fwd_groups_status(p, many, n) == 2                          # above the maximum
    ok, n = group_array(*[(1, 4, 4)] * dk.MAX_GROUPS)
    assert lib.dualkv_bwd_groups_workspace_bytes(ctypes.byref(p), ok, n) > 0
    for bad in ((0, 4, 4), (1, -1, 4), (1, 4, -1)):
        arr, n = group_array((2, 16, 8), bad)
        assert fwd_groups_status(p, arr, n) == 1, bad
        assert lib.dualkv_bwd_groups_workspace_bytes(ctypes.byref(p), arr, n) == 0
    arr, n = group_array((3, 0, 0), (1, 0, 0))                         # no rows at all
    assert lib.dualkv_fwd_groups(ctypes.byref(p), arr, n, *[None] * 6) == 0
    d = ctypes.c_void_p(0x1000)
    assert lib.dualkv_repack_groups(d, d, 16, None, 1, 0, None) == 1
    assert lib.dualkv_repack_groups(d, d, 16, many, dk.MAX_GROUPS + 1, 0, None) == 2
    arr, n = group_array((2, 3, 4), (0, 3, 4))
    assert lib.dualkv_repack_groups(d, d, 16, arr, n, 0, None) == 1
    arr, n = group_array((2, 0, 0), (1, 0, 0))
    assert lib.dualkv_repack_groups(None, None, 16, arr, n, 1, None) == 0


@pytest.mark.parametrize("dtype,impl", [(dk.DUALKV_BF16, dk.IMPL_AUTO), (dk.DUALKV_F32, dk.IMPL_AUTO),
                                        (dk.DUALKV_BF16, dk.IMPL_SCALAR)])
def test_one_group_matches_single_entry_points(dtype, impl):
    lib = dk.load_library()
    for N, P, R, W in ((4, 64, 32, 0), (8, 300, 70, 0), (3, 1000, 100, 128), (2, 0, 50, 0)):
        p = params(n_resp=N, prompt_len=P, resp_len=R, window=W, dtype=dtype, impl=impl)
        arr, n = group_array((N, P, R))
        q = params(n_resp=99, prompt_len=7, resp_len=5, window=W, dtype=dtype, impl=impl)  # ignored fields
        assert lib.dualkv_bwd_groups_workspace_bytes(ctypes.byref(q), arr, n) == \
            lib.dualkv_bwd_workspace_bytes(ctypes.byref(p))


def test_group_workspace_covers_every_row():
    # per-row statistics for all rows of the launch, plus each group's partials
    lib = dk.load_library()
    p = params()
    g1, g2 = (4, 640, 160), (8, 320, 64)
    rows = sum(P + N * R for N, P, R in (g1, g2))
    arr, n = group_array(g1, g2)
    both = lib.dualkv_bwd_groups_workspace_bytes(ctypes.byref(p), arr, n)
    assert both >= 2 * 4 * p.n_q_heads * rows
    sep = 0
    for g in (g1, g2):
        a1, _ = group_array(g)
        sep += lib.dualkv_bwd_groups_workspace_bytes(ctypes.byref(p), a1, 1)
    assert both <= sep + 1024


def layer_params(**kw):
    base = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=384, window=0, rope_base=1e4,
                norm_eps=1e-6, valid_len=None)
    base.update(kw)
    return dk.make_layer_params(**base)


@fake_ptr
def test_layer_argument_checks():
    lib = dk.load_library()
    arr, n = group_array((2, 30, 20))
    ok = layer_params()
    assert lib.dualkv_layer_saved_bytes(ctypes.byref(ok), arr, n) > 0
    assert lib.dualkv_layer_workspace_bytes(ctypes.byref(ok), arr, n) > 0
    for bad in (dict(hidden=200), dict(ffn=100), dict(head_dim=48)):        # not whole 128-wide blocks
        p = layer_params(**bad)
        w = dk.LayerWeights()
        assert lib.dualkv_layer_fwd(ctypes.byref(p), arr, n, ctypes.byref(w), None, None, None, 0, None) == 2, bad
    for bad in (dict(rope_base=1.0), dict(norm_eps=0.0), dict(n_kv_heads=3)):
        p = layer_params(**bad)
        w = dk.LayerWeights()
        assert lib.dualkv_layer_fwd(ctypes.byref(p), arr, n, ctypes.byref(w), None, None, None, 0, None) == 1, bad
        assert lib.dualkv_layer_saved_bytes(ctypes.byref(p), arr, n) == 0
    w = dk.LayerWeights()
    assert lib.dualkv_layer_fwd(ctypes.byref(ok), None, 1, ctypes.byref(w), None, None, None, 0, None) == 1
    need = lib.dualkv_layer_saved_bytes(ctypes.byref(ok), arr, n)
    d = ctypes.c_void_p(0x1000)
    assert lib.dualkv_layer_fwd(ctypes.byref(ok), arr, n, ctypes.byref(w), d, d, d, need - 1, None) == 3
    empty, ne = group_array((2, 0, 0))                                        # nothing to compute
    assert lib.dualkv_layer_fwd(ctypes.byref(ok), empty, ne, ctypes.byref(w), None, None, None, 0, None) == 0


@fake_ptr
def test_layer_op_argument_checks():
    lib = dk.load_library()
    d = ctypes.c_void_p(0x1000)
    # GEMM: both operands transposed; k not a whole 64-wide block; k-major B with ragged n
    assert lib.dualkv_gemm_bf16(1, 1, 128, 128, 64, d, 128, d, 64, d, 128, None, 0, None) == 2
    assert lib.dualkv_gemm_bf16(0, 0, 100, 128, 70, d, 70, d, 128, d, 128, None, 0, None) == 2
    assert lib.dualkv_gemm_bf16(0, 0, 100, 100, 64, d, 64, d, 100, d, 100, None, 0, None) == 2
    assert lib.dualkv_gemm_bf16(2, 0, 100, 128, 64, d, 64, d, 128, d, 128, None, 0, None) == 1
    assert lib.dualkv_gemm_bf16(0, 0, 100, 128, 64, ctypes.c_void_p(0x1008), 64, d, 128, d, 128, None, 0,
                                None) == 1                                    # A not 16-byte aligned
    assert lib.dualkv_gemm_bf16(0, 0, 0, 128, 64, None, 64, None, 128, None, 128, None, 0, None) == 0
    assert lib.dualkv_rmsnorm_fwd(10, 12, 1e-6, d, d, d, d, None) == 1       # H % 8
    assert lib.dualkv_rmsnorm_fwd(10, 16, 0.0, d, d, d, d, None) == 1        # eps
    assert lib.dualkv_swiglu_fwd(12, d, d, d, None) == 1                      # n % 8
    arr, n = group_array((2, 3, 4))
    assert lib.dualkv_rope(arr, n, 2, 7, 1e4, 0, d, None) == 1                # odd head dim
    assert lib.dualkv_rope(arr, n, 2, 8, 1e4, 2, d, None) == 1                # inverse flag
    assert lib.dualkv_rope(None, 1, 2, 8, 1e4, 0, d, None) == 1
