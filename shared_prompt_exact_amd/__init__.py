"""Python binding of libdualkv.so (shared-prompt / DualKV attention on MI355X).

Argument marshalling only: every step runs in the HIP kernels of the
library.  torch supplies device memory and the current stream.  The
functions carry the names of the C entry points declared in
include/dualkv.h; see that header for layouts, masks and errors.

There is no fallback: if the library is not built, or a call fails, a
RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdualkv.so")

DUALKV_OK = 0
DUALKV_F32, DUALKV_BF16 = 0, 1
DUALKV_GATHER, DUALKV_SCATTER = 0, 1
IMPL_AUTO, IMPL_SCALAR, IMPL_MFMA = 0, 1, 2

_lib = None


class Params(ctypes.Structure):
    _fields_ = [
        ("n_resp", ctypes.c_int32),
        ("prompt_len", ctypes.c_int32),
        ("resp_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("impl", ctypes.c_int32),
        ("resp_valid_len", ctypes.c_void_p),
    ]


class Group(ctypes.Structure):
    _fields_ = [("n_resp", ctypes.c_int32), ("prompt_len", ctypes.c_int32), ("resp_len", ctypes.c_int32)]


MAX_GROUPS = 32

LAYER_WEIGHTS = ("norm1", "wq", "wk", "wv", "wo", "norm2", "w1", "w3", "w2")


class LayerParams(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float), ("resp_valid_len", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHTS]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHTS]


def load_library():
    """Load libdualkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m shared_prompt_exact_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pp = ctypes.POINTER(Params)
    lib.dualkv_repack.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp]
    lib.dualkv_repack.restype = ctypes.c_int
    lib.dualkv_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp]
    lib.dualkv_fwd.restype = ctypes.c_int
    lib.dualkv_bwd_workspace_bytes.argtypes = [pp]
    lib.dualkv_bwd_workspace_bytes.restype = sz
    lib.dualkv_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dualkv_bwd.restype = ctypes.c_int
    lib.dualkv_bwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dualkv_bwd_noalloc.restype = ctypes.c_int
    gp = ctypes.POINTER(Group)
    lib.dualkv_repack_groups.argtypes = [vp, vp, i64, gp, i32, i32, vp]
    lib.dualkv_repack_groups.restype = ctypes.c_int
    lib.dualkv_fwd_groups.argtypes = [pp, gp, i32, vp, vp, vp, vp, vp, vp]
    lib.dualkv_fwd_groups.restype = ctypes.c_int
    lib.dualkv_bwd_groups_workspace_bytes.argtypes = [pp, gp, i32]
    lib.dualkv_bwd_groups_workspace_bytes.restype = sz
    lib.dualkv_bwd_groups.argtypes = [pp, gp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dualkv_bwd_groups.restype = ctypes.c_int
    f32, i64p = ctypes.c_float, ctypes.c_int64
    lib.dualkv_gemm_bf16.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.dualkv_rmsnorm_fwd.argtypes = [i32, i32, f32, vp, vp, vp, vp, vp]
    lib.dualkv_rmsnorm_bwd_workspace_bytes.argtypes = [i32, i32]
    lib.dualkv_rmsnorm_bwd_workspace_bytes.restype = sz
    lib.dualkv_rmsnorm_bwd.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dualkv_rope.argtypes = [gp, i32, i32, i32, f32, i32, vp, vp]
    lib.dualkv_swiglu_fwd.argtypes = [i64p, vp, vp, vp, vp]
    lib.dualkv_swiglu_bwd.argtypes = [i64p, vp, vp, vp, vp, vp, vp]
    lpp = ctypes.POINTER(LayerParams)
    lib.dualkv_layer_saved_bytes.argtypes = [lpp, gp, i32]
    lib.dualkv_layer_saved_bytes.restype = sz
    lib.dualkv_layer_workspace_bytes.argtypes = [lpp, gp, i32]
    lib.dualkv_layer_workspace_bytes.restype = sz
    lib.dualkv_layer_fwd.argtypes = [lpp, gp, i32, ctypes.POINTER(LayerWeights), vp, vp, vp, sz, vp]
    lib.dualkv_layer_bwd.argtypes = [lpp, gp, i32, ctypes.POINTER(LayerWeights), vp, vp, sz, vp, vp,
                                     ctypes.POINTER(LayerGrads), vp, sz, vp]
    lib.dualkv_mfma_probe.argtypes = [i32, i32, vp]
    lib.dualkv_mfma_probe.restype = ctypes.c_int64
    lib.dualkv_strerror.argtypes = [ctypes.c_int]
    lib.dualkv_strerror.restype = ctypes.c_char_p
    lib.dualkv_profile_start.argtypes = []
    lib.dualkv_profile_stop.argtypes = []
    lib.dualkv_profile_count.argtypes = []
    lib.dualkv_profile_kernel.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                          ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    _lib = lib
    return lib


def _check(code: int, what: str):
    if code != DUALKV_OK:
        msg = load_library().dualkv_strerror(code).decode()
        raise RuntimeError(f"{what}: {msg} (status {code})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DUALKV_F32
    if t.dtype == torch.bfloat16:
        return DUALKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _require(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_params(q: torch.Tensor, k: torch.Tensor, n_resp: int, prompt_len: int, resp_len: int,
                window: int = 0, softmax_scale: float = 0.0,
                valid_len: Optional[torch.Tensor] = None, impl: int = IMPL_AUTO) -> Params:
    T = prompt_len + n_resp * resp_len
    _require(q, "q")
    _require(k, "k", dtype=q.dtype)
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != T or k.shape[0] != T or q.shape[2] != k.shape[2]:
        raise ValueError(f"q {tuple(q.shape)} / k {tuple(k.shape)} do not match T = P + N*R = {T}")
    if valid_len is not None:
        _require(valid_len, "valid_len", dtype=torch.int32, shape=(n_resp,))
    return Params(n_resp, prompt_len, resp_len, q.shape[1], k.shape[1], q.shape[2], window,
                  softmax_scale, _dtype_code(q), impl, None if valid_len is None else valid_len.data_ptr())


def dualkv_repack(src: torch.Tensor, n_resp: int, prompt_len: int, resp_len: int, direction: int,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GATHER (replicated -> packed) or SCATTER (packed -> replicated) rows
    of `src` (first dimension = rows, the rest is the opaque row)."""
    lib = load_library()
    _require(src, "src")
    rows_in = n_resp * (prompt_len + resp_len) if direction == DUALKV_GATHER else prompt_len + n_resp * resp_len
    rows_out = prompt_len + n_resp * resp_len if direction == DUALKV_GATHER else n_resp * (prompt_len + resp_len)
    if src.shape[0] != rows_in:
        raise ValueError(f"src has {src.shape[0]} rows, expected {rows_in}")
    if out is None:
        out = torch.empty((rows_out,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    _require(out, "out", dtype=src.dtype, shape=(rows_out,) + tuple(src.shape[1:]))
    row_bytes = src[0].numel() * src.element_size() if src.shape[0] else max(1, src.element_size())
    _check(lib.dualkv_repack(_ptr(src), _ptr(out), row_bytes, n_resp, prompt_len, resp_len,
                             direction, _stream()), "dualkv_repack")
    return out


def dualkv_fwd(q, k, v, n_resp, prompt_len, resp_len, window=0, softmax_scale=0.0,
               valid_len=None, impl=IMPL_AUTO, out=None, lse=None):
    """Forward pass; returns (o [T,Hq,D], lse [Hq,T] fp32)."""
    lib = load_library()
    p = make_params(q, k, n_resp, prompt_len, resp_len, window, softmax_scale, valid_len, impl)
    _require(v, "v", dtype=q.dtype, shape=k.shape)
    T, Hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _require(out, "out", dtype=q.dtype, shape=q.shape)
    _require(lse, "lse", dtype=torch.float32, shape=(Hq, T))
    _check(lib.dualkv_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream()),
           "dualkv_fwd")
    return out, lse


def dualkv_bwd_workspace_bytes(q, k, n_resp, prompt_len, resp_len, window=0, softmax_scale=0.0,
                               valid_len=None, impl=IMPL_AUTO) -> int:
    p = make_params(q, k, n_resp, prompt_len, resp_len, window, softmax_scale, valid_len, impl)
    return int(load_library().dualkv_bwd_workspace_bytes(ctypes.byref(p)))


def dualkv_bwd(q, k, v, o, lse, dout, n_resp, prompt_len, resp_len, window=0, softmax_scale=0.0,
               valid_len=None, impl=IMPL_AUTO, workspace=None, dq=None, dk=None, dv=None):
    """Backward pass; returns (dq, dk, dv)."""
    lib = load_library()
    p = make_params(q, k, n_resp, prompt_len, resp_len, window, softmax_scale, valid_len, impl)
    _require(v, "v", dtype=q.dtype, shape=k.shape)
    _require(o, "o", dtype=q.dtype, shape=q.shape)
    _require(dout, "dout", dtype=q.dtype, shape=q.shape)
    _require(lse, "lse", dtype=torch.float32, shape=(q.shape[1], q.shape[0]))
    need = int(lib.dualkv_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", dtype=torch.uint8)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _require(t, name, dtype=ref.dtype, shape=ref.shape)
    _check(lib.dualkv_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream()),
           "dualkv_bwd")
    return dq, dk, dv


def dualkv_bwd_noalloc(q, k, v, o, lse, dout, n_resp, prompt_len, resp_len, window=0, softmax_scale=0.0,
                       valid_len=None, impl=IMPL_AUTO, dq=None, dk=None, dv=None):
    """dualkv_bwd with the library's static per-device workspace (the call
    allocates nothing on the device; pass dq, dk, dv to allocate nothing
    here either).  Returns (dq, dk, dv)."""
    lib = load_library()
    p = make_params(q, k, n_resp, prompt_len, resp_len, window, softmax_scale, valid_len, impl)
    _require(v, "v", dtype=q.dtype, shape=k.shape)
    _require(o, "o", dtype=q.dtype, shape=q.shape)
    _require(dout, "dout", dtype=q.dtype, shape=q.shape)
    _require(lse, "lse", dtype=torch.float32, shape=(q.shape[1], q.shape[0]))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _require(t, name, dtype=ref.dtype, shape=ref.shape)
    _check(lib.dualkv_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _stream()),
           "dualkv_bwd_noalloc")
    return dq, dk, dv


def dualkv_mfma_probe(workgroups, iters):
    """Enqueue the matrix-core rate probe on the current stream; returns its FLOPs."""
    fl = int(load_library().dualkv_mfma_probe(workgroups, iters, _stream()))
    if fl < 0:
        raise RuntimeError("dualkv_mfma_probe failed")
    return fl


def dualkv_profile_start():
    """Start bracketing every library launch with HIP events."""
    _check(load_library().dualkv_profile_start(), "dualkv_profile_start")


def dualkv_profile_stop():
    """Stop, wait for the events and return {kernel: (launches, total_ms)}."""
    lib = load_library()
    _check(lib.dualkv_profile_stop(), "dualkv_profile_stop")
    out = {}
    for i in range(lib.dualkv_profile_count()):
        name, n, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        _check(lib.dualkv_profile_kernel(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)),
               "dualkv_profile_kernel")
        out[name.value.decode()] = (int(n.value), float(ms.value))
    return out


# ---------------------------------------------------------------- groups
# `groups` is a sequence of (n_resp, prompt_len, resp_len); the packed rows
# of the groups follow one another (include/dualkv.h, dualkv_fwd_groups).

def _group_array(groups):
    gs = [tuple(int(x) for x in g) for g in groups]
    arr = (Group * max(1, len(gs)))(*[Group(*g) for g in gs])
    return arr, len(gs), gs


def packed_rows(groups) -> int:
    return sum(P + N * R for N, P, R in groups)


def make_group_params(q, k, groups, window=0, softmax_scale=0.0, valid_len=None, impl=IMPL_AUTO) -> Params:
    T = packed_rows(groups)
    _require(q, "q")
    _require(k, "k", dtype=q.dtype)
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != T or k.shape[0] != T or q.shape[2] != k.shape[2]:
        raise ValueError(f"q {tuple(q.shape)} / k {tuple(k.shape)} do not match the groups' {T} rows")
    if valid_len is not None:
        _require(valid_len, "valid_len", dtype=torch.int32, shape=(sum(g[0] for g in groups),))
    return Params(0, 0, 0, q.shape[1], k.shape[1], q.shape[2], window, softmax_scale, _dtype_code(q), impl,
                  None if valid_len is None else valid_len.data_ptr())


def dualkv_repack_groups(src, groups, direction, out=None):
    """dualkv_repack over groups laid out one after the other."""
    lib = load_library()
    arr, n, gs = _group_array(groups)
    _require(src, "src")
    rep = sum(N * (P + R) for N, P, R in gs)
    pk = packed_rows(gs)
    rows_in, rows_out = (rep, pk) if direction == DUALKV_GATHER else (pk, rep)
    if src.shape[0] != rows_in:
        raise ValueError(f"src has {src.shape[0]} rows, expected {rows_in}")
    if out is None:
        out = torch.empty((rows_out,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    _require(out, "out", dtype=src.dtype, shape=(rows_out,) + tuple(src.shape[1:]))
    row_bytes = src[0].numel() * src.element_size() if src.shape[0] else max(1, src.element_size())
    _check(lib.dualkv_repack_groups(_ptr(src), _ptr(out), row_bytes, arr, n, direction, _stream()),
           "dualkv_repack_groups")
    return out


def dualkv_fwd_groups(q, k, v, groups, window=0, softmax_scale=0.0, valid_len=None, impl=IMPL_AUTO,
                      out=None, lse=None):
    """Forward over groups; returns (o [Tld,Hq,D], lse [Hq,Tld] fp32)."""
    lib = load_library()
    arr, n, gs = _group_array(groups)
    p = make_group_params(q, k, gs, window, softmax_scale, valid_len, impl)
    _require(v, "v", dtype=q.dtype, shape=k.shape)
    T, Hq, _ = q.shape
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(out, "out", dtype=q.dtype, shape=q.shape)
    _require(lse, "lse", dtype=torch.float32, shape=(Hq, T))
    _check(lib.dualkv_fwd_groups(ctypes.byref(p), arr, n, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _stream()), "dualkv_fwd_groups")
    return out, lse


def dualkv_bwd_groups_workspace_bytes(q, k, groups, window=0, softmax_scale=0.0, valid_len=None,
                                      impl=IMPL_AUTO) -> int:
    arr, n, gs = _group_array(groups)
    p = make_group_params(q, k, gs, window, softmax_scale, valid_len, impl)
    return int(load_library().dualkv_bwd_groups_workspace_bytes(ctypes.byref(p), arr, n))


def dualkv_bwd_groups(q, k, v, o, lse, dout, groups, window=0, softmax_scale=0.0, valid_len=None,
                      impl=IMPL_AUTO, workspace=None, dq=None, dk=None, dv=None):
    """Backward over groups; returns (dq, dk, dv)."""
    lib = load_library()
    arr, n, gs = _group_array(groups)
    p = make_group_params(q, k, gs, window, softmax_scale, valid_len, impl)
    _require(v, "v", dtype=q.dtype, shape=k.shape)
    _require(o, "o", dtype=q.dtype, shape=q.shape)
    _require(dout, "dout", dtype=q.dtype, shape=q.shape)
    _require(lse, "lse", dtype=torch.float32, shape=(q.shape[1], q.shape[0]))
    need = int(lib.dualkv_bwd_groups_workspace_bytes(ctypes.byref(p), arr, n))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", dtype=torch.uint8)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _require(t, name, dtype=ref.dtype, shape=ref.shape)
    _check(lib.dualkv_bwd_groups(ctypes.byref(p), arr, n, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                 _stream()), "dualkv_bwd_groups")
    return dq, dk, dv


# ------------------------------------------------------- packed layer ops
# bf16 tensors throughout (include/dualkv.h, "A packed transformer layer").

def dualkv_gemm_bf16(a, b, trans_a=False, trans_b=False, residual=None, out=None):
    """C = op(a) op(b) (+ residual) for 2-D bf16 tensors; op transposes the
    stored matrix when its flag is set."""
    lib = load_library()
    for t, n in ((a, "a"), (b, "b")):
        _require(t, n, dtype=torch.bfloat16)
        if t.dim() != 2:
            raise ValueError(f"{n} must be 2-D")
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    Kb, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if out is None else out
    _require(out, "out", dtype=torch.bfloat16, shape=(M, N))
    if residual is not None:
        _require(residual, "residual", dtype=torch.bfloat16, shape=(M, N))
    _check(lib.dualkv_gemm_bf16(int(trans_a), int(trans_b), M, N, K, _ptr(a), a.shape[1], _ptr(b), b.shape[1],
                                _ptr(out), N, _ptr(residual), N, _stream()), "dualkv_gemm_bf16")
    return out


def dualkv_rmsnorm_fwd(x, w, eps=1e-6):
    """(y, rstd) of RMSNorm over the last dimension of a 2-D bf16 x."""
    lib = load_library()
    _require(x, "x", dtype=torch.bfloat16)
    T, H = x.shape
    _require(w, "w", dtype=torch.bfloat16, shape=(H,))
    y = torch.empty_like(x)
    rstd = torch.empty((T,), dtype=torch.float32, device=x.device)
    _check(lib.dualkv_rmsnorm_fwd(T, H, eps, _ptr(x), _ptr(w), _ptr(y), _ptr(rstd), _stream()),
           "dualkv_rmsnorm_fwd")
    return y, rstd


def dualkv_rmsnorm_bwd(x, w, rstd, dy, dres=None):
    """(dx, dw) of RMSNorm; dres (optional) is added to dx."""
    lib = load_library()
    T, H = x.shape
    for t, n in ((x, "x"), (dy, "dy")):
        _require(t, n, dtype=torch.bfloat16, shape=(T, H))
    _require(w, "w", dtype=torch.bfloat16, shape=(H,))
    _require(rstd, "rstd", dtype=torch.float32, shape=(T,))
    if dres is not None:
        _require(dres, "dres", dtype=torch.bfloat16, shape=(T, H))
    ws = torch.empty(max(256, int(lib.dualkv_rmsnorm_bwd_workspace_bytes(T, H))), dtype=torch.uint8,
                     device=x.device)
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    _check(lib.dualkv_rmsnorm_bwd(T, H, _ptr(x), _ptr(w), _ptr(rstd), _ptr(dy), _ptr(dres), _ptr(dx), _ptr(dw),
                                  _ptr(ws), ws.numel(), _stream()), "dualkv_rmsnorm_bwd")
    return dx, dw


def dualkv_rope(x, groups, base=1e4, inverse=False):
    """Rotary embedding in place on x [rows, heads, head_dim] (bf16) of the
    packed groups, at logical positions."""
    lib = load_library()
    _require(x, "x", dtype=torch.bfloat16)
    arr, n, gs = _group_array(groups)
    if x.dim() != 3 or x.shape[0] != packed_rows(gs):
        raise ValueError(f"x {tuple(x.shape)} does not match the groups' {packed_rows(gs)} rows")
    _check(lib.dualkv_rope(arr, n, x.shape[1], x.shape[2], base, int(inverse), _ptr(x), _stream()), "dualkv_rope")
    return x


def dualkv_swiglu_fwd(u, g):
    lib = load_library()
    _require(u, "u", dtype=torch.bfloat16)
    _require(g, "g", dtype=torch.bfloat16, shape=u.shape)
    m = torch.empty_like(u)
    _check(lib.dualkv_swiglu_fwd(u.numel(), _ptr(u), _ptr(g), _ptr(m), _stream()), "dualkv_swiglu_fwd")
    return m


def dualkv_swiglu_bwd(u, g, dm):
    lib = load_library()
    for t, n in ((u, "u"), (g, "g"), (dm, "dm")):
        _require(t, n, dtype=torch.bfloat16, shape=u.shape)
    du, dg = torch.empty_like(u), torch.empty_like(u)
    _check(lib.dualkv_swiglu_bwd(u.numel(), _ptr(u), _ptr(g), _ptr(dm), _ptr(du), _ptr(dg), _stream()),
           "dualkv_swiglu_bwd")
    return du, dg


def make_layer_params(hidden, n_q_heads, n_kv_heads, head_dim, ffn, window=0, rope_base=1e4, norm_eps=1e-6,
                      valid_len=None):
    return LayerParams(hidden, n_q_heads, n_kv_heads, head_dim, ffn, window, rope_base, norm_eps,
                       None if valid_len is None else valid_len.data_ptr())


def _layer_weights(W, cls=LayerWeights):
    return cls(*[W[n].data_ptr() for n in LAYER_WEIGHTS])


def dualkv_layer_saved_bytes(p, groups):
    arr, n, _ = _group_array(groups)
    return int(load_library().dualkv_layer_saved_bytes(ctypes.byref(p), arr, n))


def dualkv_layer_workspace_bytes(p, groups):
    arr, n, _ = _group_array(groups)
    return int(load_library().dualkv_layer_workspace_bytes(ctypes.byref(p), arr, n))


def dualkv_layer_fwd(x, W, groups, p, saved=None, out=None):
    """Forward of the packed layer: returns (y, saved)."""
    lib = load_library()
    arr, n, gs = _group_array(groups)
    _require(x, "x", dtype=torch.bfloat16, shape=(packed_rows(gs), p.hidden))
    need = int(lib.dualkv_layer_saved_bytes(ctypes.byref(p), arr, n))
    saved = torch.empty(max(256, need), dtype=torch.uint8, device=x.device) if saved is None else saved
    out = torch.empty_like(x) if out is None else out
    w = _layer_weights(W)
    _check(lib.dualkv_layer_fwd(ctypes.byref(p), arr, n, ctypes.byref(w), _ptr(x), _ptr(out), _ptr(saved),
                                saved.numel(), _stream()), "dualkv_layer_fwd")
    return out, saved


def dualkv_layer_bwd(x, saved, dy, W, groups, p, workspace=None, dx=None, grads=None):
    """Backward of the packed layer: returns (dx, {weight name: gradient})."""
    lib = load_library()
    arr, n, gs = _group_array(groups)
    _require(dy, "dy", dtype=torch.bfloat16, shape=x.shape)
    need = int(lib.dualkv_layer_workspace_bytes(ctypes.byref(p), arr, n))
    if workspace is None:
        workspace = torch.empty(max(256, need), dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x) if dx is None else dx
    grads = {k: torch.empty_like(W[k]) for k in LAYER_WEIGHTS} if grads is None else grads
    w, g = _layer_weights(W), _layer_weights(grads, LayerGrads)
    _check(lib.dualkv_layer_bwd(ctypes.byref(p), arr, n, ctypes.byref(w), _ptr(x), _ptr(saved), saved.numel(),
                                _ptr(dy), _ptr(dx), ctypes.byref(g), _ptr(workspace), workspace.numel(),
                                _stream()), "dualkv_layer_bwd")
    return dx, grads
