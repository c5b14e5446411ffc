"""Comparison helpers for the GPU parity tests (HIP path vs fp64 oracle)."""
import numpy as np
import torch

import workloads

# Tolerances: relative L2 error over a whole tensor, fp64 in both cases.
REL_L2 = {"f32": 1e-5, "bf16": 1e-2}
# bf16 element gate: |x - y| <= 2e-2 * max(RMS(y), |y|).  On unit-variance
# tensors this is the absolute 2e-2 bound; on tensors whose entries exceed
# one (dV summed over hundreds of queries) or sit far below it (O of the
# 0.5-scaled workloads) it measures the error in the element's own scale,
# since bf16 output rounding alone is 2^-9 of |y|.
MAX_ERR_BF16 = 2e-2


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref):
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def check(name, got, ref, dtype):
    """Assert the documented tolerance; returns (rel-L2, max-abs)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if name == "lse":
        inf_ref, inf_got = np.isneginf(ref), np.isneginf(got)
        assert np.array_equal(inf_ref, inf_got), f"{name}: -inf positions differ"
        got, ref = got[~inf_ref], ref[~inf_ref]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = rel_l2(got, ref)
    mab = float(np.abs(got - ref).max()) if got.size else 0.0
    assert err <= REL_L2[dtype], f"{name}: rel-L2 {err:.3e} > {REL_L2[dtype]}"
    if dtype == "bf16" and name != "lse" and got.size:
        rms = float(np.sqrt(np.mean(ref ** 2)))
        scaled = np.abs(got - ref) / np.maximum(np.maximum(rms, np.abs(ref)), 1e-30)
        worst = float(scaled.max())
        assert worst <= MAX_ERR_BF16, (f"{name}: element error {worst:.3e} of max(RMS, |y|) "
                                       f"> {MAX_ERR_BF16} (max-abs {mab:.3e}, RMS {rms:.3e})")
    return err, mab


def inputs_on_device(w: workloads.Workload, x: workloads.Inputs):
    d = {n: to_dev(getattr(x, n), w.dtype) for n in ("q", "k", "v", "do")}
    d["valid"] = None if x.valid_len is None else torch.from_numpy(x.valid_len).cuda()
    return d
