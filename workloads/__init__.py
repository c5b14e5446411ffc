"""Seeded synthetic workloads for shared-prompt attention.

This module is the only code that both the fp64 oracle and the HIP path
use: it draws the random inputs and describes the shapes.  It holds none
of the attention arithmetic (no masks, no softmax, no gradients).

The workload shapes follow the problem statement of "DualKV: Shared-Prompt
Flash Attention for Efficient RL Training with Large Rollouts and Long
Contexts" (arXiv 2605.15422, Abstract): one shared prompt of P tokens and
N sampled responses of R tokens, packed as P + N*R rows.  The concrete
sizes (Qwen3-8B-, 30B-MoE- and Gemma-hybrid-shaped layers) are the
benchmark layer shapes; the pages name no dataset, so i.i.d. Gaussian
activations of those shapes stand in for real hidden states.

Draw order per workload (one ``numpy.random.default_rng(seed)``):
  1. per-response valid lengths, only if the workload has them:
     ``rng.integers(lo, hi, endpoint=True, size=N)``;
  2. Q, K, V, dO, each ``rng.standard_normal(shape, dtype=float32)`` in
     packed ``[T, H, D]`` C order (padded rows included);
  3. multiplied by ``value_scale`` (exact in fp32 for 0.5 and 1.0);
  4. rounded to bfloat16 (round to nearest, ties to even) when the
     workload dtype is bf16.  The arrays stay float32 but hold values
     that bf16 represents exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    n_resp: int           # N
    prompt_len: int       # P
    resp_len: int         # R (padded)
    n_q_heads: int        # Hq
    n_kv_heads: int       # Hkv
    head_dim: int         # D
    window: int = 0       # <= 0: no sliding window
    seed: int = 0
    value_scale: float = 0.5
    len_range: Optional[tuple] = None   # inclusive (lo, hi) for valid lengths
    description: str = ""

    @property
    def packed_len(self) -> int:
        return self.prompt_len + self.n_resp * self.resp_len

    @property
    def replicated_len(self) -> int:
        return self.n_resp * (self.prompt_len + self.resp_len)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The benchmark layer shapes.  Softmax scale is 1/sqrt(D) throughout.
WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "f32", 4, 64, 32, 2, 2, 64, 0, seed=0, value_scale=1.0,
        description="tiny exactness case, fp32, unit-variance inputs"),
    "qwen3_8b": Workload(
        "qwen3_8b", "bf16", 32, 8192, 1024, 32, 8, 128, 0, seed=1,
        description="Qwen3-8B-shaped GRPO attention layer"),
    "dapo_long": Workload(
        "dapo_long", "bf16", 16, 8192, 4096, 32, 8, 128, 0, seed=2,
        len_range=(1024, 4096),
        description="DAPO-style layer, response lengths uniform in [1024, 4096]"),
    "moe_30b": Workload(
        "moe_30b", "bf16", 32, 16384, 2048, 32, 4, 128, 0, seed=3,
        description="30B-MoE-shaped attention layer, one GPU's share"),
    "gemma_global": Workload(
        "gemma_global", "bf16", 8, 57344, 8192, 16, 4, 512, 0, seed=4,
        description="Gemma-style global layer, head dim 512, 64K context"),
    "gemma_swa": Workload(
        "gemma_swa", "bf16", 8, 57344, 8192, 16, 4, 256, 1024, seed=4,
        description="Gemma-style sliding-window layer, window 1024 across "
                    "the prompt/response boundary"),
}

# The unit-variance bf16 copy of the tiny case (the literal max-abs gate
# is meaningful only on unit-variance data).
WORKLOADS["tiny_bf16"] = WORKLOADS["tiny_f32"].replace(name="tiny_bf16", dtype="bf16")


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 holding the rounded values.  Inputs here are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclasses.dataclass
class Inputs:
    q: np.ndarray          # [T, Hq, D] float32
    k: np.ndarray          # [T, Hkv, D]
    v: np.ndarray          # [T, Hkv, D]
    do: np.ndarray         # [T, Hq, D]
    valid_len: Optional[np.ndarray]   # [N] int32, or None (all R)


def generate(w: Workload, with_grad: bool = True) -> Inputs:
    """Draw the seeded inputs of workload ``w`` in the documented order."""
    rng = np.random.default_rng(w.seed)
    valid = None
    if w.len_range is not None:
        lo, hi = w.len_range
        valid = rng.integers(lo, hi, endpoint=True, size=w.n_resp).astype(np.int32)
    T = w.packed_len

    def draw(h):
        a = rng.standard_normal((T, h, w.head_dim), dtype=np.float32)
        if w.value_scale != 1.0:
            a *= np.float32(w.value_scale)
        if w.dtype == "bf16":
            a = round_to_bf16(a)
        return a

    q = draw(w.n_q_heads)
    k = draw(w.n_kv_heads)
    v = draw(w.n_kv_heads)
    do = draw(w.n_q_heads) if with_grad else None
    return Inputs(q, k, v, do, valid)


def softmax_scale(w: Workload) -> float:
    return 1.0 / float(np.sqrt(w.head_dim))


# ------------------------------------------------------------------ groups
# A micro-batch that mixes prompts: groups g = 0.. of (N_g, P_g, R_g) laid
# out one after the other in the packed rows (each group packed as above).

@dataclasses.dataclass(frozen=True)
class GroupedWorkload:
    name: str
    dtype: str
    groups: tuple          # ((N, P, R), ...)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int = 0
    seed: int = 0
    value_scale: float = 0.5
    len_ranges: Optional[tuple] = None  # per group inclusive (lo, hi), or None (all R_g)
    description: str = ""

    @property
    def packed_len(self) -> int:
        return sum(P + N * R for N, P, R in self.groups)

    @property
    def replicated_len(self) -> int:
        return sum(N * (P + R) for N, P, R in self.groups)

    def replace(self, **kw) -> "GroupedWorkload":
        return dataclasses.replace(self, **kw)


GROUPED = {
    # three prompts of different lengths and group sizes in one Qwen3-8B-
    # shaped micro-batch, ragged response lengths (38,912 packed tokens)
    "qwen3_8b_groups": GroupedWorkload(
        "qwen3_8b_groups", "bf16", ((8, 8192, 1024), (8, 4096, 1024), (16, 2048, 512)), 32, 8, 128,
        seed=5, len_ranges=((256, 1024), (512, 1024), (128, 512)),
        description="Qwen3-8B-shaped layer over three prompt groups, ragged responses"),
}


def generate_groups(w: GroupedWorkload, with_grad: bool = True) -> Inputs:
    """Seeded inputs of a grouped workload, drawn like ``generate``: the
    valid lengths of every group in group order (only if ``len_ranges``),
    then Q, K, V, dO over all packed rows."""
    rng = np.random.default_rng(w.seed)
    valid = None
    if w.len_ranges is not None:
        valid = np.concatenate([rng.integers(lo, hi, endpoint=True, size=N)
                                for (N, _, _), (lo, hi) in zip(w.groups, w.len_ranges)]).astype(np.int32)
    T = w.packed_len

    def draw(h):
        a = rng.standard_normal((T, h, w.head_dim), dtype=np.float32)
        if w.value_scale != 1.0:
            a *= np.float32(w.value_scale)
        if w.dtype == "bf16":
            a = round_to_bf16(a)
        return a

    q = draw(w.n_q_heads)
    k = draw(w.n_kv_heads)
    v = draw(w.n_kv_heads)
    do = draw(w.n_q_heads) if with_grad else None
    return Inputs(q, k, v, do, valid)
