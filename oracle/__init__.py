"""fp64 CPU oracle for shared-prompt (DualKV) attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls,
links or executes this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path: the only module both sides use is ``workloads`` (the seeded
input generator, which holds none of the attention arithmetic).

What is computed follows "DualKV: Shared-Prompt Flash Attention for
Efficient RL Training with Large Rollouts and Long Contexts" (arXiv
2605.15422), Abstract: the method is an exact re-arrangement of standard
causal softmax attention over N sequences that share a P-token prompt, so
the oracle is standard attention written out plainly:

* ``oracle.mask``        packed-row bookkeeping and the visibility
                         definition (two disjoint KV regions);
* ``oracle.dense``       O1: dense attention over the packed P+NR layout
                         with the explicit visibility mask (tiny inputs);
* ``oracle.replicated``  O2: the N replicated (P+R)-token causal
                         sequences, standard attention + its analytic
                         backward per sequence, then the fold of prompt
                         gradients over N (the graded oracle);
* ``oracle.repack``      the N(P+R) <-> P+NR row maps;
* ``oracle.groups``      several prompt groups in one packed micro-batch;
* ``oracle.rows``        selected rows of the outputs, for full-size checks;
* ``oracle.layer``       a pre-norm decoder layer (RMSNorm, RoPE at logical
                         positions, attention, SwiGLU MLP) on packed rows;
* ``oracle.rounding``    the per-element error envelope of a bf16 backward
                         (a tolerance model for ill-conditioned inputs).

All floating point is fp64.  Parity of every function is pinned by the
``-m "not gpu"`` tests (closed forms, library routines, finite
differences, sum rules); see ``tests/test_oracle_*.py``.
"""
from . import mask, dense, replicated, repack, groups, layer, rounding  # noqa: F401
