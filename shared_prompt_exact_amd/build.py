"""Build libdualkv.so (gfx950) in-tree with hipcc.

Every call compiles every translation unit (in parallel) and links the
shared library next to this file.  Works without a GPU: hipcc
cross-compiles for gfx950.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libdualkv.so")
SOURCES = ["repack.hip", "attn_scalar.hip", "attn_fwd_mfma.hip", "attn_bwd_mfma.hip", "attn_bwd_dq.hip",
           "attn_bwd_dq_wide.hip", "attn_bwd_dkdv_wide.hip", "api.hip", "profile.hip", "gemm.hip", "layer_ops.hip", "layer.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"),
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA results in ordinary VGPRs (accumulation registers then serve as
# overflow): the kernels of two waves per SIMD stop spilling to scratch.
# Not for the one-wave-per-SIMD kernels whose accumulators live in the
# accumulation registers.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACCUMULATORS = {"attn_bwd_dq_wide.hip", "attn_bwd_dkdv_wide.hip"}


def _compile(src: str) -> tuple[str, int, str]:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    extra = [] if src in AGPR_ACCUMULATORS else VGPR_FORM
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    return obj, p.returncode, msg


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    failed = [(o, m) for o, rc, m in results if rc != 0]
    if verbose:
        for o, rc, m in results:
            if m.strip():
                print(m, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(m for _, m in failed))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _, _ in results]]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
