"""Builds libattnjvp.so (HIP kernels for gfx950 + host C ABI) in-tree with hipcc.

Usage: python -m attention_jvp_causal_amd.build  (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libattnjvp.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["attn_jvp_fwd.hip", "attn_fwd_q32.hip", "attn_bwd.hip", "attn_jvp_api.cpp", "mask_desc.cpp"]
ARCH = os.environ.get("AJ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# Per-source scheduler choice. The gradient kernels run 1-2.5 % faster under
# LLVM's iterative ILP scheduler than under the default (same-box A/B, both head
# dims) and still spill nothing. The 32-row forward kernels gain about as much but
# spill under it, and the 16-row JVP kernel gains nothing: both keep the default.
SOURCE_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def compile_flags(src: str | None = None):
    """hipcc flags shared by every source, plus the per-source ones for `src`."""
    hip = src is None or src.endswith(".hip")
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 instructions stay off: plain float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        # kernels never produce NaN (masked scores are -inf and guarded), so
        # fmaxf needs no NaN canonicalisation; the host sources keep IEEE NaN
        # semantics (their argument checks test for NaN)
        *(["-fno-honor-nans"] if hip else []),
        # MFMA accumulators in VGPRs: the online-softmax rescale multiplies them
        # with VALU ops, which cannot address AGPRs
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        f"-I{os.path.join(ROOT, 'include')}",
        *SOURCE_FLAGS.get(src, []),
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cc = hipcc()
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *compile_flags(src), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed for {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
