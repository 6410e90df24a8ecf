"""Builds libattnjvp.so (HIP kernels for gfx950 + host C ABI) in-tree with hipcc.

Usage: python -m attention_jvp_causal_amd.build  (or call build()).
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libattnjvp.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Hash of every kernel's generated gfx950 code, written next to the library:
# records of counter runs (profiles/traffic_*.json) name the code they were
# taken on, whatever source edits left that code unchanged.
ISA_PATH = os.path.join(PKG, "libattnjvp.isa.json")

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
# The iterative min-register strategy spills nowhere but ran every forward
# kernel 1-7 % slower (the 16-row JVP 7 %); the AMDGPU register-pressure
# trackers and a latency-only schedule metric leave the plain kernels' code as
# it is.
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


def kernel_isa_hashes(asm: str) -> dict:
    """{demangled kernel name: sha256[:16] of its instructions} for the kernels
    in one device assembly listing (comments, blank lines and assembler
    directives left out; branch labels without the function number the
    assembler gives them, which moves when other kernels are added to the
    file)."""
    bodies = {}
    kernels = set(re.findall(r"^\s*\.amdhsa_kernel (\S+)", asm, flags=re.M))
    for m in re.finditer(r"^(\S+):(?:\s*;.*)?$", asm, flags=re.M):
        name = m.group(1)
        if name not in kernels:
            continue
        end = asm.find(".Lfunc_end", m.end())
        lines = []
        for line in asm[m.end():end].splitlines():
            line = line.split(";")[0].split("//")[0].strip()
            if line and not line.startswith("."):
                lines.append(re.sub(r"\.LBB\d+_", ".LBB_", line))
        bodies[name] = hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]
    if not bodies:
        return {}
    names = list(bodies)
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    demangled = r.stdout.splitlines() if r.returncode == 0 else names
    return {d: bodies[n] for n, d in zip(names, demangled)}


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path.
    Also writes the per-kernel code hashes (ISA_PATH)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    noise = "is not a recognized feature for this target"

    def run(src, cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed for {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)

    jobs, objs, asms = [], [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append((src, [cc, *compile_flags(src), *lang, "-c", os.path.join(CSRC, src), "-o", obj]))
        objs.append(obj)
        if src.endswith(".hip"):
            asm = os.path.join(objdir, os.path.splitext(src)[0] + ".s")
            jobs.append((src, [cc, *compile_flags(src), *lang, "-S", "--cuda-device-only", os.path.join(CSRC, src),
                               "-o", asm]))
            asms.append(asm)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        for f in [ex.submit(run, src, cmd) for src, cmd in jobs]:
            f.result()
    isa = {}
    for asm in asms:
        with open(asm) as f:
            isa.update(kernel_isa_hashes(f.read()))
    with open(ISA_PATH + ".tmp", "w") as f:
        json.dump(isa, f, indent=1, sort_keys=True)
    os.replace(ISA_PATH + ".tmp", ISA_PATH)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
