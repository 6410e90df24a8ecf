"""Build-time guards on the generated gfx950 code (CPU only: hipcc cross-compiles).

The key-tile DMA is issued from a small asm block that sets m0; that is safe
only while the compiler itself keeps nothing in m0 in these kernels.
"""
import os
import re
import shutil
import subprocess

import pytest

from attention_jvp_causal_amd import build as B


def _device_asm(tmp_path):
    text = []
    for src in (x for x in B.SOURCES if x.endswith(".hip")):
        out = tmp_path / (src + ".s")
        cmd = [B.hipcc(), *B.compile_flags(src), "-x", "hip", "-S", "--cuda-device-only",
               os.path.join(B.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text.append(out.read_text())
    return "\n".join(text)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_m0_only_used_by_the_dma_asm_blocks(tmp_path):
    asm = _device_asm(tmp_path)
    kernels = re.findall(r"^(_ZN2aj\w+kernel\w+):", asm, flags=re.M)
    assert any("bf16" in k for k in kernels) and any("f32" in k for k in kernels)
    assert any("attn_bwd_dq" in k for k in kernels) and any("attn_bwd_dkdv" in k for k in kernels)
    inside = False
    outside_uses = []
    for line in asm.splitlines():
        if "ASMSTART" in line:
            inside = True
        elif "ASMEND" in line:
            inside = False
        elif re.search(r"\bm0\b", line.split(";")[0]) and not inside:
            outside_uses.append(line.strip())
    assert not outside_uses, outside_uses[:5]
    # no private (scratch) segment in the hot kernels
    for spill in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm):
        assert int(spill) == 0


# Waves per SIMD each kernel is built for.  A kernel at w waves must fit 512 / w
# VGPRs (rounded down to the 8-register allocation granule); more would
# silently cost occupancy, which the d = 64 kernels depend on.
OCCUPANCY = [
    (r"attn_jvp_fwd_bf16_q16_kernelILi128E", 2),
    (r"attn_jvp_fwd_bf16_q32_kernelILi128ELb.ELb0E", 2),   # d = 128 primal forward
    (r"attn_jvp_fwd_bf16_q32_kernelILi64ELb.ELb1E", 2),    # d = 64 JVP
    (r"attn_jvp_fwd_bf16_q32_kernelILi64ELb.ELb0E", 3),    # d = 64 primal forward
    (r"attn_bwd_dq32_kernelILi128E", 2),
    (r"attn_bwd_dq32_kernelILi64E", 3),
    (r"attn_bwd_dkdv_kernelILi128E", 2),
    (r"attn_bwd_dkdv32_kernelILi64E", 2),
]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_register_budgets_keep_the_intended_occupancy(tmp_path):
    asm = _device_asm(tmp_path)
    names = re.findall(r"\.amdhsa_kernel (\S+)", asm)
    vgprs = [int(v) for v in re.findall(r"\.amdhsa_next_free_vgpr (\d+)", asm)]
    assert len(names) == len(vgprs) and names
    seen = set()
    for name, v in zip(names, vgprs):
        for pat, waves in OCCUPANCY:
            if re.search(pat, name):
                budget = (512 // waves) // 8 * 8
                assert v <= budget, f"{name}: {v} VGPRs exceed {budget} ({waves} waves per SIMD)"
                seen.add(pat)
    assert seen == {p for p, _ in OCCUPANCY}, f"kernels not found: {set(p for p, _ in OCCUPANCY) - seen}"
