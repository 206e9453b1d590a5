"""Build the HIP library in-tree: linear_attention_transformer_amd/liblinattn.so.

Compiles csrc/la_api.hip (which includes the kernels) and csrc/la_layer.hip
(the layer around them; its projections call rocBLAS) for gfx950 with hipcc.
Packed fp32 VALU instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("la_api.hip", "la_layer.hip")]
LIB = os.path.join(PKG, "liblinattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Wall", "-I", os.path.join(ROOT, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in VGPRs: the running states of the causal
           # kernels are both accumulators and A operands, and the AGPR form
           # would keep a copy of them in each register file
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-o", tmp] + SRCS + ["-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the device feature; drop that
    noise = "-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
