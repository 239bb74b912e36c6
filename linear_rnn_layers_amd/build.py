"""Build the gfx950 HIP library in-tree: linear_rnn_layers_amd/liblinattn.so.

One translation unit (csrc/la_api.hip, which includes the kernels) compiled
with hipcc for gfx950 only.  Packed-FP32 instruction selection is disabled
for all device code, and MFMA results are kept in ordinary VGPRs (the
accumulators are read by vector code after every product, which the AGPR
form would turn into copies).
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "la_api.hip")
HEADERS = [os.path.join(PKG, "csrc", h) for h in ("la_device.h", "la_kernels.h", "la_decay.h", "la_feature.h", "la_bwd2.h", "la_wide.h")] + [
    os.path.join(ROOT, "include", "la.h")]
LIB = os.path.join(PKG, "liblinattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def command(out: str = LIB) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-o", out, SRC]


def build(verbose: bool = False) -> str:
    """Compile unconditionally (atomic replace of the library file)."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
        if msgs:
            print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in [SRC] + HEADERS)


def ensure_built() -> str:
    """Build only when no library exists (tests, smoke and bench load what is built)."""
    if not os.path.exists(LIB):
        build()
    return LIB
