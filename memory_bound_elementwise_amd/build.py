"""Build the HIP libraries of this package for gfx950, in-tree.

``libswiglu_probs.so`` holds the activation kernels and their C ABI
(``include/swiglu_probs.h``); ``libmoe_elementwise.so`` the MoE elementwise
operations next to it (``include/moe_elementwise.h``); ``libhbm_probe.so`` plain
streaming kernels that measure the practical HBM ceiling and calibrate the hardware
byte counters (``include/hbm_probe.h``). All three are written to
``memory_bound_elementwise_amd/_lib``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
# kernarg preload: the first 14 dwords of kernel arguments arrive in SGPRs when a wave
# starts, so a kernel whose waves each handle one row issues its loads without first
# waiting on the kernel-argument fetch (the kernels order their arguments for it).
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", f"-I{CSRC}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-Wall", "-Wno-unused-result"]

LIBS = {
    "swiglu_probs": ["swiglu_probs.hip"],
    "moe_elementwise": ["moe_elementwise.hip"],
    "hbm_probe": ["hbm_probe.hip"],
}


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    return found


def lib_path(name: str) -> str:
    return os.path.join(LIB_DIR, f"lib{name}.so")


def build_lib(name: str, extra_flags=()) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    out = lib_path(name)
    srcs = [os.path.join(CSRC, s) for s in LIBS[name]]
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=LIB_DIR)
    os.close(fd)
    try:
        cmd = [hipcc(), *HIPFLAGS, f"-I{INCLUDE}", *extra_flags, "-o", tmp, *srcs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"build of {name} failed:\n{' '.join(cmd)}\n{res.stderr}")
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out


def build_all() -> list:
    return [build_lib(name) for name in LIBS]


if __name__ == "__main__":
    for p in build_all():
        print(p)
