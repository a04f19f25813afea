"""Build the plain-C check of the activation's C ABI (test infrastructure).

The program links the HIP library (memory_bound_elementwise_amd/_lib) and the CPU
oracle (oracle/liboracle_swiglu.so) and finds them at run time through rpaths
relative to its own location, so the built tree can move.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "swiglu_c_check.c")
BINARY = os.path.join(HERE, "swiglu_c_check")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C ABI check")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib = os.path.join(ROOT, "memory_bound_elementwise_amd", "_lib")
    orc = os.path.join(ROOT, "oracle")
    tmp = BINARY + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", "-isystem", f"{rocm}/include", SOURCE, "-o", tmp,
           f"-L{lib}", "-lswiglu_probs", f"-L{orc}", "-loracle_swiglu", f"-L{rocm}/lib", "-lamdhip64",
           "-lm", "-lpthread",
           "-Wl,-rpath,$ORIGIN/../../memory_bound_elementwise_amd/_lib",
           "-Wl,-rpath,$ORIGIN/../../oracle", f"-Wl,-rpath,{rocm}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build of the C ABI check failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, BINARY)
    return BINARY


if __name__ == "__main__":
    print(build())
