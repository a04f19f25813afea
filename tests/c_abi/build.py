"""Build the plain-C checks of the C ABIs (test infrastructure).

swiglu_c_check links the activation's HIP library and its CPU oracle; moe_c_check
links the MoE elementwise library and the MoE oracle. Both find the libraries at run
time through rpaths relative to their own location, so the built tree can move.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))

# program -> (HIP library, oracle library)
PROGRAMS = {
    "swiglu_c_check": ("swiglu_probs", "oracle_swiglu"),
    "moe_c_check": ("moe_elementwise", "oracle_moe"),
}


def _build_one(name: str, hip_lib: str, oracle_lib: str) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C ABI check")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib = os.path.join(ROOT, "memory_bound_elementwise_amd", "_lib")
    orc = os.path.join(ROOT, "oracle")
    binary = os.path.join(HERE, name)
    tmp = binary + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", "-isystem", f"{rocm}/include", os.path.join(HERE, name + ".c"), "-o", tmp,
           f"-L{lib}", f"-l{hip_lib}", f"-L{orc}", f"-l{oracle_lib}", f"-L{rocm}/lib", "-lamdhip64",
           "-lm", "-lpthread",
           "-Wl,-rpath,$ORIGIN/../../memory_bound_elementwise_amd/_lib",
           "-Wl,-rpath,$ORIGIN/../../oracle", f"-Wl,-rpath,{rocm}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build of {name} failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, binary)
    return binary


def build() -> list[str]:
    return [_build_one(name, *libs) for name, libs in PROGRAMS.items()]


if __name__ == "__main__":
    for path in build():
        print(path)
