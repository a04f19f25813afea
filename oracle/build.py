"""Compile the CPU oracle (plain C, gcc) into ``oracle/liboracle_swiglu.so``.

Test infrastructure: the oracle is built so that the tests, the smoke check and
the bench's CPU-baseline leg can call it. Building the checker is not using it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "swiglu_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle_swiglu.so")
MOE_SOURCE = os.path.join(HERE, "moe_oracle.c")
MOE_LIB_PATH = os.path.join(HERE, "liboracle_moe.so")

# No fast-math and no FMA contraction: every fp32 operation is rounded as written.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-pthread"]


def compile_oracle(source: str = SOURCE, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile ``source`` to the shared library ``out`` and return ``out``.

    The library is written to a temporary name first and renamed, so a reader
    never sees a half-written file.
    """
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found to build the oracle")
    out_dir = os.path.dirname(os.path.abspath(out))
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=out_dir)
    os.close(fd)
    try:
        cmd = [cc, *CFLAGS, *extra_flags, "-o", tmp, source, "-lm"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out


def build() -> str:
    """Compile both oracle libraries; returns the SwiGLU one's path."""
    compile_oracle(MOE_SOURCE, MOE_LIB_PATH)
    return compile_oracle()


if __name__ == "__main__":
    print(build())
