"""Host code under AddressSanitizer, UndefinedBehaviorSanitizer and ThreadSanitizer, no GPU
needed.

* The CPU oracle (plain C) is built with gcc and both sanitizers and driven over every
  function, small inputs with every special value and every row rule
  (tests/sanitize/oracle_drive.c).
* The three C-ABI libraries are built with the sanitizers on their host code only
  (hipcc, -Xarch_host before each -fsanitize=) and their argument checks driven from C
  (tests/sanitize/abi_drive.c): every call fails validation or has nothing to do, so
  nothing reaches the HIP runtime or a GPU.
* The oracle's row blocks run on POSIX threads; the same drive under ThreadSanitizer
  checks that no two threads touch the same memory unordered.
* A planted out-of-bounds write and a planted race (two threads' row blocks overlapping
  by one row), each in a copy of the oracle, must be reported, which shows the
  instrumentation is live.

AddressSanitizer must be the first library a program loads, so these tests skip where
the environment preloads a library of its own.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ORACLE_SOURCES = [os.path.join(ROOT, "oracle", "swiglu_oracle.c"), os.path.join(ROOT, "oracle", "moe_oracle.c")]
CFLAGS_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")) or os.path.exists("/etc/ld.so.preload"),
                                reason="a preloaded library would come before the sanitizer runtime")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, env=ENV, **kw)


def _build_oracle_drive(out, sources, flags=CFLAGS_SAN):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math", "-pthread", *flags,
           os.path.join(HERE, "oracle_drive.c"), *sources, "-lm", "-o", out]
    res = _run(cmd)
    assert res.returncode == 0, res.stderr[-3000:]


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    _build_oracle_drive(exe, ORACLE_SOURCES)
    res = _run([exe], timeout=300)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "oracle sanitizer drive: ok" in res.stdout


def test_a_planted_overrun_is_reported(tmp_path):
    """Plant a one-past-the-end write (the router-weight forward's column loop running
    to <= hidden) in a copy of the oracle: AddressSanitizer must stop the drive."""
    src = open(ORACLE_SOURCES[1]).read()
    needle = "for (int64_t h = 0; h < hidden; ++h)\n            store_elem(A->out"
    assert src.count(needle) == 1, "the planted mistake no longer matches the oracle source"
    planted = tmp_path / "moe_oracle_planted.c"
    planted.write_text(src.replace(needle, "for (int64_t h = 0; h <= hidden; ++h)\n            store_elem(A->out"))
    exe = str(tmp_path / "oracle_drive_planted")
    _build_oracle_drive(exe, [ORACLE_SOURCES[0], str(planted)])
    res = _run([exe], timeout=300)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr and "heap-buffer-overflow" in res.stderr, res.stderr[-3000:]


CFLAGS_TSAN = ["-fsanitize=thread", "-g", "-O1"]


def test_oracle_threads_under_tsan(tmp_path):
    exe = str(tmp_path / "oracle_drive_tsan")
    _build_oracle_drive(exe, ORACLE_SOURCES, CFLAGS_TSAN)
    res = _run([exe], timeout=300)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "oracle sanitizer drive: ok" in res.stdout and "ThreadSanitizer" not in res.stderr


@pytest.mark.parametrize("which,needle,planted_text", [
    (0, "blk[t].r1 = r + n;", "blk[t].r1 = r + n + (t + 1 < threads);"),
    (1, "blk[t] = (row_block_t){args, r, r + n, body};", "blk[t] = (row_block_t){args, r, r + n + (t + 1 < threads), body};"),
], ids=["swiglu_oracle", "moe_oracle"])
def test_a_planted_race_is_reported(tmp_path, which, needle, planted_text):
    """Let each thread's block of rows run one row into the next thread's (the last
    block stays in range): two threads then write that row's outputs unordered, and
    ThreadSanitizer must report it (for each oracle's thread split)."""
    src = open(ORACLE_SOURCES[which]).read()
    assert src.count(needle) == 1, "the planted race no longer matches the oracle source"
    planted = tmp_path / "oracle_planted.c"
    planted.write_text(src.replace(needle, planted_text))
    exe = str(tmp_path / "oracle_drive_race")
    sources = list(ORACLE_SOURCES)
    sources[which] = str(planted)
    _build_oracle_drive(exe, sources, CFLAGS_TSAN)
    res = _run([exe], timeout=300)
    assert res.returncode != 0
    assert "ThreadSanitizer: data race" in res.stderr, res.stderr[-3000:]


def test_abi_argument_checks_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    runtimes = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not (os.path.exists(hipcc) and os.path.exists(clang) and runtimes):
        pytest.skip("no ROCm compiler with the host sanitizer runtimes")
    rt_dir = os.path.dirname(runtimes[0])
    csrc = os.path.join(ROOT, "memory_bound_elementwise_amd", "csrc")
    libs = []
    for name in ("swiglu_probs", "moe_elementwise", "hbm_probe"):
        out = str(tmp_path / f"lib{name}.so")
        cmd = [hipcc, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan", f"-I{ROOT}/include", f"-I{csrc}", os.path.join(csrc, f"{name}.hip"), "-o", out]  # noqa: E501
        res = _run(cmd)
        assert res.returncode == 0, res.stderr[-3000:]
        libs.append(name)
    exe = str(tmp_path / "abi_drive")
    cmd = [clang, "-std=c11", "-Wall", "-Wextra", "-Werror", *CFLAGS_SAN, "-shared-libsan", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", "-isystem", f"{ROCM}/include", os.path.join(HERE, "abi_drive.c"), "-o", exe,
           f"-L{tmp_path}", *[f"-l{n}" for n in libs], f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{ROCM}/lib", f"-Wl,-rpath,{rt_dir}"]
    res = _run(cmd)
    assert res.returncode == 0, res.stderr[-3000:]
    res = _run([exe], timeout=300)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "ABI sanitizer drive: ok" in res.stdout
