"""The C ABI libraries load on the host and export every symbol their headers
declare; argument validation rejects bad calls before anything reaches HIP.

No kernel is launched here (no GPU in this environment): every call below fails
validation, or has rows == 0, and returns before the first HIP runtime call.
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from memory_bound_elementwise_amd import build as mbuild
from memory_bound_elementwise_amd import load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_TO_LIB = {"swiglu_probs.h": "swiglu_probs", "hbm_probe.h": "hbm_probe",
                 "moe_elementwise.h": "moe_elementwise"}


def declared_functions(header: str):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*\b([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def built():
    for name in HEADER_TO_LIB.values():
        if not os.path.exists(mbuild.lib_path(name)):
            mbuild.build_lib(name)


def test_every_header_is_mapped():
    heads = sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert heads == sorted(HEADER_TO_LIB)


@pytest.mark.parametrize("header,lib", sorted(HEADER_TO_LIB.items()))
def test_library_exports_declared_symbols(built, header, lib):
    names = declared_functions(os.path.join(ROOT, "include", header))
    assert names, f"no declarations parsed from {header}"
    so = ctypes.CDLL(mbuild.lib_path(lib))
    missing = [n for n in names if not hasattr(so, n)]
    assert not missing, f"{lib} does not export {missing}"
    nm = subprocess.run(["nm", "-D", "--defined-only", mbuild.lib_path(lib)],
                        capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), f"{n} not a defined text symbol"


def test_swiglu_declarations_expected():
    names = declared_functions(os.path.join(ROOT, "include", "swiglu_probs.h"))
    for n in ("swiglu_probs_fwd", "swiglu_probs_bwd", "swiglu_probs_fwd_ex", "swiglu_probs_bwd_ex",
              "swiglu_probs_fwd_timed", "swiglu_probs_bwd_timed",
              "swiglu_probs_status_string", "swiglu_probs_abi_version",
              "swiglu_probs_last_hip_error", "swiglu_probs_default_workgroups"):
        assert n in names


A16 = 1 << 20  # a 16-byte aligned fake address; never dereferenced on these paths


def fwd(lib, x=A16, probs=A16 + (1 << 24), y=A16 + (2 << 24), rows=4, inter=8, limit=7.0,
        n_used=None, perm=None, zp=0, nwg=0):
    return lib.swiglu_probs_fwd_ex(x, probs, y, rows, inter, limit, n_used, perm, zp, None, nwg)


def bwd(lib, x=A16, probs=A16 + (1 << 24), gy=A16 + (2 << 24), gx=A16 + (3 << 24),
        gp=A16 + (4 << 24), rows=4, inter=8, limit=7.0, n_used=None, perm=None, zp=0, nwg=0):
    return lib.swiglu_probs_bwd_ex(x, probs, gy, gx, gp, rows, inter, limit, n_used, perm, zp,
                                   None, nwg)


def test_validation_fwd():
    lib = load_library()
    assert fwd(lib, rows=0) == 0                       # empty: no launch
    assert fwd(lib, rows=0, x=None, y=None, probs=None) == 0
    assert fwd(lib, rows=-1) == 1
    assert fwd(lib, inter=0) == 1
    assert fwd(lib, inter=-8) == 1
    assert fwd(lib, inter=12) == 2                     # not a multiple of 8
    assert fwd(lib, limit=float("nan")) == 1
    assert fwd(lib, limit=0.0) == 1
    assert fwd(lib, limit=-7.0) == 1
    assert fwd(lib, nwg=-1) == 1
    assert fwd(lib, nwg=1 << 24) == 1                   # past 2^32 - 1 work-items per dispatch
    assert fwd(lib, nwg=2 ** 31 - 1) == 1
    assert fwd(lib, x=None) == 1
    assert fwd(lib, probs=None) == 1
    assert fwd(lib, y=None) == 1
    assert fwd(lib, x=A16 + 8) == 2
    assert fwd(lib, y=A16 + (2 << 24) + 2) == 2
    assert fwd(lib, probs=A16 + (1 << 24) + 2) == 2
    assert fwd(lib, n_used=A16 + (5 << 24) + 1) == 2
    assert fwd(lib, perm=A16 + (6 << 24) + 3) == 2
    assert fwd(lib, y=A16 + 16) == 1                    # y overlaps x
    assert fwd(lib, y=A16 + (1 << 24)) == 1             # y overlaps probs
    assert fwd(lib, rows=1 << 40) == 1                  # too many rows
    assert fwd(lib, inter=1 << 40) == 1


def test_validation_bwd():
    lib = load_library()
    assert bwd(lib, rows=0) == 0
    assert bwd(lib, rows=-3) == 1
    assert bwd(lib, inter=20) == 2
    assert bwd(lib, nwg=1 << 24) == 1
    assert bwd(lib, limit=float("nan")) == 1
    assert bwd(lib, x=None) == 1
    assert bwd(lib, gy=None) == 1
    assert bwd(lib, gx=None) == 1
    assert bwd(lib, probs=None) == 1
    assert bwd(lib, gp=A16 + (4 << 24) + 1) == 2
    assert bwd(lib, gx=A16 + (3 << 24) + 4) == 2
    assert bwd(lib, gx=A16) == 1                        # grad_x over x
    assert bwd(lib, gx=A16 + (2 << 24)) == 1            # grad_x over grad_y
    assert bwd(lib, gp=A16 + (1 << 24)) == 1            # grad_probs over probs
    assert bwd(lib, gp=A16 + (3 << 24) + 16) == 1       # grad_probs inside grad_x
    assert bwd(lib, perm=A16 + (3 << 24)) == 1          # map overlaps an output


def test_status_strings_and_version():
    lib = load_library()
    assert lib.swiglu_probs_abi_version() == 1
    for st in range(4):
        assert lib.swiglu_probs_status_string(st)
    assert lib.swiglu_probs_status_string(99) == b"unknown status"


def test_probe_validation(built):
    so = ctypes.CDLL(mbuild.lib_path("hbm_probe"))
    so.hbm_probe_stream.restype = ctypes.c_int
    so.hbm_probe_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    s = (ctypes.c_void_p * 1)(A16)
    d = (ctypes.c_void_p * 1)(A16 + (1 << 24))
    assert so.hbm_probe_stream(s, 1, d, 1, 0, 0, None) == 0
    assert so.hbm_probe_stream(s, 0, d, 1, 4, 0, None) == 1
    assert so.hbm_probe_stream(s, 1, d, 3, 4, 0, None) == 1
    d2 = (ctypes.c_void_p * 1)(A16 + 16)
    assert so.hbm_probe_stream(s, 1, d2, 1, 4, 0, None) == 1   # overlap
    assert so.hbm_probe_stream(s, 1, d, 1, 4, 1 << 24, None) == 1
    assert so.hbm_probe_stream(s, 1, d, 1, (1 << 44) + 1, 0, None) == 1   # byte count past 2^48
    assert so.hbm_probe_stream(s, 1, d, 1, 2 ** 63 - 1, 0, None) == 1


def test_probe_one_way_validation(built):
    """The read-only and write-only streams check their arguments before any launch."""
    so = ctypes.CDLL(mbuild.lib_path("hbm_probe"))
    so.hbm_probe_read.restype = so.hbm_probe_fill.restype = ctypes.c_int
    so.hbm_probe_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    so.hbm_probe_fill.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
    s = (ctypes.c_void_p * 3)(A16, A16 + (1 << 24), A16 + (2 << 24))
    sink = A16 + (3 << 24)
    assert so.hbm_probe_read(s, 3, 0, 7, sink, 0, None) == 0           # empty: no launch
    assert so.hbm_probe_read(s, 0, 4, 7, sink, 0, None) == 1
    assert so.hbm_probe_read(s, 4, 4, 7, sink, 0, None) == 1
    assert so.hbm_probe_read(s, 1, 4, 7, None, 0, None) == 1            # no sink
    assert so.hbm_probe_read(s, 1, 4, 7, sink + 8, 0, None) == 1        # misaligned sink
    assert so.hbm_probe_read(s, 1, 4, 7, A16 + 16, 0, None) == 1        # sink inside a source
    assert so.hbm_probe_read(s, 1, -1, 7, sink, 0, None) == 1
    assert so.hbm_probe_read(s, 1, (1 << 44) + 1, 7, sink, 0, None) == 1
    assert so.hbm_probe_read(s, 1, 4, 7, sink, 1 << 24, None) == 1
    bad = (ctypes.c_void_p * 1)(A16 + 4)
    assert so.hbm_probe_read(bad, 1, 4, 7, sink, 0, None) == 1
    d = (ctypes.c_void_p * 2)(A16, A16 + 32)
    assert so.hbm_probe_fill(d, 1, 0, 7, 0, None) == 0                  # empty: no launch
    assert so.hbm_probe_fill(d, 0, 4, 7, 0, None) == 1
    assert so.hbm_probe_fill(d, 3, 4, 7, 0, None) == 1
    assert so.hbm_probe_fill(d, 2, 4, 7, 0, None) == 1                  # the two overlap
    assert so.hbm_probe_fill(bad, 1, 4, 7, 0, None) == 1
    assert so.hbm_probe_fill(d, 1, 2 ** 63 - 1, 7, 0, None) == 1


def test_moe_validation():
    from memory_bound_elementwise_amd.moe_elementwise import load_library as load_moe
    lib = load_moe()
    a, b, c, d = A16, A16 + (1 << 24), A16 + (2 << 24), A16 + (3 << 24)
    assert lib.moe_residual_add(a, b, c, d, 0, 0, None, 0) == 0           # empty: no launch
    assert lib.moe_residual_add(a, b, c, d, -1, 0, None, 0) == 1
    assert lib.moe_residual_add(a, b, c, d, 8, 7, None, 0) == 1            # bad dtype
    assert lib.moe_residual_add(a + 2, b, c, d, 8, 0, None, 0) == 2
    assert lib.moe_residual_add(a, b, c, a + 16, 64, 0, None, 0) == 1      # partial overlap
    assert lib.moe_residual_add(None, b, c, d, 8, 0, None, 0) == 1
    assert lib.moe_residual_add(a, b, c, d, 8, 0, None, -1) == 1
    assert lib.moe_residual_add(a, b, c, d, 8, 0, None, 1 << 24) == 1     # past the dispatch limit
    assert lib.moe_residual_add(a, b, c, d, (1 << 48) + 8, 0, None, 0) == 1  # past 2^48 elements
    assert lib.moe_residual_add(a, b, c, d, 2 ** 63 - 1, 2, None, 0) == 1
    f = lib.moe_router_weight_fwd
    assert f(a, 0, b, c, 0, 0, 8, None, 0) == 0
    assert f(a, 0, b, c, 1, 4, 8, None, 0) == 1                           # out must be x's type or fp32
    assert f(a, 0, b, c, 2, 4, 12, None, 0) == 2                          # hidden % 8
    assert f(a, 0, b + 2, c, 2, 4, 8, None, 0) == 2
    assert f(a, 0, b, a, 0, 4, 8, None, 0) == 1                           # out over x
    assert f(a, 0, b, c, 0, 4, 8, None, 1 << 24) == 1
    g = lib.moe_router_weight_bwd
    assert g(a, 0, None, 0, b, c, d, 4, 8, None, 0) == 1                  # grad_probs needs x
    assert g(a, 0, A16 + (5 << 24), 0, b, c, d, 4, 8, None, 1 << 24) == 1
    sq = lib.moe_squared_relu_probs_fwd
    assert sq(a, b, c, 4, 8, 1, 0.0, None, None, 0, None, 0) == 1         # clamp needs scale > 0
    assert sq(a, b, c, 4, 8, 1, float("inf"), None, None, 0, None, 0) == 1
    assert sq(a, b, c, 4, 8, 1, float("nan"), None, None, 0, None, 0) == 1
    assert sq(a, b, c, 0, 8, 0, 0.0, None, None, 0, None, 0) == 0
    assert sq(a, b, a, 4, 8, 0, 0.0, None, None, 0, None, 0) == 1
    assert sq(a, b, c, 4, 8, 0, 0.0, None, None, 0, None, 1 << 24) == 1
    sb = lib.moe_squared_relu_probs_bwd
    e = A16 + (4 << 24)
    assert sb(a, b, c, d, e, 0, 8, 1, 2.0, None, None, 0, None, 0) == 0   # empty: no launch
    assert sb(a, b, c, d, e, 4, 8, 1, -2.0, None, None, 0, None, 0) == 1  # clamp needs scale > 0
    assert sb(a, b, c, d, e, 4, 12, 0, 0.0, None, None, 0, None, 0) == 2  # hidden % 8
    assert sb(a, b, c + 8, d, e, 4, 8, 0, 0.0, None, None, 0, None, 0) == 2   # grad_y alignment
    assert sb(a, b, c, d + 8, e, 4, 8, 0, 0.0, None, None, 0, None, 0) == 2   # grad_x alignment
    assert sb(a, b, c, d, e + 2, 4, 8, 0, 0.0, None, None, 0, None, 0) == 2   # grad_probs alignment
    assert sb(a, b, None, d, e, 4, 8, 0, 0.0, None, None, 0, None, 0) == 1    # grad_y required
    assert sb(a, b, c, None, e, 4, 8, 0, 0.0, None, None, 0, None, 0) == 1    # grad_x required
    assert sb(a, b, c, c, e, 4, 8, 0, 0.0, None, None, 0, None, 0) == 1       # grad_x over grad_y
    assert sb(a, b, c, d, b, 4, 8, 0, 0.0, None, None, 0, None, 0) == 1       # grad_probs over probs
    assert sb(a, b, c, d, d + 16, 4, 8, 0, 0.0, None, None, 0, None, 0) == 1  # outputs overlap
    assert sb(a, b, c, d, e, 4, 8, 0, 0.0, d, None, 0, None, 0) == 1         # n_used under grad_x
    assert sb(a, b, c, d, e, 4, 8, 0, 0.0, None, None, 0, None, 1 << 24) == 1
    u = lib.moe_unpermute_expert_order
    assert u(a, 10, b, None, c, 2, 0, 8, 4, None, 0) == 0
    assert u(a, 10, b, None, c, 1, 4, 8, 4, None, 0) == 1                 # fp16 out not supported
    assert u(a, 10, b, None, c, 2, 4, 8, 0, None, 0) == 1                 # no experts
    assert u(a, 10, b, None, c, 2, 4, 8, 2000, None, 0) == 1
    assert u(a, 10, b + 1, None, c, 2, 4, 8, 4, None, 0) == 2
    assert u(a, 10, b, None, c, 2, 4, 8, 4, None, 1 << 24) == 1
    assert lib.moe_elementwise_abi_version() == 1


def test_headers_compile_as_c(tmp_path):
    """The headers are plain C: a C11 translation unit includes them, takes every
    declared function's address, and links against the libraries."""
    import shutil
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    names = []
    for h in HEADER_TO_LIB:
        names += declared_functions(os.path.join(ROOT, "include", h))
    src = tmp_path / "abi_check.c"
    src.write_text("#include \"swiglu_probs.h\"\n#include \"moe_elementwise.h\"\n#include \"hbm_probe.h\"\n"
                   "#include <stdio.h>\ntypedef void (*fn_t)(void);\nstatic const fn_t table[] = {\n"
                   + "".join(f"    (fn_t)&{n},\n" for n in names)
                   + "};\nint main(void) {\n    unsigned n = 0;\n"
                   "    for (unsigned i = 0; i < sizeof table / sizeof table[0]; ++i) n += table[i] != 0;\n"
                   "    printf(\"%u\\n\", n);\n    return 0;\n}\n")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    libdir = os.path.dirname(mbuild.lib_path("swiglu_probs"))
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", "-isystem", f"{rocm}/include", str(src), "-o", str(tmp_path / "abi_check"),
           f"-L{libdir}", "-lswiglu_probs", "-lmoe_elementwise", "-lhbm_probe",
           f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
