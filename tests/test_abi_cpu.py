"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host (validation runs
before any HIP call)."""

import ctypes
import os
import re
import subprocess

import pytest

from spectral_convolution_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fno.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fno_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfno.so not built (run python -m spectral_convolution_amd.build)")
    return _lib.lib()


def test_header_symbols_exported(L):
    names = declared_functions()
    assert "fno_plan_create" in names and "fno_spectral_conv3d" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in fno.h but not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature in the binding"


def test_status_strings(L):
    for code, name in _lib.STATUS_NAMES.items():
        assert L.fno_status_string(code).decode() == name


def _create(L, ndim, batch, ci, co, grid, modes, dtype=0, device=0):
    h = ctypes.c_void_p(12345)
    g = (ctypes.c_int * len(grid))(*grid)
    m = (ctypes.c_int * len(modes))(*modes)
    st = L.fno_plan_create(ctypes.byref(h), ndim, batch, ci, co, g, m, dtype, device)
    return st, h


@pytest.mark.parametrize("args,expect", [
    ((4, 2, 4, 4, (16, 16), (4, 4)), INVALID),          # ndim
    ((2, 0, 4, 4, (16, 16), (4, 4)), INVALID),          # batch
    ((2, 2, 0, 4, (16, 16), (4, 4)), INVALID),          # c_in
    ((2, 2, 4, -1, (16, 16), (4, 4)), INVALID),         # c_out
    ((2, 2, 4, 4, (16, 16), (9, 4)), INVALID),          # m1 > H/2
    ((2, 2, 4, 4, (16, 16), (4, 0)), INVALID),          # m2 < 1
    ((2, 2, 4, 4, (24, 16), (4, 4)), UNSUPPORTED),      # non power of two
    ((2, 2, 4, 4, (4, 16), (2, 4)), UNSUPPORTED),       # axis below 8
    ((2, 2, 4, 4, (512, 16), (4, 4)), UNSUPPORTED),     # axis above 256
    ((2, 2, 4, 4, (16, 256), (4, 64)), UNSUPPORTED),    # register FFT above 32
    ((2, 2, 4, 4, (16, 128), (4, 16)), UNSUPPORTED),    # MP = 16 > H/2 = 8
    ((3, 2, 4, 4, (16, 16, 16), (4, 4, 9)), INVALID),   # m3 > Z/2
    ((2, 2, 4, 4, (16, 16), (4, 4), 7), INVALID),       # dtype
    # batch * channels overflows a 32-bit int: rejected before any use
    ((2, 65535, 65535, 4, (16, 16), (4, 4)), UNSUPPORTED),
    ((2, 65535, 4, 65535, (64, 64), (4, 4)), UNSUPPORTED),
    ((3, 65535, 65535, 65535, (8, 8, 8), (4, 4, 4)), UNSUPPORTED),
])
def test_plan_create_rejects_on_host(L, args, expect):
    st, h = _create(L, *args)
    assert st == expect
    assert h.value is None  # *plan set to NULL on failure


def test_null_arguments(L):
    g = (ctypes.c_int * 2)(16, 16)
    m = (ctypes.c_int * 2)(4, 4)
    assert L.fno_plan_create(None, 2, 2, 4, 4, g, m, 0, 0) == INVALID
    h = ctypes.c_void_p()
    assert L.fno_plan_create(ctypes.byref(h), 2, 2, 4, 4, None, m, 0, 0) == INVALID
    assert L.fno_plan_destroy(None) == OK
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    assert L.fno_spectral_conv2d(None, p, p, p, None) == INVALID
    assert L.fno_spectral_conv3d(None, p, p, p, None) == INVALID
    assert L.fno_spectral_conv2d_backward(None, p, p, p, p, p, None) == INVALID
    assert L.fno_spectral_conv3d_backward(None, p, p, p, p, p, None) == INVALID
    assert L.fno_spectral_conv_forward_save(None, p, p, p, p, None) == INVALID
    assert L.fno_spectral_conv_backward_saved(None, p, p, p, p, p, None) == INVALID
    sz0 = ctypes.c_size_t()
    assert L.fno_plan_saved_bytes(None, ctypes.byref(sz0)) == INVALID
    assert L.fno_weights_pack(None, 0, p, p, p, None) == INVALID
    assert L.fno_weights_unpack(None, 1, p, p, None, None) == INVALID
    n = ctypes.c_int()
    assert L.fno_plan_num_launches(None, ctypes.byref(n)) == INVALID
    sz = ctypes.c_size_t()
    assert L.fno_plan_workspace_bytes(None, ctypes.byref(sz)) == INVALID


def test_plain_c_program_builds_and_links(tmp_path):
    """The header is plain C (c99, pedantic, no warnings) and a C program
    links against the library and calls it (destroying a NULL plan needs no
    GPU)."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_fno.c"
    src.write_text('#include "fno.h"\n'
                   "int main(void) {\n"
                   "  fno_plan_t plan = 0;\n"
                   "  return fno_plan_destroy(plan) == FNO_OK ? 0 : 1;\n"
                   "}\n")
    exe = tmp_path / "use_fno"
    libdir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                        os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lfno",
                        f"-Wl,-rpath,{libdir}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)], timeout=60).returncode == 0


def test_noalloc_rejects_null_plan_on_host(L):
    # argument checks run before any HIP call, so no GPU is needed
    assert L.fno_spectral_conv_noalloc(None, None, None, None, None) == INVALID


def test_launch_shape_calls_reject_null_plan_on_host(L):
    n = ctypes.c_int()
    assert L.fno_plan_set_launch_shape(None, 1) == INVALID
    assert L.fno_plan_get_launch_shape(None, ctypes.byref(n)) == INVALID
    assert L.fno_plan_check(None) == INVALID
