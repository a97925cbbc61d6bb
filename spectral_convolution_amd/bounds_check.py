"""Bounds-check build: the library's host code on the CPU, every launch checked.

    python -m spectral_convolution_amd.bounds_check      # build and run

Compiles every source host-only with FNO_BOUNDS_CHECK defined (each launcher
then states the spans and assumptions of its kernel, csrc/bounds.hpp) and
with the address and undefined-behaviour sanitizers on the host code, links
them with csrc/check/ (a recording HIP runtime whose allocations are known,
and a driver over every public entry point on a spread of shapes) and runs
the result. No GPU is used; no device code is built. Objects and the
program go to spectral_convolution_amd/_build_check/.
"""

import concurrent.futures as cf
import os
import re
import subprocess
import sys

from .build import CSRC, HERE, ROOT, SOURCES, _hipcc

OUT = os.path.join(HERE, "_build_check")
CHECK_SOURCES = ["check/hip_stub.cpp", "check/launch_checks.cpp", "check/driver.cpp"]
FLAGS = [
    "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", "-DFNO_BOUNDS_CHECK",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
    "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
]
CLANG = "/opt/rocm/llvm/bin/clang++"


def _compile(src):
    obj = os.path.join(OUT, src.replace("/", "_").rsplit(".", 1)[0] + ".o")
    r = subprocess.run([_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"bounds-check build failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4) -> str:
    """Compile and link the bounds-check program; returns its path."""
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + CHECK_SOURCES))
    # host-only objects still name the (absent) device code images they would
    # register: define them as empty
    names = set()
    for o in objs:
        r = subprocess.run(["nm", "-u", o], capture_output=True, text=True, check=True)
        names.update(re.findall(r"\b(__hip_fatbin_[A-Za-z0-9_]+)", r.stdout))
    stub = os.path.join(OUT, "images.cpp")
    with open(stub, "w") as f:
        f.write("// empty device-code images of the host-only build\n")
        for n in sorted(names):
            f.write(f'extern "C" char {n}[16];\nchar {n}[16];\n')
    objs.append(stub)
    prog = os.path.join(OUT, "fno_bounds_check")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", *objs,
                        "-lm", "-lpthread", "-o", prog], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"bounds-check link failed:\n{r.stdout}\n{r.stderr}")
    return prog


def run(prog: str, timeout: float = 600.0) -> subprocess.CompletedProcess:
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:allocator_may_return_null=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([prog], capture_output=True, text=True, timeout=timeout, env=env)


if __name__ == "__main__":
    r = run(build())
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    sys.exit(r.returncode)
