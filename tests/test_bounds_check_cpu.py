"""The bounds-check build (spectral_convolution_amd/bounds_check.py): the
library's host code compiled host-only with the address and undefined-
behaviour sanitizers, every launcher stating its kernel's spans and
assumptions, run on the CPU against a recording runtime over every public
entry point. Passes when no span or assumption is broken, no sanitizer
fires, and the checker's self-test (planted out-of-range spans) is caught."""

import re
import shutil

import pytest

from spectral_convolution_amd import bounds_check


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc (host-only compile)")
def test_every_launch_in_bounds():
    prog = bounds_check.build()
    r = bounds_check.run(prog)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    m = re.search(r"launches checked: (\d+), bounds reports: (\d+), driver failures: (\d+)", r.stdout)
    assert m, out[-2000:]
    launches, reports, fails = map(int, m.groups())
    assert reports == 0 and fails == 0
    assert launches > 1000
    assert "self-test" in r.stderr and r.stderr.count("bounds: fno_channel_mix") == 3
