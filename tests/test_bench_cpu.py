"""The benchmark's host-side contract, checked without a GPU: the byte
accounting behind GB/s and the roofline (minimal bytes of the workloads,
written out here from their shapes), the one-GPU rule, and that without a
GPU it fails loudly instead of timing anything on the CPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


# read x + read w + write y once; w holds K = 2 m1 m2 (3D: 4 m1 m2 m3)
# complex modes of Ci x Co
@pytest.mark.parametrize("name,dtype,expect", [
    ("c0", "f32", 20_480),
    ("c1", "f32", 71_303_168),
    ("c1", "f16", 35_651_584),
    ("c2", "f16", 570_425_344),
    ("c2", "bf16", 570_425_344),
    ("c3", "f32", 402_653_184),
])
def test_minimal_bytes(name, dtype, expect):
    assert wl.CONFIGS[name].minimal_bytes(dtype) == expect


def test_backward_minimal_bytes():
    # 128^2 fp32: x, dL/dy, grad_x (3 x 32 MiB) + w, grad_w (2 x 4 MiB)
    assert bench.backward_minimal_bytes(wl.CONFIGS["c1"], "f32") == 3 * 33_554_432 + 2 * 4_194_304


def test_per_launch_bytes_2d():
    # forward planes: x + forward spectra; contraction: spectra in + w + spectra out;
    # inverse planes: spectra + y (complex fp32 spectra, 8 bytes per mode)
    cfg = wl.CONFIGS["c2"]
    b = bench._bytes_per_launch(cfg, "f16")
    x = 32 * 64 * 256 * 256 * 2
    xh = 32 * 64 * 2 * 32 * 32 * 8
    w = 2 * 32 * 32 * 64 * 64 * 4
    assert b["fno_fwd_plane_mx"] == x + xh
    assert b["fno_contract"] == xh + w + xh
    assert b["fno_inv_plane_mx"] == xh + x


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert r.stdout.strip() == ""
