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
    # from the saved spectra: those instead of x, the rest unchanged
    assert bench.backward_saved_minimal_bytes(wl.CONFIGS["c1"], "f32", 1000) == 1000 + 2 * 33_554_432 + 2 * 4_194_304


def test_per_launch_bytes_2d():
    # algorithmic bytes of each step: x for the forward planes, w for the
    # contraction, y for the inverse planes; the spectra they exchange
    # (complex fp32, 8 bytes per mode) are counted apart
    cfg = wl.CONFIGS["c2"]
    x = 32 * 64 * 256 * 256 * 2
    xh = 32 * 64 * 2 * 32 * 32 * 8
    w = 2 * 32 * 32 * 64 * 64 * 4
    assert bench._kernel_bytes(cfg, "f16", "fno_fwd_plane_mx") == (x, xh)
    assert bench._kernel_bytes(cfg, "f16", "fno_contract_mx") == (w, 2 * xh)
    assert bench._kernel_bytes(cfg, "f16", "fno_inv_plane_mx") == (x, xh)
    # half exchange: fp16 pairs, an int32 exponent per forward plane and an
    # int8 one per four contracted modes
    K = 2 * 32 * 32
    xh16 = 32 * 64 * (K * 4 + 4)
    yh16 = 32 * 64 * (K * 4 + K // 4)
    assert bench._kernel_bytes(cfg, "f16", "fno_fwd_plane_mx", True) == (x, xh16)
    assert bench._kernel_bytes(cfg, "f16", "fno_contract_mx", True) == (w, xh16 + yh16)


def test_per_launch_bytes_3d():
    # 64^3 fp32: the outer-axis passes move only slab transforms and spectra
    cfg = wl.CONFIGS["c3"]
    x = 4 * 32 * 64 ** 3 * 4
    w = 4 * 16 ** 3 * 32 * 32 * 8
    t = 4 * 32 * 64 * (2 * 16 * 16) * 8
    xh = 4 * 32 * 4 * 16 ** 3 * 8
    assert bench._kernel_bytes(cfg, "f32", "fno_fwd_plane_mx") == (x, t)
    assert bench._kernel_bytes(cfg, "f32", "fno_fwd_axis") == (0, t + xh)
    assert bench._kernel_bytes(cfg, "f32", "fno_contract") == (w, 2 * xh)
    assert bench._kernel_bytes(cfg, "f32", "fno_inv_plane_mx") == (x, t)


def test_roofline_takes_the_longest_kernel():
    cfg = wl.CONFIGS["c2"]
    ks = [{"kernel": "a", "ms": 0.05, "gbps": 5000.0, "algorithmic_bytes": 1, "exchange_bytes": 2,
           "gbps_with_exchange": 6000.0},
          {"kernel": "fno_fwd_plane_mx", "ms": 0.06, "gbps": 4000.0, "algorithmic_bytes": 3,
           "exchange_bytes": 4, "gbps_with_exchange": 4500.0}]
    r = bench._roofline(cfg, "f16", ks)
    assert r["kernel"] == "fno_fwd_plane_mx" and r["frac"] == 0.5 and r["peak"] == 8000.0
    assert set(r) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}


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


def test_measured_traffic_needs_every_source_unchanged(tmp_path, monkeypatch):
    # a counter summary counts only while every source it names still has the
    # recorded digest
    import hashlib
    (tmp_path / "profiles").mkdir()
    (tmp_path / "a.hip").write_text("kernel a\n")
    (tmp_path / "b.hpp").write_text("header b\n")
    dig = {n: hashlib.sha256((tmp_path / n).read_bytes()).hexdigest() for n in ("a.hip", "b.hpp")}
    (tmp_path / "profiles" / "k_c9_f16_traffic.md").write_text(
        "# HBM traffic\n\ntraffic_bytes_per_launch: 1234\n"
        f"source: a.hip sha256 {dig['a.hip']}\nsource: b.hpp sha256 {dig['b.hpp']}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("k", "c9", "f16") == 1234
    assert bench.measured_traffic("k", "c9", "f32") is None
    (tmp_path / "b.hpp").write_text("header b, changed\n")
    assert bench.measured_traffic("k", "c9", "f16") is None
