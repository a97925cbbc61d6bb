"""Workload registry: the five FNO configurations this library is measured and
checked on.

The 2D layer workloads are 128x128 and 256x256 flow fields and the 3D one a
64^3 field, the shapes the TurboFNO write-up ("TurboFNO: FFT-GEMM-iFFT fusion
kernels", sections 1 and 2) uses for its 2D flow-field reconstruction and 3D
flow-field prediction examples. Those datasets are not available, so Gaussian
random fields with power spectrum (|k|^2 + 49)^-2.5 stand in for them.

Modes: ``m1`` counts kx rows per corner (kx in [0, m1) and [H - m1, H)),
``m2`` counts ky columns of the half spectrum (ky in [0, m2)); in 3D the
corners are in kx and ky and the half spectrum is along kz.
"""

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    ndim: int
    batch: int
    c_in: int
    c_out: int
    grid: Tuple[int, ...]
    modes: Tuple[int, ...]
    dtypes: Tuple[str, ...]
    seed: int
    input_kind: str  # "uniform" (U[-1,1)) or "grf"
    description: str = ""

    @property
    def n_modes(self) -> int:
        """Retained complex modes per plane: 2*m1*m2 (2D), 4*m1*m2*m3 (3D)."""
        k = 1
        for m in self.modes:
            k *= m
        return k * (2 if self.ndim == 2 else 4)

    def weight_shape(self) -> Tuple[int, ...]:
        """Complex weight shape: retained-spectrum axes then (Ci, Co).

        2D: (2*m1, m2, Ci, Co); 3D: (2*m1, 2*m2, m3, Ci, Co). Along a corner
        axis the low corner comes first (k = 0..m-1), then the high corner
        (k = N-m..N-1).
        """
        if self.ndim == 2:
            m1, m2 = self.modes
            return (2 * m1, m2, self.c_in, self.c_out)
        m1, m2, m3 = self.modes
        return (2 * m1, 2 * m2, m3, self.c_in, self.c_out)

    def storage_bytes(self, dtype: str) -> int:
        return 4 if dtype == "f32" else 2

    def minimal_bytes(self, dtype: str) -> int:
        """Read x once + read the weights once + write y once."""
        s = self.storage_bytes(dtype)
        pts = 1
        for g in self.grid:
            pts *= g
        x = self.batch * self.c_in * pts * s
        y = self.batch * self.c_out * pts * s
        w = self.n_modes * self.c_in * self.c_out * 2 * s
        return x + w + y


@dataclass(frozen=True)
class ModelConfig:
    name: str
    batch: int
    grid: Tuple[int, int]
    in_channels: int
    width: int
    n_layers: int
    modes: Tuple[int, int]
    proj_hidden: int
    out_channels: int
    dtype: str
    seed: int
    description: str = ""
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "c0": LayerConfig(
        "c0", 2, 2, 4, 4, (16, 16), (4, 4), ("f32",), 0, "uniform",
        "FNO2d spectral-conv layer, fp32, B=2, Cin=Cout=4, 16x16, modes 4x4"),
    "c1": LayerConfig(
        "c1", 2, 16, 32, 32, (128, 128), (16, 16), ("f32", "f16"), 1, "grf",
        "FNO2d spectral-conv layer, B=16, Cin=Cout=32, 128x128, modes 16x16"),
    "c2": LayerConfig(
        "c2", 2, 32, 64, 64, (256, 256), (32, 32), ("f16", "bf16"), 2, "grf",
        "FNO2d spectral-conv layer, B=32, Cin=Cout=64, 256x256, modes 32x32"),
    "c3": LayerConfig(
        "c3", 3, 4, 32, 32, (64, 64, 64), (16, 16, 16), ("f32",), 3, "grf",
        "FNO3d spectral-conv layer, fp32, B=4, Cin=Cout=32, 64^3, modes 16^3"),
    "c4": ModelConfig(
        "c4", 20, (256, 256), 3, 64, 4, (24, 24), 128, 1, "f16", 4,
        "Full FNO2d forward, fp16 storage: lift 3->64, 4x(spectral conv "
        "64->64 modes 24x24 + 1x1 bypass + GELU), project 64->128->1"),
}


def get_config(name: str):
    return CONFIGS[name]
