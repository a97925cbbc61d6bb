"""Seeded synthetic workloads for the FNO spectral-convolution layer.

This package is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It holds the workload registry (shapes, modes, storage dtypes, seeds)
and the input generators, and nothing of the layer's own arithmetic: no DFT,
no contraction, no inverse transform. (The Gaussian-random-field generator
shapes white noise with numpy.fft; that is input synthesis, not the layer.)
"""

from .configs import CONFIGS, LayerConfig, ModelConfig, get_config  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_to_float64,
    complex_to_interleaved,
    gaussian_random_field,
    layer_grad_output,
    layer_inputs,
    model_inputs,
    round_to_storage,
    spectral_weights,
    storage_to_float64,
)
