"""CPU float64 oracle of the FNO spectral-convolution layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library never calls it and has
no fallback to it. It shares no code, tables or constants with the HIP path.

What it computes follows the TurboFNO write-up ("TurboFNO: FFT-GEMM-iFFT
fusion kernels"): section 1 and section 2.1-2.3 name the pipeline as a real
2D FFT, a per-mode weight contraction ``einsum("xyij,xyik->xyjk")`` over the
input channel with a learnable complex weight of shape
(modes_x, modes_y, in_ch, out_ch), and an inverse real FFT; section 4.3 gives
the layer's call shape (input [B, C, H, W], weight split into real and
imaginary parts). The DFTs here are the plain definitions written as dense
matrices (no FFT); the inverse is the closed-form c2r sum. Readings of what
the pages leave open (normalisation, sign, corner indices, c2r convention)
are listed in the module docstrings.

Functions:
  spectral.forward2d / forward3d      truncated forward DFT (spectra)
  spectral.contract                   per-mode complex contraction
  spectral.inverse2d / inverse3d      closed-form inverse on retained modes
  spectral.spectral_conv2d / 3d       the whole layer
  fno2d.fno_block2d                   one block: act(spectral conv + 1x1 + bias)
  fno2d.fno2d_forward                 the full FNO2d network (composition)
  backward.spectral_conv2d_backward   gradients of the layer (dx, dw): the
  backward.spectral_conv3d_backward   adjoints of its linear steps in reverse
"""

from .spectral import (  # noqa: F401
    contract,
    corner_indices,
    forward2d,
    forward3d,
    inverse2d,
    inverse3d,
    spectral_conv2d,
    spectral_conv3d,
)
from .fno2d import fno2d_forward, fno_block2d, gelu  # noqa: F401
from .backward import spectral_conv2d_backward, spectral_conv3d_backward  # noqa: F401
