"""ctypes loader for libfno.so (the HIP library). Fails loudly when missing."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfno.so")

FNO_OK = 0
STATUS_NAMES = {0: "FNO_OK", 1: "FNO_ERR_INVALID_ARG", 2: "FNO_ERR_UNSUPPORTED",
                3: "FNO_ERR_OUT_OF_MEMORY", 4: "FNO_ERR_DEVICE"}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # FNO_NOALLOC_SCRATCH_BYTES

# every symbol include/fno.h declares, with its ctypes signature
_c_int, _c_void_p, _c_size_t = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_IntP = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "fno_plan_create": (_c_int, [ctypes.POINTER(_c_void_p), _c_int, _c_int, _c_int, _c_int,
                                 _IntP, _IntP, _c_int, _c_int]),
    "fno_spectral_conv2d": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fno_spectral_conv3d": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fno_spectral_conv_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fno_block2d": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p,
                             _c_void_p]),
    "fno_block2d_prepare": (_c_int, [_c_void_p]),
    "fno_spectral_conv2d_backward": (_c_int, [_c_void_p] * 7),
    "fno_spectral_conv3d_backward": (_c_int, [_c_void_p] * 7),
    "fno_plan_saved_bytes": (_c_int, [_c_void_p, ctypes.POINTER(_c_size_t)]),
    "fno_spectral_conv_forward_save": (_c_int, [_c_void_p] * 6),
    "fno_spectral_conv_backward_saved": (_c_int, [_c_void_p] * 7),
    "fno_weights_pack": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fno_weights_unpack": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fno_plan_destroy": (_c_int, [_c_void_p]),
    "fno_status_string": (ctypes.c_char_p, [_c_int]),
    "fno_plan_workspace_bytes": (_c_int, [_c_void_p, ctypes.POINTER(_c_size_t)]),
    "fno_plan_num_launches": (_c_int, [_c_void_p, _IntP]),
    "fno_plan_launch_name": (_c_int, [_c_void_p, _c_int, ctypes.POINTER(ctypes.c_char_p)]),
    "fno_plan_run_launch": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fno_plan_spectra": (_c_int, [_c_void_p, _c_int, ctypes.POINTER(_c_void_p)]),
    "fno_plan_spectra_format": (_c_int, [_c_void_p, _IntP]),
    "fno_plan_set_launch_shape": (_c_int, [_c_void_p, _c_int]),
    "fno_plan_get_launch_shape": (_c_int, [_c_void_p, _IntP]),
    "fno_plan_check": (_c_int, [_c_void_p]),
    "fno_channel_mix": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                 _c_int, ctypes.c_long, _c_int, _c_int, _c_void_p]),
    "fno_projection": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                _c_int, _c_int, _c_int, ctypes.c_long, _c_int, _c_void_p]),
    "fno_model2d_create": (_c_int, [ctypes.POINTER(_c_void_p), _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "fno_model2d_forward": (_c_int, [_c_void_p, _c_void_p, ctypes.POINTER(_c_void_p), _c_void_p,
                                     _c_void_p]),
    "fno_model2d_set_graph": (_c_int, [_c_void_p, _c_int]),
    "fno_model2d_destroy": (_c_int, [_c_void_p]),
}

_lib = None


class FnoError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


def lib():
    """The loaded library; raises if libfno.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m spectral_convolution_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status, where):
    if status != FNO_OK:
        raise FnoError(status, where)
