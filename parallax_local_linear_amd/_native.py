"""ctypes binding of libparallax.so: argument marshalling only.

Every step of the forward pass runs in the HIP kernels behind the C ABI
(include/parallax.h).  Torch is used for device memory and for the current
HIP stream; there is no fallback path: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PLX_LIBRARY", os.path.join(HERE, "libparallax.so"))

PLX_F32, PLX_BF16 = 0, 1
STATUS = {0: "PLX_OK", 1: "PLX_EINVAL", 2: "PLX_EUNSUPPORTED", 3: "PLX_ENOMEM", 4: "PLX_EHIP"}

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/parallax.h
SIGNATURES = {
    "parallax_abi_version": (_i, []),
    "parallax_last_error": (ctypes.c_char_p, []),
    "parallax_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "parallax_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _sz,
                              _vp]),
    "parallax_prefill_stage_v": (_i, [_vp, _vp, _i, _i, _i, _i, _vp]),
    "parallax_prefill_attend": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp]),
    "parallax_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "parallax_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i,
                             _vp, _sz, _vp]),
    "parallax_decode_partials": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i,
                                      _i, _vp]),
    "parallax_decode_combine": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "parallax_decode_default_split": (_i, [_i, _i, _i, _i]),
    "parallax_decode_noalloc_max_bytes": (_sz, []),
    "parallax_decode_noalloc": (_i, [_vp] * 7 + [_i, _i, _i, _i, _f, _i, _i, _vp]),
    "parallax_softmax_prefill": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _sz,
                                      _vp]),
    "parallax_softmax_prefill_attend": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp]),
    "parallax_softmax_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp,
                                     _sz, _vp]),
    "parallax_prefill_train": (_i, [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "parallax_prefill_backward_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "parallax_prefill_backward": (_i, [_vp] * 15 + [_i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "parallax_prefill_chunk_workspace_bytes": (_sz, [_i] * 7),
    "parallax_prefill_chunk": (_i, [_vp] * 8 + [_i] * 6 + [_f, _i, _i, _vp, _sz, _vp]),
    "parallax_prefill_chunk_default_split": (_i, [_i] * 5),
    "parallax_prefill_chunk_vt_workspace_bytes": (_sz, [_i] * 7),
    "parallax_stage_v_rows": (_i, [_vp] * 4 + [_i] * 6 + [_vp]),
    "parallax_prefill_chunk_vt": (_i, [_vp] * 8 + [_i] * 6 + [_f, _i, _i, _vp, _sz, _vp]),
}

_lib = None


class ParallaxError(RuntimeError):
    """A library call returned a status other than PLX_OK."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with {STATUS.get(status, status)}: {text}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libparallax.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m parallax_local_linear_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise ParallaxError(name, st, lib().parallax_last_error().decode())
    return st
