"""ctypes loader of libfp8step.so (the C ABI declared in include/fp8step.h).

Argument marshalling only.  If the library is missing this raises; there is
no fallback implementation of any operation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8step.so")

c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t


class QWeightC(ctypes.Structure):
    """Mirror of fp8s_qweight."""
    _fields_ = [("w", c_vp), ("ld_w", c_i64), ("scale", c_vp),
                ("scale_stride_row", c_i64), ("scale_stride_colblk", c_i64)]


# name -> (restype, argtypes)
SIGNATURES = {
    "qlinear_quantize": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int, c_vp, c_i64, c_vp,
                                        c_i64, c_i64, c_vp]),
    "swiglu_mlp_fp8_workspace_size": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
    "swiglu_mlp_fp8": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int, QWeightC, QWeightC, QWeightC,
                                      c_vp, c_vp, c_sz, c_vp, c_vp]),
    "gqa_decode_attn_workspace_size": (c_sz, [c_i64, c_i32, c_i32, c_i64]),
    "gqa_decode_attn": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i32, c_i32, c_i32,
                                       c_i64, c_i64, ctypes.c_float, c_vp, c_vp, c_sz, c_vp, c_vp]),
    "fp8s_profile_start": (ctypes.c_int, [ctypes.c_int]),
    "fp8s_profile_stop": (ctypes.c_int, []),
    "fp8s_profile_record": (ctypes.c_int, [ctypes.c_int, ctypes.c_char_p, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_float)]),
    "fp8s_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_transformer_step_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class Fp8sError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"fp8step error {code}: {msg}")
        self.code = code


def check(rc):
    if rc != 0:
        raise Fp8sError(rc, load().fp8s_last_error().decode())
    return rc
