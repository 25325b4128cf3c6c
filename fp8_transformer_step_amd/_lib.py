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


class BlockWeightsC(ctypes.Structure):
    """Mirror of fp8s_block_weights."""
    _fields_ = [("qkv", QWeightC), ("o", QWeightC), ("gate", QWeightC), ("up", QWeightC), ("down", QWeightC),
                ("norm_attn", c_vp), ("norm_mlp", c_vp)]


class DualArModelC(ctypes.Structure):
    """Mirror of fp8s_dual_ar_model (array fields are host pointers)."""
    _fields_ = [("hidden", c_i64), ("inter", c_i64), ("codebook_size", c_i64),
                ("n_heads", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32),
                ("n_codebooks", c_i32), ("n_slow_layers", c_i32), ("n_fast_layers", c_i32),
                ("rms_eps", ctypes.c_float),
                ("slow", ctypes.POINTER(BlockWeightsC)), ("fast", ctypes.POINTER(BlockWeightsC)),
                ("slow_norm", c_vp), ("fast_norm", c_vp),
                ("embed", ctypes.POINTER(c_vp)), ("heads", ctypes.POINTER(QWeightC))]


class KvStateC(ctypes.Structure):
    """Mirror of fp8s_kv_state (cache arrays are host pointers)."""
    _fields_ = [("k_cache", ctypes.POINTER(c_vp)), ("v_cache", ctypes.POINTER(c_vp)),
                ("stride_b", c_i64), ("stride_h", c_i64), ("stride_t", c_i64), ("cap", c_i64),
                ("kv_len", c_vp), ("max_kv_len_hint", c_i64), ("live_rows", c_vp),
                ("kv_format", c_i32),
                ("k_q", ctypes.POINTER(c_vp)), ("k_e", ctypes.POINTER(c_vp)),
                ("v_q", ctypes.POINTER(c_vp)), ("v_e", ctypes.POINTER(c_vp)),
                ("sstride_b", c_i64), ("sstride_h", c_i64), ("sstride_t", c_i64)]


# name -> (restype, argtypes)
SIGNATURES = {
    "qlinear_quantize": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int, c_vp, c_i64, c_vp,
                                        c_i64, c_i64, c_vp]),
    "swiglu_mlp_fp8_workspace_size": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
    "fp8s_packed_weight_bytes": (c_sz, [c_i64, c_i64]),
    "fp8s_set_debug_tap": (ctypes.c_int, [ctypes.c_int, c_vp, c_sz]),
    "fp8s_stream_read": (ctypes.c_int, [c_vp, c_sz, c_vp, c_vp]),
    "fp8s_pack_weight": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "swiglu_mlp_fp8": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int, QWeightC, QWeightC, QWeightC,
                                      c_vp, c_vp, c_sz, c_vp, c_vp]),
    "swiglu_mlp_fp8_noalloc_max_bytes": (c_sz, []),
    "swiglu_mlp_fp8_noalloc": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int, QWeightC, QWeightC,
                                              QWeightC, c_vp, c_vp, c_vp]),
    "gqa_decode_attn_workspace_size": (c_sz, [c_i64, c_i32, c_i32, c_i64]),
    "gqa_decode_attn": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i32, c_i32, c_i32,
                                       c_i64, c_i64, ctypes.c_float, c_vp, c_vp, c_sz, c_vp, c_vp]),
    "gqa_decode_attn_mxkv": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64,
                                            c_vp, c_i64, c_i32, c_i32, c_i32, c_i64, c_i64, ctypes.c_float, c_vp,
                                            c_vp, c_sz, c_vp, c_vp]),
    "gqa_decode_attn_paged": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_i64,
                                             c_i64, c_vp, c_i64, c_i32, c_i32, c_i32, c_i64, ctypes.c_float, c_vp,
                                             c_vp, c_sz, c_vp, c_vp]),
    "gqa_decode_attn_paged_mxkv": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                                  c_i64, c_i64, c_i32, c_vp, c_i64, c_i64, c_vp, c_i64, c_i32, c_i32,
                                                  c_i32, c_i64, ctypes.c_float, c_vp, c_vp, c_sz, c_vp, c_vp]),
    "fp8_gemm_mx": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64,
                                   c_i64, c_vp, c_i64, c_vp]),
    "extend_attn": (ctypes.c_int, [c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i32, c_i32,
                                   c_i32, c_i64, c_i64, ctypes.c_float, c_vp, c_vp, c_vp]),
    "extend_attn_paged": (ctypes.c_int, [c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_vp,
                                         c_i64, c_i64, c_vp, c_i64, c_i32, c_i32, c_i32, c_i64, ctypes.c_float, c_vp,
                                         c_vp, c_vp]),
    "fp8_mx_packed_bytes": (c_sz, [c_i64, c_i64]),
    "fp8_pack_mx": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_sz, c_vp]),
    "fp8_gemm_mx_packed": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "fp8_bs_packed_bytes": (c_sz, [c_i64, c_i64]),
    "fp8_pack_bs": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i32, c_i64, c_i64, c_vp, c_sz, c_vp]),
    "fp8_gemm_bs_packed": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "swiglu_mlp_fp8_large_workspace_size": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "swiglu_mlp_fp8_large": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp,
                                            c_sz, c_vp]),
    "sample_top_k_top_p": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_float, c_i32, ctypes.c_float, c_vp,
                                          c_vp, c_i64, c_vp]),
    "prev_tokens_shift_inplace": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp]),
    "qlinear_fp8_workspace_size": (c_sz, [c_i64, c_i64, c_i64]),
    "qlinear_fp8": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_float, QWeightC, c_i64, c_vp, c_i64,
                                   ctypes.c_int, c_vp, c_i64, c_vp, c_sz, c_vp]),
    "qkv_proj_kv_append": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_float, QWeightC, c_i32, c_i32,
                                          c_i32, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_sz,
                                          c_vp, c_vp]),
    "qkv_proj_kv_append_mxkv": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_float, QWeightC, c_i32,
                                               c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                               c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_sz, c_vp, c_vp]),
    "embed_sum_bf16": (ctypes.c_int, [ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_vp,
                                      c_vp, c_vp]),
    "argmax_rows_f32": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "dual_ar_decode_step_workspace_size": (c_sz, [ctypes.POINTER(DualArModelC), c_i64, c_i64]),
    "dual_ar_decode_step": (ctypes.c_int, [ctypes.POINTER(DualArModelC), c_i64, c_vp, ctypes.POINTER(KvStateC), c_vp,
                                           c_vp, c_vp, c_vp, c_vp, c_sz, c_vp, c_vp]),
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
