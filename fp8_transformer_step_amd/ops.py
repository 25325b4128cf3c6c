"""Thin torch-facing wrappers over the C ABI of libfp8step.so.

Each function only checks tensor placement and dtypes, allocates outputs with
torch when the caller does not pass them, and forwards raw device pointers and
sizes to the library on the current HIP stream.  All arithmetic runs in the
HIP kernels.
"""

import math
from dataclasses import dataclass

import torch

from . import _lib

# Quantisation and MLP modes (include/fp8step.h).
Q_ACT_1x128, Q_WGT_128x128, Q_MX_1x32 = 0, 1, 2
MLP_BSGEMM, MLP_MXFP8 = 0, 1
DEV_KVLEN_RANGE, DEV_WAIT_TIMEOUT = 1, 2


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fp8step operates on GPU tensors only")


def _bits(t):
    """bf16 tensor -> its storage pointer (the library reads uint16 bits)."""
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected a bfloat16 tensor, got {t.dtype}")
    return t.data_ptr()


def qlinear_quantize(x, mode, q=None, scale=None, k_major=None):
    """Quantise a 2-D bf16 tensor; returns (q uint8, scale).

    Scale tensors: mode 0 -> fp32 [rows, cols/128]; mode 1 -> fp32
    [rows/128, cols/128]; mode 2 -> uint8 [rows, cols/32].  With
    k_major=True (the MX default) the scale tensor is allocated as a K-major
    view (stride (1, rows)).
    """
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if k_major is None:
        k_major = mode == Q_MX_1x32
    if scale is None:
        if mode == Q_ACT_1x128:
            shape, dt = (rows, cols // 128), torch.float32
        elif mode == Q_WGT_128x128:
            shape, dt = (rows // 128, cols // 128), torch.float32
        else:
            shape, dt = (rows, cols // 32), torch.uint8
        if k_major:
            scale = torch.empty((shape[1], shape[0]), dtype=dt, device=x.device).t()
        else:
            scale = torch.empty(shape, dtype=dt, device=x.device)
    _lib.check(_lib.load().qlinear_quantize(
        _bits(x), rows, cols, x.stride(0), mode, q.data_ptr(), q.stride(0),
        scale.data_ptr(), scale.stride(0), scale.stride(1), _stream()))
    return q, scale


@dataclass
class QWeight:
    """An e4m3 weight [N, K] with its block scales (see fp8s_qweight)."""
    w: torch.Tensor
    scale: torch.Tensor

    def as_c(self):
        return _lib.QWeightC(self.w.data_ptr(), self.w.stride(0), self.scale.data_ptr(),
                             self.scale.stride(0), self.scale.stride(1))


def quantize_weight(w_bf16, mlp_mode):
    """Quantise a bf16 weight for the given MLP path (load-time step)."""
    if mlp_mode == MLP_BSGEMM:
        q, s = qlinear_quantize(w_bf16, Q_WGT_128x128)
    else:
        q, s = qlinear_quantize(w_bf16, Q_MX_1x32, k_major=True)
    return QWeight(q, s)


def mlp_workspace_bytes(M, hidden, inter, mode):
    return int(_lib.load().swiglu_mlp_fp8_workspace_size(M, hidden, inter, mode))


def new_mlp_workspace(M, hidden, inter, mode, device="cuda"):
    """A zero-filled workspace (the library keeps it zeroed between calls)."""
    n = mlp_workspace_bytes(M, hidden, inter, mode)
    if n == 0:
        raise ValueError("unsupported MLP shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def swiglu_mlp_fp8(x, gate, up, down, mode, y=None, workspace=None, err=None):
    """y = SwiGLU MLP of x [M, hidden] bf16 with FP8 weights; returns y bf16."""
    _require_cuda(x)
    if not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous [M, hidden] tensor")
    M, H = x.shape
    I = gate.w.shape[0]
    if y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = new_mlp_workspace(M, H, I, mode, x.device)
    _lib.check(_lib.load().swiglu_mlp_fp8(
        _bits(x), M, H, I, mode, gate.as_c(), up.as_c(), down.as_c(), _bits(y),
        workspace.data_ptr(), workspace.numel(), err.data_ptr() if err is not None else None,
        _stream()))
    return y


def attn_workspace_bytes(B, Hq, D, max_kv_len):
    return int(_lib.load().gqa_decode_attn_workspace_size(B, Hq, D, max_kv_len))


def new_attn_workspace(B, Hq, D, max_kv_len, device="cuda"):
    """A zero-filled attention workspace (its split counters stay zeroed)."""
    return torch.zeros(max(attn_workspace_bytes(B, Hq, D, max_kv_len), 16), dtype=torch.uint8, device=device)


def gqa_decode_attn(q, k_cache, v_cache, kv_len, max_kv_len_hint, softmax_scale=None,
                    out=None, workspace=None, err=None):
    """Decode attention of q [B, Hq, D] over caches [B, Hkv, cap, D] (any
    strides with unit stride along D) for positions < kv_len[b]."""
    _require_cuda(q, k_cache, v_cache, kv_len)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    B, Hq, D = q.shape
    _, Hkv, cap, _ = k_cache.shape
    if k_cache.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    hint = min(int(max_kv_len_hint), cap)
    if workspace is None:
        workspace = new_attn_workspace(B, Hq, D, hint, q.device)
    _lib.check(_lib.load().gqa_decode_attn(
        _bits(q.contiguous()), _bits(k_cache), _bits(v_cache), k_cache.stride(0), k_cache.stride(1),
        k_cache.stride(2), kv_len.data_ptr(), B, Hq, Hkv, D, cap, hint, float(softmax_scale),
        _bits(out), workspace.data_ptr(), workspace.numel(),
        err.data_ptr() if err is not None else None, _stream()))
    return out


def profile_start(max_records=200000):
    """Start recording per-kernel HIP events inside the library."""
    _lib.check(_lib.load().fp8s_profile_start(int(max_records)))


def profile_stop():
    """Stop recording; returns [(kernel name, milliseconds), ...] in launch order."""
    import ctypes
    lib = _lib.load()
    n = lib.fp8s_profile_stop()
    if n < 0:
        _lib.check(n)
    out = []
    buf = ctypes.create_string_buffer(64)
    ms = ctypes.c_float()
    for i in range(n):
        _lib.check(lib.fp8s_profile_record(i, buf, 64, ctypes.byref(ms)))
        out.append((buf.value.decode(), float(ms.value)))
    return out
