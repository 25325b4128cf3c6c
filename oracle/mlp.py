"""Dequantised FP8 GEMM and the SwiGLU MLP, in float64 NumPy.

Test infrastructure only (see the package header).

Follows the page "How We Made Our Text-to-Speech API Free":
  * "Why cuBLAS Wasn't Enough" -- a SwiGLU MLP forward is a gate/up projection,
    the gated activation, and a down projection, at decode shapes M <= 128.
  * "Kernel Benchmark Results" -- the activation of each FP8 GEMM is quantised
    (1x128 groups with fp32 scales on the bsgemm path, 1x32 groups with UE8M0
    exponents on the MXFP8 path), and the SwiGLU output is quantised the same
    way as the input of the down projection.

Reading of the steps the page leaves open (also listed with the others in the
design notes):
  * SwiGLU is h = silu(g) * u with silu(g) = g * sigmoid(g), g the gate and u
    the up projection (the usual Qwen3 MLP that the page names).
  * The GEMMs accumulate exactly here (float64 over exactly-dequantised
    operands).  h is rounded to fp32 before it is re-quantised, because the
    GPU holds it in fp32 registers at that point; the final y stays float64.

Parity: pinned by tests/test_oracle_mlp.py -- an exact-integer GEMM with a
distinct power-of-two scale per block (a transposed or mis-strided scale
changes the result), an exact rational brute force at M = 1, and SwiGLU against
torch's silu in float64.  The re-quantised h bytes themselves are "parity
unpinned" against the GPU: they depend on the fp32 accumulation order there,
so a byte may differ by one e4m3 step; only the MLP output is compared.
"""

import numpy as np

from .fp8 import (
    dequant_block_fp32,
    dequant_mx_1x32,
    quant_act_1x128,
    quant_mx_1x32,
)

MODE_BSGEMM = 0
MODE_MXFP8 = 1


def linear_dequant(x_deq, w_deq):
    """y[m, n] = sum_k x[m, k] * w[n, k] over exactly dequantised operands."""
    return np.asarray(x_deq, np.float64) @ np.asarray(w_deq, np.float64).T


def quant_act(x, mode):
    """Quantise an activation [M, K] the way its GEMM consumes it.

    Returns (q, scale, dequantised float64 value).
    """
    if mode == MODE_BSGEMM:
        q, s = quant_act_1x128(x)
        return q, s, dequant_block_fp32(q, s, 1, 128)
    if mode == MODE_MXFP8:
        q, e = quant_mx_1x32(x)
        return q, e, dequant_mx_1x32(q, e)
    raise ValueError(f"unknown mode {mode}")


def swiglu(g, u):
    """h = silu(g) * u = g * sigmoid(g) * u, float64."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return g * sig * np.asarray(u, np.float64)


def swiglu_mlp(x, wg_deq, wu_deq, wd_deq, mode):
    """One SwiGLU MLP forward at decode shape.

    x       : [M, H] activations (fp32 values, normally exact bf16)
    w*_deq  : exactly dequantised FP8 weights, gate/up [I, H], down [H, I]
    mode    : MODE_BSGEMM or MODE_MXFP8 (how activations are quantised)
    Returns a dict with y (float64 [M, H]) and the intermediates.
    """
    qx, sx, xd = quant_act(x, mode)
    g = linear_dequant(xd, wg_deq)
    u = linear_dequant(xd, wu_deq)
    h = swiglu(g, u).astype(np.float32)
    qh, sh, hd = quant_act(h, mode)
    y = linear_dequant(hd, wd_deq)
    return {"y": y, "qx": qx, "sx": sx, "g": g, "u": u, "h": h, "qh": qh, "sh": sh}
