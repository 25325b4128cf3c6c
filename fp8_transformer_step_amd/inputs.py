"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the storage formats
of the inputs (bf16, int32).  It holds none of the method's arithmetic (no
quantisation, GEMM, activation or attention), so the oracle and the HIP path
can both be fed from it without sharing any computation.

Recipe (seed = 1000 * workload + tensor id, NumPy default_rng, fp32 draws
rounded to bf16 with round-to-nearest-even):
  * MLP activations x ~ N(0, 1); on the MX workload 1% of entries (Bernoulli
    mask) are multiplied by 50 as outliers.
  * MLP weights ~ N(0, 0.02), bf16, later quantised by each side on its own.
  * Attention q, K, V ~ N(0, 1) bf16; kv_len ~ U{lo..hi} per sequence.  Only
    the prefix [0, kv_len) is drawn here; the cache tail is filled with
    random bytes on the device by the caller.
"""

import numpy as np

# Workload ids used in the seed formula.
W_TINY, W_BSGEMM, W_MXFP8, W_ATTN, W_STEP = 0, 1, 2, 3, 4

# Tensor ids used in the seed formula.
T_X, T_WG, T_WU, T_WD, T_Q, T_K, T_V, T_KVLEN, T_MASK = range(9)


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact fp32 value of bf16 bits."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rng(workload, tensor_id, extra=0):
    return np.random.default_rng(1000 * workload + tensor_id + 100000 * extra)


def normal_bf16(workload, tensor_id, shape, std=1.0, extra=0):
    g = rng(workload, tensor_id, extra)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return f32_to_bf16_bits(x)


def mlp_activations(workload, M, hidden, extra=0):
    """x [M, hidden] as bf16 bits (N(0,1); outliers x50 on the MX workload)."""
    x = rng(workload, T_X, extra).standard_normal(size=(M, hidden), dtype=np.float32)
    if workload == W_MXFP8:
        mask = rng(workload, T_MASK, extra).random(size=(M, hidden)) < 0.01
        x = np.where(mask, x * np.float32(50.0), x)
    return f32_to_bf16_bits(x)


def mlp_weights(workload, hidden, inter, extra=0):
    """gate [I, H], up [I, H], down [H, I] as bf16 bits, N(0, 0.02)."""
    return (normal_bf16(workload, T_WG, (inter, hidden), 0.02, extra),
            normal_bf16(workload, T_WU, (inter, hidden), 0.02, extra),
            normal_bf16(workload, T_WD, (hidden, inter), 0.02, extra))


def kv_lengths(workload, B, lo, hi, extra=0):
    """Ragged kv_len, uniform on the integers lo..hi inclusive."""
    return rng(workload, T_KVLEN, extra).integers(lo, hi + 1, size=B).astype(np.int32)


def attention_prefix(workload, B, Hq, Hkv, D, max_len, extra=0):
    """q [B, Hq, D] and the K/V prefixes [B, Hkv, max_len, D] as bf16 bits."""
    return (normal_bf16(workload, T_Q, (B, Hq, D), 1.0, extra),
            normal_bf16(workload, T_K, (B, Hkv, max_len, D), 1.0, extra),
            normal_bf16(workload, T_V, (B, Hkv, max_len, D), 1.0, extra))
