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
T_WQKV, T_WO, T_NORM, T_EMB, T_HEAD, T_CODES, T_POOL_W, T_POOL_KV, T_PAGES = range(9, 18)


def f32_to_bf16_bits(x):
    """Round finite fp32 to bf16 (nearest, ties to even); the uint16 bits.

    uint32 arithmetic cannot overflow for finite inputs (bit patterns up to
    0xFF7FFFFF plus at most 0x8000)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
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


def page_table(workload, B, max_pages, n_pages, extra=0):
    """A block table int32 [B, max_pages] of distinct page ids: the first
    B * max_pages entries of a seeded permutation of range(n_pages)."""
    if n_pages < B * max_pages:
        raise ValueError("pool smaller than the table")
    perm = rng(workload, T_PAGES, extra).permutation(n_pages)
    return perm[:B * max_pages].reshape(B, max_pages).astype(np.int32)


# ---- the full Dual-AR decode step ---------------------------------------------
# Thirty-six slow layers and four fast layers hold 4 GB of weights; drawing
# every value from the generator would take minutes.  Instead each weight
# matrix is a window, at a seeded offset, into one seeded pool of N(0, 0.02)
# bf16 values (and each K/V prefix row block a window into an N(0, 1) pool).
# Windows are views: nothing is copied until the caller uploads them.

FAST_LAYER_ID = 1000          # layer ids of the fast AR start here


def normal_pool(workload, tensor_id, n, std):
    """n seeded N(0, std) values as bf16 bits."""
    return normal_bf16(workload, tensor_id, (n,), std)


def pool_window(pool, workload, tensor_id, extra, shape):
    """A [shape] view of `pool` at an offset drawn from the seed."""
    n = int(np.prod(shape))
    if n > pool.size:
        raise ValueError(f"pool of {pool.size} values is smaller than the window {shape}")
    off = int(rng(workload, tensor_id, extra).integers(0, pool.size - n + 1))
    return pool[off:off + n].reshape(shape)


def norm_weight(workload, extra, H):
    """RMSNorm weight [H] ~ 1 + N(0, 0.1), as bf16 bits."""
    w = np.float32(1.0) + np.float32(0.1) * rng(workload, T_NORM, extra).standard_normal(H, dtype=np.float32)
    return f32_to_bf16_bits(w)


def layer_weights(pool, workload, layer_id, H, I, Hq, Hkv, D):
    """bf16 bits of one block: qkv [(Hq+2Hkv)D, H], o [H, Hq D], gate/up [I, H],
    down [H, I], and the two RMSNorm weights [H]."""
    e = 10 * layer_id
    return {
        "qkv": pool_window(pool, workload, T_WQKV, e, ((Hq + 2 * Hkv) * D, H)),
        "o": pool_window(pool, workload, T_WO, e, (H, Hq * D)),
        "gate": pool_window(pool, workload, T_WG, e, (I, H)),
        "up": pool_window(pool, workload, T_WU, e, (I, H)),
        "down": pool_window(pool, workload, T_WD, e, (H, I)),
        "norm_attn": norm_weight(workload, e, H),
        "norm_mlp": norm_weight(workload, e + 1, H),
    }


def codebook_tables(pool, workload, C, V, H):
    """Embedding tables and heads, C of each, [V, H] bf16 bits."""
    emb = [pool_window(pool, workload, T_EMB, c, (V, H)) for c in range(C)]
    heads = [pool_window(pool, workload, T_HEAD, c, (V, H)) for c in range(C)]
    return emb, heads


def prev_codes(workload, B, C, V):
    """The previous frame's codes, uniform on 0..V-1, int32 [B, C]."""
    return rng(workload, T_CODES).integers(0, V, size=(B, C)).astype(np.int32)


def kv_prefix(kv_pool, workload, set_id, b, L, Hkv, D):
    """K and V prefix rows [Hkv, L, D] of sequence b in physical cache set
    `set_id` (bf16 bits)."""
    e = 1000 * set_id + b
    return (pool_window(kv_pool, workload, T_K, e, (Hkv, L, D)),
            pool_window(kv_pool, workload, T_V, e, (Hkv, L, D)))
