"""Synthetic Dual-AR models and KV state on the device, for the decode step.

Weights come from the seeded generators of `inputs` (bf16), are uploaded and
quantised by the library's own quantiser (128x128 fp32 block scales), exactly
as a loader would do once at start-up.  Nothing here computes any part of the
step itself.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch

from . import inputs, ops


@dataclass(frozen=True)
class DualArConfig:
    hidden: int
    inter: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    codebook_size: int
    n_codebooks: int
    n_slow_layers: int
    n_fast_layers: int
    batch: int
    cap: int          # cache slots per sequence
    kv_lo: int        # kv_len ~ U{kv_lo .. kv_hi}, counting this step's token
    kv_hi: int
    kv_sets: int      # physical K/V cache sets; slow layer l uses set l % kv_sets
    rms_eps: float = 1e-6
    pool: int = 1 << 26       # values in the weight pool
    kv_pool: int = 1 << 24    # values in the K/V pool


# The full step: Qwen3-4B-sized slow AR (36 layers), a 4-layer fast AR of the
# same width, 10 codebooks of 4096 entries, batch 64, caches of 32768 slots.
# 36 layers x 64 sequences x 32768 slots of K and V would need 309 GB, more
# than one GPU holds, so the 36 logical layers share 4 physical cache sets.
FULL = DualArConfig(hidden=2560, inter=9728, n_heads=32, n_kv_heads=8, head_dim=128, codebook_size=4096,
                    n_codebooks=10, n_slow_layers=36, n_fast_layers=4, batch=64, cap=32768, kv_lo=234,
                    kv_hi=4096, kv_sets=4)

# A small model with the same structure, for parity runs of every layer.
TINY = DualArConfig(hidden=256, inter=384, n_heads=4, n_kv_heads=2, head_dim=64, codebook_size=256,
                    n_codebooks=10, n_slow_layers=3, n_fast_layers=2, batch=5, cap=64, kv_lo=1, kv_hi=64,
                    kv_sets=3, pool=1 << 20, kv_pool=1 << 18)


def scaled(cfg, **kw):
    return replace(cfg, **kw)


class HostModel:
    """The bf16 bits of every weight of a config (views into the seeded pools)."""

    def __init__(self, cfg, workload=inputs.W_STEP):
        self.cfg, self.workload = cfg, workload
        c = cfg
        pool = inputs.normal_pool(workload, inputs.T_POOL_W, c.pool, 0.02)
        self.slow = [inputs.layer_weights(pool, workload, l, c.hidden, c.inter, c.n_heads, c.n_kv_heads,
                                          c.head_dim) for l in range(c.n_slow_layers)]
        self.fast = [inputs.layer_weights(pool, workload, inputs.FAST_LAYER_ID + f, c.hidden, c.inter, c.n_heads,
                                          c.n_kv_heads, c.head_dim) for f in range(c.n_fast_layers)]
        self.slow_norm = inputs.norm_weight(workload, 90000, c.hidden)
        self.fast_norm = inputs.norm_weight(workload, 90001, c.hidden)
        self.embed, self.heads = inputs.codebook_tables(pool, workload, c.n_codebooks, c.codebook_size, c.hidden)
        self.prev_codes = inputs.prev_codes(workload, c.batch, c.n_codebooks, c.codebook_size)
        self.kv_len = inputs.kv_lengths(workload, c.batch, c.kv_lo, c.kv_hi)
        self.kv_pool = inputs.normal_pool(workload, inputs.T_POOL_KV, c.kv_pool, 1.0)

    def kv_prefix(self, s, b):
        """K, V prefix rows [Hkv, kv_len[b], D] of set s, sequence b (bf16 bits)."""
        c = self.cfg
        return inputs.kv_prefix(self.kv_pool, self.workload, s, b, int(self.kv_len[b]), c.n_kv_heads, c.head_dim)


def _bf16(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def _qweight(bits, device, packed):
    qw = ops.quantize_weight(_bf16(bits, device), ops.MLP_BSGEMM)
    return ops.pack_weight(qw) if packed else qw


def device_model(host, device="cuda", packed=True):
    """Upload and quantise every weight; returns an ops.DualArModel.
    packed: store the e4m3 matrices fragment-packed (fp8s_pack_weight), the
    layout the decode GEMMs stream fastest; results are identical."""
    c = host.cfg

    def block(d):
        return {k: _qweight(d[k], device, packed) for k in ("qkv", "o", "gate", "up", "down")} | \
               {"norm_attn": _bf16(d["norm_attn"], device), "norm_mlp": _bf16(d["norm_mlp"], device)}
    slow = [block(d) for d in host.slow]
    fast = [block(d) for d in host.fast]
    embed = [_bf16(t, device) for t in host.embed]
    heads = [_qweight(t, device, packed) for t in host.heads]
    return ops.DualArModel(slow, fast, _bf16(host.slow_norm, device), _bf16(host.fast_norm, device), embed, heads,
                           c.n_heads, c.n_kv_heads, c.head_dim, c.inter, c.rms_eps)


def device_kv(host, device="cuda", garbage_seed=1234, mx=False):
    """Physical K/V sets [B, Hkv, cap, D] with the seeded prefixes and random
    bytes (NaN and Inf patterns included) in every unfilled slot.
    mx: MXFP8 caches (ops.MxKvCache) instead, each set the library's 1x32
    quantisation of the bf16 set, garbage slots included (they stay garbage:
    NaN codes and arbitrary exponents)."""
    c = host.cfg
    g = torch.Generator(device=device)
    g.manual_seed(garbage_seed)
    ks, vs = [], []
    for s in range(c.kv_sets):
        kc = torch.randint(-32768, 32768, (c.batch, c.n_kv_heads, c.cap, c.head_dim), dtype=torch.int16,
                           device=device, generator=g)
        vc = torch.randint(-32768, 32768, kc.shape, dtype=torch.int16, device=device, generator=g)
        for b in range(c.batch):
            kp, vp = host.kv_prefix(s, b)
            L = kp.shape[1]
            kc[b, :, :L].copy_(torch.from_numpy(kp.view(np.int16)))
            vc[b, :, :L].copy_(torch.from_numpy(vp.view(np.int16)))
        ks.append(kc.view(torch.bfloat16))
        vs.append(vc.view(torch.bfloat16))
    kv_len = torch.from_numpy(host.kv_len).to(device)
    if mx:
        ks = [ops.quantize_kv_mx(k) for k in ks]
        vs = [ops.quantize_kv_mx(v) for v in vs]
        torch.cuda.synchronize()
    layers_k = [ks[l % c.kv_sets] for l in range(c.n_slow_layers)]
    layers_v = [vs[l % c.kv_sets] for l in range(c.n_slow_layers)]
    return ops.KvState(layers_k, layers_v, kv_len, int(host.kv_len.max())), ks, vs
