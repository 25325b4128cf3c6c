"""gqa_decode_attn_mxkv (MXFP8 KV caches) on the GPU against the oracle: the
cache quantiser's bytes, the tiny workload, the 32/8/128 workload with ragged
kv_len, long prefixes through the split path, garbage-tail invariance (random
codes and exponents, NaN patterns included), split invariance and invalid
kv_len handling.  Both sides quantise the same bf16 rows independently: the
GPU with qlinear_quantize mode 2, the oracle with its OCP MX rule."""

import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import fp8 as ofp8
from fp8_transformer_step_amd import inputs, ops
from _helpers import TOL_BF16_ATTN, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _random_tail(cache, kv, seed):
    """Overwrite rows t >= kv_len[b] of an MX cache with random bytes."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for t in (cache.q, cache.e):
        noise = torch.randint(0, 256, t.shape, dtype=torch.int32, device="cuda", generator=g).to(torch.uint8)
        for b in range(t.shape[0]):
            L = int(kv[b])
            t[b, :, L:] = noise[b, :, L:]


def _make(workload, B, Hq, Hkv, D, cap, kv, tail_seed=1, extra=0):
    Lmax = int(kv.max())
    qb, kb, vb = inputs.attention_prefix(workload, B, Hq, Hkv, D, Lmax, extra=extra)
    caches = []
    for src in (kb, vb):
        c = torch.zeros((B, Hkv, cap, D), dtype=torch.bfloat16, device="cuda")
        c[:, :, :Lmax] = to_dev_bf16(src)
        mx = ops.quantize_kv_mx(c)
        _random_tail(mx, kv, tail_seed + len(caches))
        caches.append(mx)
    torch.cuda.synchronize()
    return qb, kb, vb, caches[0], caches[1]


def _oracle_mx(src_bits):
    """The oracle's MX codes and exponents of bf16 rows [B, Hkv, T, D]."""
    x = f32(src_bits)
    D = x.shape[-1]
    q, e = ofp8.quant_mx_1x32(x.reshape(-1, D))
    return q.reshape(x.shape), e.reshape(x.shape[:-1] + (D // 32,))


def _oracle(qb, kb, vb, kv):
    kq, ke = _oracle_mx(kb)
    vq, ve = _oracle_mx(vb)
    return oattn.gqa_decode_attention_mxkv(f32(qb), kq, ke, vq, ve, kv)


def _run(qb, kc, vc, kv, hint, err=None):
    out = ops.gqa_decode_attn_mxkv(to_dev_bf16(qb), kc, vc, torch.from_numpy(kv).cuda(), hint, err=err)
    torch.cuda.synchronize()
    return out


def test_cache_quantiser_bytes_match_oracle():
    need_gpu()
    kv = np.array([300, 177], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, 2, 32, 8, 128, 512, kv, extra=60)
    kq, ke = _oracle_mx(kb)
    for b in range(2):
        L = int(kv[b])
        assert np.array_equal(kc.q[b, :, :L].cpu().numpy(), kq[b, :, :L])
        assert np.array_equal(kc.e[b, :, :L].cpu().numpy(), ke[b, :, :L])


def test_tiny_workload():
    need_gpu()
    kv = np.array([37], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_TINY, 1, 4, 1, 64, 128, kv, extra=61)
    out = _run(qb, kc, vc, kv, 128)
    assert max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


@pytest.mark.parametrize("B", [1, 16])
def test_qwen_shape_short_context(B):
    need_gpu()
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, 400, extra=70 + B)
    log(f"attn mxkv B={B} kv range {kv.min()}..{kv.max()}")
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, 4096, kv, extra=70 + B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _run(qb, kc, vc, kv, 400, err)
    e = max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv))
    log(f"  max rel err {e:.3e}")
    assert int(err.item()) == 0
    assert e <= TOL_BF16_ATTN


@pytest.mark.parametrize("B,lo,hi", [(4, 1024, 4096), (2, 8192, 8192)])
def test_long_prefixes(B, lo, hi):
    need_gpu()
    kv = inputs.kv_lengths(inputs.W_ATTN, B, lo, hi, extra=80 + B)
    log(f"attn mxkv long B={B} kv range {kv.min()}..{kv.max()}")
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, hi, kv, extra=80 + B)
    out = _run(qb, kc, vc, kv, hi)
    assert max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


def test_garbage_tail_invariance_and_split_invariance():
    need_gpu()
    B = 8
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, 400, extra=90)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, 1024, kv, tail_seed=5, extra=90)
    base = _run(qb, kc, vc, kv, 400)
    _, _, _, kc2, vc2 = _make(inputs.W_ATTN, B, 32, 8, 128, 1024, kv, tail_seed=11, extra=90)
    assert torch.equal(base, _run(qb, kc2, vc2, kv, 400))
    ref = _oracle(qb, kb, vb, kv)
    for hint in (401, 1024):
        assert max_rel_err(from_dev_bf16(_run(qb, kc, vc, kv, hint)), ref) <= TOL_BF16_ATTN


@pytest.mark.parametrize("hint", [256, 16])
def test_invalid_kv_len_sets_flag_and_zeroes(hint):
    need_gpu()
    B, cap = 3, 256
    kv = np.array([10, 10, 10], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=95)
    bad = np.array([10, 0, 257], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _run(qb, kc, vc, bad, hint, err)
    assert int(err.item()) == ops.DEV_KVLEN_RANGE
    assert not out[1].float().abs().sum().item() and not out[2].float().abs().sum().item()
    assert max_rel_err(from_dev_bf16(out[:1]), _oracle(qb[:1], kb[:1], vb[:1], kv[:1])) <= TOL_BF16_ATTN


def test_balanced_split_mixed_lengths():
    """The balanced split (16+ sequences) over MXFP8 caches, tiny and
    full-capacity prefixes mixed."""
    need_gpu()
    B, cap = 24, 1024
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 1, cap, extra=203)
    kv[:3] = [1, cap, 3]
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=203)
    out = _run(qb, kc, vc, kv, cap)
    assert max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


@pytest.mark.timeout(600)
@pytest.mark.parametrize("hi", [4096, 8192])
def test_b64_sampled_rows(hi):
    """B = 64, kv U[234, hi] over MXFP8 caches in one launch; the oracle
    checks sampled sequences (first, last, longest, shortest and a spread)."""
    need_gpu()
    B = 64
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, hi, extra=910 + hi)
    log(f"attn mxkv B=64 kv range {kv.min()}..{kv.max()}")
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, hi, kv, extra=910 + hi)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = from_dev_bf16(_run(qb, kc, vc, kv, hi, err))
    rows = sorted({0, 13, 29, 47, B - 1, int(np.argmax(kv)), int(np.argmin(kv))})
    ref = _oracle(qb[rows], kb[rows], vb[rows], kv[rows])
    e = max_rel_err(out[rows], ref)
    log(f"  rows {rows} kv {[int(kv[b]) for b in rows]}: max rel err {e:.3e}")
    assert int(err.item()) == 0
    assert e <= TOL_BF16_ATTN
