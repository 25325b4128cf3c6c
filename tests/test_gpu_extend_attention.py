"""extend_attn (prefill / extend attention) on the GPU against the oracle:
whole prefills and extends at the 32/8/128 shape with a garbage cache tail,
one new token per sequence (the decode case), a long prefill checked on
sampled rows (each sampled row is the oracle's one-token case at its
position), group sizes 1, 2 and 8, an empty sequence between others,
tail invariance and invalid lengths."""

import numpy as np
import pytest
import torch

from oracle import attention as oattn
from fp8_transformer_step_amd import inputs, ops
from _helpers import TOL_BF16_ATTN, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _garbage(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(-32768, 32768, shape, dtype=torch.int32, device="cuda", generator=g).to(torch.int16).view(
        torch.bfloat16)


class Case:
    def __init__(self, T, L, Hq=32, Hkv=8, D=128, cap=None, extra=0, tail_seed=1):
        self.T, self.L = np.array(T, np.int32), np.array(L, np.int32)
        B = len(T)
        self.cap = cap or int(max(L)) + 40
        self.q_start = np.concatenate([[0], np.cumsum(self.T)]).astype(np.int32)
        total = max(int(self.q_start[-1]), 1)
        self.qb = inputs.normal_bf16(inputs.W_ATTN, inputs.T_Q, (total, Hq, D), 1.0, extra)
        _, self.kb, self.vb = inputs.attention_prefix(inputs.W_ATTN, B, 1, Hkv, D, int(max(L)), extra=extra)
        self.kc = _garbage((B, Hkv, self.cap, D), tail_seed)
        self.vc = _garbage((B, Hkv, self.cap, D), tail_seed + 1)
        kd, vd = to_dev_bf16(self.kb), to_dev_bf16(self.vb)
        for b in range(B):
            self.kc[b, :, :L[b]] = kd[b, :, :L[b]]
            self.vc[b, :, :L[b]] = vd[b, :, :L[b]]
        self.hint = max(int(self.T.max()), 1)
        torch.cuda.synchronize()

    def run(self, err=None, L=None):
        kv = torch.from_numpy(self.L if L is None else L).cuda()
        out = ops.extend_attn(to_dev_bf16(self.qb), torch.from_numpy(self.q_start).cuda(), self.kc, self.vc, kv,
                              self.hint, err=err)
        torch.cuda.synchronize()
        return out

    def oracle(self):
        return oattn.extend_attention(f32(self.qb), f32(self.kb), f32(self.vb), self.q_start, self.L)


@pytest.mark.parametrize("T,L", [([100, 37], [100, 37]),          # prefill
                                 ([20, 64, 1], [300, 513, 77]),    # extend
                                 ([16, 17, 33], [16, 40, 33])])    # tile edges
def test_matches_oracle(T, L):
    need_gpu()
    c = Case(T, L, extra=400 + sum(T))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = c.run(err)
    e = max_rel_err(from_dev_bf16(out), c.oracle())
    log(f"extend T={T} L={L}: max rel err {e:.2e}")
    assert int(err.item()) == 0
    assert e <= TOL_BF16_ATTN


def test_one_new_token_matches_decode_kernel():
    need_gpu()
    L = [234, 400, 1, 57]
    c = Case([1, 1, 1, 1], L, extra=410)
    out = from_dev_bf16(c.run())
    ref = oattn.gqa_decode_attention(f32(c.qb), f32(c.kb), f32(c.vb), np.array(L))
    assert max_rel_err(out, ref) <= TOL_BF16_ATTN
    dec = ops.gqa_decode_attn(to_dev_bf16(c.qb), c.kc, c.vc, torch.from_numpy(np.array(L, np.int32)).cuda(), max(L))
    torch.cuda.synchronize()
    assert max_rel_err(out, from_dev_bf16(dec)) <= TOL_BF16_ATTN


def test_long_prefill_sampled_rows():
    """A 2048-token prefill: 40 sampled rows, each the oracle's one-token
    attention over positions 0 .. p."""
    need_gpu()
    T = 2048
    c = Case([T], [T], extra=420)
    out = from_dev_bf16(c.run())
    rows = np.unique(np.concatenate([[0, 1, 15, 16, T - 1], np.random.default_rng(7).integers(0, T, 35)]))
    for t in rows:
        ref = oattn.gqa_decode_attention(f32(c.qb[t:t + 1]), f32(c.kb), f32(c.vb), np.array([t + 1]))
        assert max_rel_err(out[t:t + 1], ref) <= TOL_BF16_ATTN, t


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (64, 8), (32, 8)])
@pytest.mark.parametrize("T,L", [([40, 9], [90, 9]), ([12, 5], [70, 5])])
def test_group_sizes(Hq, Hkv, T, L):
    """Every group size, with more than 16 new tokens (several token rows per
    workgroup) and with at most 16 (one row)."""
    need_gpu()
    c = Case(T, L, Hq=Hq, Hkv=Hkv, extra=430 + Hq + T[0])
    assert max_rel_err(from_dev_bf16(c.run()), c.oracle()) <= TOL_BF16_ATTN


def test_empty_sequence_and_tail_invariance():
    need_gpu()
    c = Case([30, 0, 18], [50, 20, 18], extra=440)
    base = c.run()
    assert max_rel_err(from_dev_bf16(base), c.oracle()) <= TOL_BF16_ATTN
    c2 = Case([30, 0, 18], [50, 20, 18], extra=440, tail_seed=9)
    assert torch.equal(base.view(torch.int16), c2.run().view(torch.int16))


def test_invalid_lengths_zero_their_rows():
    need_gpu()
    c = Case([10, 12, 8], [40, 30, 20], extra=450)
    good = c.run()
    bad = np.array([40, 5, 20], np.int32)                        # T = 12 > kv_len = 5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = c.run(err, L=bad)
    assert int(err.item()) == ops.DEV_KVLEN_RANGE
    assert not out[10:22].float().abs().sum().item()
    keep = list(range(10)) + list(range(22, 30))
    assert torch.equal(out[keep].view(torch.int16), good[keep].view(torch.int16))


def _paged(c, P, seed):
    """Pools [pages, Hkv, P, D] holding c's caches on shuffled pages (garbage
    elsewhere) and the block table [B, cap / P]."""
    B, Hkv, cap, D = c.kc.shape
    mp = (cap + P - 1) // P
    n_pages = B * mp + 3
    table = inputs.page_table(inputs.W_ATTN, B, mp, n_pages, extra=seed)
    kp, vp = _garbage((n_pages, Hkv, P, D), seed + 1), _garbage((n_pages, Hkv, P, D), seed + 2)
    for b in range(B):
        n = (int(c.L[b]) + P - 1) // P
        idx = torch.from_numpy(table[b, :n].astype(np.int64)).cuda()
        kp[idx] = c.kc[b, :, :n * P].reshape(Hkv, n, P, D).transpose(0, 1)
        vp[idx] = c.vc[b, :, :n * P].reshape(Hkv, n, P, D).transpose(0, 1)
        table[b, n:] = -1                                       # never read
    torch.cuda.synchronize()
    return kp, vp, table


@pytest.mark.parametrize("T,L,P", [([100, 37], [100, 37], 16), ([20, 64, 1], [300, 513, 77], 64),
                                   ([9, 3], [40, 130], 32)])
def test_paged_equals_contiguous(T, L, P):
    need_gpu()
    c = Case(T, L, cap=(max(L) + 127) // 128 * 128, extra=460 + P)
    base = c.run()
    kp, vp, table = _paged(c, P, 470 + P)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.extend_attn_paged(to_dev_bf16(c.qb), torch.from_numpy(c.q_start).cuda(), kp, vp,
                                torch.from_numpy(table).cuda(), torch.from_numpy(c.L).cuda(), c.hint, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    assert max_rel_err(from_dev_bf16(out), c.oracle()) <= TOL_BF16_ATTN


def test_paged_bad_page_zeroes_rows():
    need_gpu()
    c = Case([20, 10], [60, 40], cap=64, extra=480)
    base = c.run()
    kp, vp, table = _paged(c, 16, 490)
    table[1, 1] = kp.shape[0]                                   # sequence 1 reads pages 0..2
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.extend_attn_paged(to_dev_bf16(c.qb), torch.from_numpy(c.q_start).cuda(), kp, vp,
                                torch.from_numpy(table).cuda(), torch.from_numpy(c.L).cuda(), c.hint, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == ops.DEV_PAGE_RANGE
    assert not out[20:30].float().abs().sum().item()
    assert torch.equal(out[:20].view(torch.int16), base[:20].view(torch.int16))
