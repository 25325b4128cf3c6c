"""qkv_proj_kv_append_mxkv on the GPU.  The MXFP8 rows it appends must equal,
bit for bit, the library's 1x32 quantisation (qlinear_quantize mode 2, which
other tests pin bit-exactly to the oracle's OCP MX rule) of the bf16 rows
that qkv_proj_kv_append appends for the same inputs; q must be the same;
nothing else in the caches may change; an out-of-range kv_len sets the flag
and writes nothing.  The shapes take the epilogue from registers (one K
split) and the last-arriver epilogue of a split K, at head dims 64 and 128."""

import numpy as np
import pytest
import torch

from fp8_transformer_step_amd import inputs, ops
from _helpers import log, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu
W = inputs.W_STEP


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _run(B, H, Hq, Hkv, D, cap, kv_len, seed):
    xb = inputs.normal_bf16(W, inputs.T_X, (B, H), 1.0, extra=700 + seed)
    wb = inputs.normal_bf16(W, inputs.T_WQKV, ((Hq + 2 * Hkv) * D, H), 0.02, extra=700 + seed)
    nw = inputs.norm_weight(W, 700 + seed, H)
    qw = ops.quantize_weight(to_dev_bf16(wb), ops.MLP_BSGEMM)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    rnd = lambda shape: torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)
    kc = rnd((B, Hkv, cap, 2 * D)).view(torch.bfloat16)
    vc = rnd((B, Hkv, cap, 2 * D)).view(torch.bfloat16)
    kx = ops.MxKvCache(rnd((B, Hkv, cap, D)), rnd((B, Hkv, cap, D // 32)))
    vx = ops.MxKvCache(rnd((B, Hkv, cap, D)), rnd((B, Hkv, cap, D // 32)))
    k0 = ops.MxKvCache(kx.q.clone(), kx.e.clone())
    v0 = ops.MxKvCache(vx.q.clone(), vx.e.clone())
    kvl = torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    err_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    err_m = torch.zeros(1, dtype=torch.int32, device="cuda")
    x, n = to_dev_bf16(xb), to_dev_bf16(nw)
    qb = ops.qkv_proj_kv_append(x, qw, Hq, Hkv, D, kc, vc, kvl, norm_w=n, err=err_b)
    qm = ops.qkv_proj_kv_append_mxkv(x, qw, Hq, Hkv, D, kx, vx, kvl, norm_w=n, err=err_m)
    torch.cuda.synchronize()
    return qb, qm, kc, vc, kx, vx, k0, v0, int(err_b.item()), int(err_m.item())


@pytest.mark.parametrize("B,H,Hq,Hkv,D,cap", [
    (5, 256, 4, 2, 64, 64),          # two K splits: the last-arriver epilogue
    (64, 2560, 32, 8, 128, 512),     # the step's shape: one split, epilogue from registers
    (24, 5120, 8, 2, 128, 64),       # two K splits at head dim 128
])
def test_mx_append_equals_quantised_bf16_append(B, H, Hq, Hkv, D, cap):
    need_gpu()
    rng = np.random.default_rng(B + H)
    kv_len = [int(x) for x in rng.integers(1, cap + 1, size=B)]
    log(f"mx kv append B={B} H={H} Hq={Hq} Hkv={Hkv} D={D}")
    qb, qm, kc, vc, kx, vx, k0, v0, eb, em = _run(B, H, Hq, Hkv, D, cap, kv_len, seed=B)
    assert eb == 0 and em == 0
    assert torch.equal(qb.view(torch.int16), qm.view(torch.int16))
    for src, got, before in ((kc, kx, k0), (vc, vx, v0)):
        gq, ge, bq, be = _bytes(got.q), _bytes(got.e), _bytes(before.q), _bytes(before.e)
        for b, L in enumerate(kv_len):
            t = L - 1
            want = ops.quantize_kv_mx(src[b, :, t:t + 1].contiguous().unsqueeze(0))
            assert np.array_equal(gq[b, :, t], _bytes(want.q)[0, :, 0])
            assert np.array_equal(ge[b, :, t], _bytes(want.e)[0, :, 0])
            keep = np.arange(cap) != t
            assert np.array_equal(gq[b][:, keep], bq[b][:, keep])
            assert np.array_equal(ge[b][:, keep], be[b][:, keep])


def test_mx_append_out_of_range_sets_the_flag_and_writes_nothing():
    need_gpu()
    B, H, Hq, Hkv, D, cap = 3, 256, 4, 2, 64, 64
    qb, qm, kc, vc, kx, vx, k0, v0, eb, em = _run(B, H, Hq, Hkv, D, cap, [0, 65, 3], seed=9)
    assert eb == ops.DEV_KVLEN_RANGE and em == ops.DEV_KVLEN_RANGE
    for got, before in ((kx, k0), (vx, v0)):
        gq, ge, bq, be = _bytes(got.q), _bytes(got.e), _bytes(before.q), _bytes(before.e)
        assert np.array_equal(gq[:2], bq[:2]) and np.array_equal(ge[:2], be[:2])
        keep = np.arange(cap) != 2
        assert np.array_equal(gq[2][:, keep], bq[2][:, keep])
