"""Guard bands around the decode outputs.

Every output (and every workspace) of the calls below lies inside a larger
buffer whose bytes before and after it hold a canary pattern.  After the
call the canaries must be intact, so nothing was written outside the output
or past the workspace size the library asked for, and the output must equal
the same call's output in an unguarded buffer bit for bit.  The shapes take
each kernel path: the two-launch MLP (M <= 4) and the four-launch one, the
balanced, chunked and single-chunk attention, the projections with bf16 and
fp32 outputs, and the full decode step."""

import numpy as np
import pytest
import torch

from fp8_transformer_step_amd import inputs, model, ops
from _helpers import log, need_gpu

pytestmark = pytest.mark.gpu

GUARD = 4096            # bytes of canary on each side (a multiple of 256: outputs stay aligned)
CANARY = 0xA5


def _guarded(shape, dtype, fill=None):
    """(buffer, view): the view of `shape` sits between two canary bands; its
    own bytes hold `fill` (a byte) or the canary."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((2 * GUARD + n,), CANARY, dtype=torch.uint8, device="cuda")
    if fill is not None:
        buf[GUARD:GUARD + n] = fill
    return buf, buf[GUARD:GUARD + n].view(dtype).view(shape)


def _intact(buf):
    n = buf.numel() - 2 * GUARD
    return bool((buf[:GUARD] == CANARY).all().item() and (buf[GUARD + n:] == CANARY).all().item())


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _weights(I, H, mode, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for shape in ((I, H), (I, H), (H, I)):
        wb = (torch.randn(shape, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        out.append(ops.pack_weight(ops.quantize_weight(wb, mode)))
    return out


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M", [1, 5, 64])
def test_mlp_output_and_workspace(mode, M):
    need_gpu()
    H, I = 2560, 9728
    w = _weights(I, H, mode, 70 + M)
    x = (torch.randn((M, H), device="cuda") * 0.5).to(torch.bfloat16)
    ref = ops.swiglu_mlp_fp8(x, *w, mode)
    ybuf, y = _guarded((M, H), torch.bfloat16)
    wbuf, ws = _guarded((ops.mlp_workspace_bytes(M, H, I, mode),), torch.uint8, fill=0)
    for _ in range(2):                         # also reusing the workspace
        ops.swiglu_mlp_fp8(x, *w, mode, y=y, workspace=ws)
        torch.cuda.synchronize()
        assert _intact(ybuf) and _intact(wbuf)
        assert _bits_equal(y, ref)


@pytest.mark.parametrize("B,lo,hi", [(64, 234, 4096), (3, 100, 1024), (64, 1, 9)])
@pytest.mark.parametrize("mx", [False, True])
def test_attention_output_and_workspace(B, lo, hi, mx):
    need_gpu()
    Hq, Hkv, D = 32, 8, 128
    cap = max(hi, 16)
    kv = inputs.kv_lengths(inputs.W_ATTN, B, lo, hi, extra=B + hi)
    g = torch.Generator(device="cuda")
    g.manual_seed(B * 7 + hi)
    kc = torch.randn((B, Hkv, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((B, Hkv, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    kvd = torch.from_numpy(kv).cuda()
    log(f"attention B={B} kv {lo}..{hi} {'MXFP8' if mx else 'bf16'}")
    fn = ops.gqa_decode_attn_mxkv if mx else ops.gqa_decode_attn
    if mx:
        kc, vc = ops.quantize_kv_mx(kc), ops.quantize_kv_mx(vc)
    ref = fn(q, kc, vc, kvd, hi)
    obuf, out = _guarded((B, Hq, D), torch.bfloat16)
    wbuf, ws = _guarded((ops.attn_workspace_bytes(B, Hq, D, hi),), torch.uint8, fill=0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        fn(q, kc, vc, kvd, hi, out=out, workspace=ws, err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert _intact(obuf) and _intact(wbuf)
        assert _bits_equal(out, ref)


@pytest.mark.parametrize("out_dtype", [ops.OUT_BF16, ops.OUT_F32])
@pytest.mark.parametrize("M,N,K", [(64, 6144, 2560), (5, 2560, 4096), (64, 4096, 2560)])
def test_projection_output_and_workspace(out_dtype, M, N, K):
    need_gpu()
    g = torch.Generator(device="cuda")
    g.manual_seed(M + N + K)
    w = ops.pack_weight(ops.quantize_weight((torch.randn((N, K), generator=g, device="cuda") * 0.02)
                                            .to(torch.bfloat16), ops.MLP_BSGEMM))
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    ref = ops.qlinear_fp8(x, w, out_dtype=out_dtype)
    dt = torch.bfloat16 if out_dtype == ops.OUT_BF16 else torch.float32
    ybuf, y = _guarded((M, N), dt)
    wbuf, ws = _guarded((ops.qlinear_workspace_bytes(M, N, K),), torch.uint8, fill=0)
    for _ in range(2):
        ops.qlinear_fp8(x, w, out_dtype=out_dtype, y=y, workspace=ws)
        torch.cuda.synchronize()
        assert _intact(ybuf) and _intact(wbuf)
        assert _bits_equal(y, ref)


@pytest.mark.parametrize("mx", [False, True], ids=["bf16_kv", "mxfp8_kv"])
def test_decode_step_outputs_and_workspace(mx):
    """The step's codes, its taps and its workspace, on the small model at
    batch 24 (two 16-row tiles), with bf16 and MXFP8 slow-layer caches."""
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=24, n_heads=8))
    c = host.cfg
    B, H, C, V = c.batch, c.hidden, c.n_codebooks, c.codebook_size
    dm = model.device_model(host)
    prev = torch.from_numpy(host.prev_codes).cuda()
    kv, _, _ = model.device_kv(host, mx=mx)
    ref = ops.dual_ar_decode_step(dm, kv, prev)
    kv, _, _ = model.device_kv(host, mx=mx)    # fresh caches: the step appends K/V
    cbuf, codes = _guarded((B, C), torch.int32)
    sbuf, slow = _guarded((2 * c.n_slow_layers + 1, B, H), torch.bfloat16)
    fbuf, fast = _guarded((C - 1, 2 * c.n_fast_layers + 1, B, H), torch.bfloat16)
    lbuf, logits = _guarded((C, B, V), torch.float32)
    wbuf, ws = _guarded((dm.workspace_bytes(B, kv.c.max_kv_len_hint),), torch.uint8, fill=0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.dual_ar_decode_step(dm, kv, prev, codes=codes, slow_taps=slow, fast_taps=fast, logits_tap=logits,
                            workspace=ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for buf in (cbuf, sbuf, fbuf, lbuf, wbuf):
        assert _intact(buf)
    assert torch.equal(codes, ref)
