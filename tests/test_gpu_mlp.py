"""swiglu_mlp_fp8 on the GPU against the oracle: the tiny workload, the
Qwen3-4B-shaped bsgemm and MXFP8 workloads at every listed M (full sizes), a
ragged M, determinism, workspace reuse and the scale-stride contract."""

import numpy as np
import pytest
import torch

from oracle import fp8, mlp as omlp
from fp8_transformer_step_amd import inputs, ops
from _helpers import TOL_FP8_PATH, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

_CACHE = {}


def _setup(workload, H, I):
    """GPU-quantised weights and the oracle's own quantisation of the same
    bf16 weights (checked bit-exact here, so both sides use equal weights)."""
    key = (workload, H, I)
    if key in _CACHE:
        return _CACHE[key]
    mode = ops.MLP_MXFP8 if workload == inputs.W_MXFP8 else ops.MLP_BSGEMM
    wbits = inputs.mlp_weights(workload, H, I)
    gpu_w, deq = [], []
    for wb in wbits:
        qw = ops.quantize_weight(to_dev_bf16(wb), mode)
        w32 = f32(wb)
        if mode == ops.MLP_BSGEMM:
            q, s = fp8.quant_weight_128x128(w32)
            d = fp8.dequant_block_fp32(q, s, 128, 128)
        else:
            q, s = fp8.quant_mx_1x32(w32)
            d = fp8.dequant_mx_1x32(q, s)
        torch.cuda.synchronize()
        assert np.array_equal(qw.w.cpu().numpy(), q), "weight bytes differ from the oracle"
        assert np.array_equal(qw.scale.cpu().numpy(), s), "weight scales differ from the oracle"
        gpu_w.append(qw)
        deq.append(d)
    _CACHE[key] = (mode, gpu_w, deq)
    return _CACHE[key]


def _check(workload, M, H, I, extra=0):
    mode, w, deq = _setup(workload, H, I)
    log(f"mlp workload={workload} mode={mode} M={M} H={H} I={I}")
    xb = inputs.mlp_activations(workload, M, H, extra=extra)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = ops.swiglu_mlp_fp8(to_dev_bf16(xb), *w, mode, err=err)
    torch.cuda.synchronize()
    ref = omlp.swiglu_mlp(f32(xb), *deq, mode)["y"]
    e = max_rel_err(from_dev_bf16(y), ref)
    log(f"  max rel err {e:.3e}")
    assert int(err.item()) == 0
    assert e <= TOL_FP8_PATH
    return y


def test_tiny_workload():
    need_gpu()
    _check(inputs.W_TINY, 1, 256, 1024)


@pytest.mark.parametrize("M", [1, 8, 32, 37, 64, 128])
def test_bsgemm_qwen3_shape(M):
    need_gpu()
    _check(inputs.W_BSGEMM, M, 2560, 9728, extra=M)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32, 37, 64, 96, 128])
def test_mxfp8_qwen3_shape(M):
    need_gpu()
    _check(inputs.W_MXFP8, M, 2560, 9728, extra=M)


@pytest.mark.parametrize("mode", [ops.MLP_BSGEMM, ops.MLP_MXFP8])
def test_small_shapes_ragged(mode):
    need_gpu()
    wl = inputs.W_MXFP8 if mode == ops.MLP_MXFP8 else inputs.W_BSGEMM
    for M in (3, 17, 100):
        _check(wl, M, 384, 640, extra=1000 + M)


def test_deterministic_and_workspace_reuse():
    need_gpu()
    mode, w, deq = _setup(inputs.W_BSGEMM, 2560, 9728)
    ws = ops.new_mlp_workspace(128, 2560, 9728, mode)
    xa = inputs.mlp_activations(inputs.W_BSGEMM, 128, 2560, extra=7)
    xs = inputs.mlp_activations(inputs.W_BSGEMM, 5, 2560, extra=8)
    y1 = ops.swiglu_mlp_fp8(to_dev_bf16(xa), *w, mode, workspace=ws)
    y2 = ops.swiglu_mlp_fp8(to_dev_bf16(xa), *w, mode, workspace=ws)
    y3 = ops.swiglu_mlp_fp8(to_dev_bf16(xs), *w, mode, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = omlp.swiglu_mlp(f32(xs), *deq, mode)["y"]
    assert max_rel_err(from_dev_bf16(y3), ref) <= TOL_FP8_PATH
    # the control words are back to zero after every call
    ctrl = ws[:16384].cpu().numpy()
    assert not ctrl.any()


def test_wrong_scale_strides_fail_loudly():
    """A row-major MX scale tensor described with K-major strides (the layout
    bug of the FP8 page) must produce a large error, the right strides pass."""
    need_gpu()
    mode, w, deq = _setup(inputs.W_MXFP8, 2560, 9728)
    xb = inputs.mlp_activations(inputs.W_MXFP8, 4, 2560, extra=3)
    ref = omlp.swiglu_mlp(f32(xb), *deq, mode)["y"]
    good = from_dev_bf16(ops.swiglu_mlp_fp8(to_dev_bf16(xb), *w, mode))
    assert max_rel_err(good, ref) <= TOL_FP8_PATH
    rowmajor = [ops.QWeight(q.w, q.scale.contiguous()) for q in w]
    # contiguous() keeps the logical layout; lie about it by swapping strides
    bad_w = []
    for q in rowmajor:
        s = q.scale
        lie = torch.as_strided(s, (s.shape[0], s.shape[1]), (1, s.shape[0]))
        bad_w.append(ops.QWeight(q.w, lie))
    bad = from_dev_bf16(ops.swiglu_mlp_fp8(to_dev_bf16(xb), *bad_w, mode))
    torch.cuda.synchronize()
    assert max_rel_err(bad, ref) > 0.2


def _pack_reference(q):
    """The fragment-packed layout written out with NumPy index arithmetic:
    fragment (nb, kb) at (nb * KB + kb) * 2048, lane l = r + 16 g holding row
    16 nb + r, columns 128 kb + 16 g .. at 16 l and 128 kb + 64 + 16 g .. at
    1024 + 16 l."""
    N, K = q.shape
    KB = K // 128
    t = q.reshape(N // 16, 16, KB, 2, 4, 16)            # nb, r, kb, half, g, byte
    t = t.transpose(0, 2, 3, 4, 1, 5)                   # nb, kb, half, g, r, byte
    return np.ascontiguousarray(t).reshape(N, K)


def test_pack_weight_layout():
    need_gpu()
    _, w, _ = _setup(inputs.W_BSGEMM, 2560, 9728)
    for qw in w:
        p = ops.pack_weight(qw)
        torch.cuda.synchronize()
        assert np.array_equal(p.w.cpu().numpy(), _pack_reference(qw.w.cpu().numpy()))


@pytest.mark.parametrize("workload", [inputs.W_BSGEMM, inputs.W_MXFP8])
@pytest.mark.parametrize("M", [1, 4, 8, 16, 37, 64, 128])
def test_packed_weights_bit_identical(workload, M):
    """The MLP reads fragment-packed weights (ld_w = 0) to the same result,
    bit for bit, at every launch shape (M <= 4, <= 16, each M tile count)."""
    need_gpu()
    mode, w, _ = _setup(workload, 2560, 9728)
    packed = [ops.pack_weight(q) for q in w]
    xb = to_dev_bf16(inputs.mlp_activations(workload, M, 2560, extra=100 + M))
    log(f"mlp packed workload={workload} M={M}")
    y0 = ops.swiglu_mlp_fp8(xb, *w, mode)
    y1 = ops.swiglu_mlp_fp8(xb, *packed, mode)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
