"""swiglu_mlp_fp8_large (the SwiGLU MLP at prefill sizes, on the packed
prefill GEMMs) on the GPU against the oracle: the Qwen3-4B-shaped bsgemm and
MXFP8 workloads at M that are one row, ragged, one tile and several tiles
(whole outputs), M = 4096 on sampled rows (the MLP acts on each row alone,
so a sampled row is the oracle's M = 1 case), the tiny workload's shape,
strided x / y, agreement with the decode kernel where both apply, and
bit-identical repeats on a reused workspace."""

import numpy as np
import pytest
import torch

from oracle import fp8, mlp as omlp
from fp8_transformer_step_amd import inputs, ops
from _helpers import TOL_FP8_PATH, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

_CACHE = {}


def _setup(workload, H, I):
    """Weights quantised on the GPU (bytes checked equal to the oracle's),
    packed for the prefill GEMMs, and the oracle's dequantised copies."""
    key = (workload, H, I)
    if key in _CACHE:
        return _CACHE[key]
    mode = ops.MLP_MXFP8 if workload == inputs.W_MXFP8 else ops.MLP_BSGEMM
    qws, deq = [], []
    for wb in inputs.mlp_weights(workload, H, I):
        qw = ops.quantize_weight(to_dev_bf16(wb), mode)
        w32 = f32(wb)
        if mode == ops.MLP_BSGEMM:
            q, s = fp8.quant_weight_128x128(w32)
            d = fp8.dequant_block_fp32(q, s, 128, 128)
        else:
            q, s = fp8.quant_mx_1x32(w32)
            d = fp8.dequant_mx_1x32(q, s)
        torch.cuda.synchronize()
        assert np.array_equal(qw.w.cpu().numpy(), q) and np.array_equal(qw.scale.cpu().numpy(), s)
        qws.append(qw)
        deq.append(d)
    gate, up, down = qws
    qgu, sgu = torch.cat([gate.w, up.w]), torch.cat([gate.scale, up.scale])
    if mode == ops.MLP_BSGEMM:
        pgu, pd = ops.fp8_pack_bs(qgu, sgu, 128), ops.fp8_pack_bs(down.w, down.scale, 128)
    else:
        pgu, pd = ops.fp8_pack_mx(qgu, sgu), ops.fp8_pack_mx(down.w, down.scale)
    torch.cuda.synchronize()
    _CACHE[key] = (mode, qws, pgu, pd, deq)
    return _CACHE[key]


def _shape(workload):
    return (2560, 9728) if workload in (inputs.W_BSGEMM, inputs.W_MXFP8) else (256, 1024)


@pytest.mark.parametrize("workload", [inputs.W_BSGEMM, inputs.W_MXFP8])
@pytest.mark.parametrize("M", [1, 37, 128, 300])
def test_matches_oracle(workload, M):
    need_gpu()
    H, I = _shape(workload)
    mode, _, pgu, pd, deq = _setup(workload, H, I)
    xb = inputs.mlp_activations(workload, M, H, extra=900 + M)
    y = ops.swiglu_mlp_fp8_large(to_dev_bf16(xb), pgu, pd, mode)
    torch.cuda.synchronize()
    ref = omlp.swiglu_mlp(f32(xb), *deq, mode)["y"]
    e = max_rel_err(from_dev_bf16(y), ref)
    log(f"mlp large workload={workload} M={M}: max rel err {e:.3e}")
    assert e <= TOL_FP8_PATH


@pytest.mark.parametrize("workload", [inputs.W_BSGEMM, inputs.W_MXFP8])
@pytest.mark.parametrize("M", [4096, 3300])
def test_large_m_sampled_rows(workload, M):
    """M = 4096 (640 down-GEMM tiles) and 3300 (520): the tiles past the
    last full round of 512 run split over K, and they hold the last row
    tiles, so rows near M are sampled on purpose."""
    need_gpu()
    H, I = _shape(workload)
    mode, _, pgu, pd, deq = _setup(workload, H, I)
    xb = inputs.mlp_activations(workload, M, H, extra=950 + M)
    y = from_dev_bf16(ops.swiglu_mlp_fp8_large(to_dev_bf16(xb), pgu, pd, mode))
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.integers(0, M, 12), rng.integers(M - 200, M, 12)]))
    for r in rows:
        ref = omlp.swiglu_mlp(f32(xb[r:r + 1]), *deq, mode)["y"]
        assert max_rel_err(y[r:r + 1], ref) <= TOL_FP8_PATH, r


def test_strided_rows_and_tail_rows_untouched():
    """x and y are row slices of wider buffers; y's columns past hidden and
    the rows of the buffer past M keep their values."""
    need_gpu()
    H, I = _shape(inputs.W_BSGEMM)
    mode, _, pgu, pd, deq = _setup(inputs.W_BSGEMM, H, I)
    M = 70
    xb = inputs.mlp_activations(inputs.W_BSGEMM, M, H, extra=960)
    xbuf = torch.zeros((M, H + 64), dtype=torch.bfloat16, device="cuda")
    xbuf[:, :H] = to_dev_bf16(xb)
    ybuf = torch.full((M + 5, H + 32), 7.0, dtype=torch.bfloat16, device="cuda")
    ops.swiglu_mlp_fp8_large(xbuf[:, :H], pgu, pd, mode, y=ybuf[:M, :H])
    torch.cuda.synchronize()
    ref = omlp.swiglu_mlp(f32(xb), *deq, mode)["y"]
    assert max_rel_err(from_dev_bf16(ybuf[:M, :H].contiguous()), ref) <= TOL_FP8_PATH
    assert bool((ybuf[:M, H:] == 7.0).all()) and bool((ybuf[M:] == 7.0).all())


@pytest.mark.parametrize("workload", [inputs.W_BSGEMM, inputs.W_MXFP8])
def test_agrees_with_decode_kernel(workload):
    """At M = 64 both kernels compute the same quantised MLP; they differ
    only in fp32 summation order."""
    need_gpu()
    H, I = _shape(workload)
    mode, qws, pgu, pd, deq = _setup(workload, H, I)
    xb = inputs.mlp_activations(workload, 64, H, extra=970)
    a = ops.swiglu_mlp_fp8_large(to_dev_bf16(xb), pgu, pd, mode)
    b = ops.swiglu_mlp_fp8(to_dev_bf16(xb), *qws, mode)
    torch.cuda.synchronize()
    assert max_rel_err(from_dev_bf16(a), from_dev_bf16(b)) <= TOL_FP8_PATH


def test_invalid_sizes_rejected():
    need_gpu()
    H, I = _shape(inputs.W_BSGEMM)
    mode, _, pgu, pd, _ = _setup(inputs.W_BSGEMM, H, I)
    x = torch.zeros((4, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ops.swiglu_mlp_fp8_large(x, pd, pgu, mode)              # operands swapped
    assert ops._lib.load().swiglu_mlp_fp8_large_workspace_size(4, 2560, 100, mode) == 0
    assert ops._lib.load().swiglu_mlp_fp8_large_workspace_size(0, 2560, 9728, mode) == 0


@pytest.mark.parametrize("M", [5, 200])
def test_tiny_workload_shape(M):
    """hidden 256, inter 1024: two K blocks for the gate/up GEMM, 16 gate/up
    tiles per row block, one or two row tiles."""
    need_gpu()
    mode, _, pgu, pd, deq = _setup(inputs.W_TINY, 256, 1024)
    xb = inputs.mlp_activations(inputs.W_TINY, M, 256, extra=980 + M)
    y = ops.swiglu_mlp_fp8_large(to_dev_bf16(xb), pgu, pd, mode)
    torch.cuda.synchronize()
    assert max_rel_err(from_dev_bf16(y), omlp.swiglu_mlp(f32(xb), *deq, mode)["y"]) <= TOL_FP8_PATH


@pytest.mark.parametrize("workload", [inputs.W_BSGEMM, inputs.W_MXFP8])
def test_deterministic_with_reused_workspace(workload):
    """Two calls on one workspace, the second after a larger call, give the
    same bits (no state carried between calls)."""
    need_gpu()
    H, I = _shape(workload)
    mode, _, pgu, pd, _ = _setup(workload, H, I)
    x = to_dev_bf16(inputs.mlp_activations(workload, 150, H, extra=990))
    big = to_dev_bf16(inputs.mlp_activations(workload, 600, H, extra=991))
    ws = torch.empty(int(ops._lib.load().swiglu_mlp_fp8_large_workspace_size(600, H, I, mode)), dtype=torch.uint8,
                     device="cuda")
    a = ops.swiglu_mlp_fp8_large(x, pgu, pd, mode, workspace=ws).clone()
    ops.swiglu_mlp_fp8_large(big, pgu, pd, mode, workspace=ws)
    b = ops.swiglu_mlp_fp8_large(x, pgu, pd, mode, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
