"""swiglu_mlp_fp8_noalloc through the C ABI against swiglu_mlp_fp8 (the same
kernels on a caller's workspace): bit-identical outputs on two calls in a
row, the second with fewer rows, both weight layouts; shapes beyond the
scratch array are refused before any launch."""

import numpy as np
import pytest
import torch

from oracle import mlp as omlp
from fp8_transformer_step_amd import _lib, inputs, ops
from _helpers import TOL_FP8_PATH, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

H, I = 2560, 9728


def _weights(mode, packed):
    wl = inputs.W_MXFP8 if mode == ops.MLP_MXFP8 else inputs.W_BSGEMM
    ws = []
    for wb in inputs.mlp_weights(wl, H, I):
        qw = ops.quantize_weight(to_dev_bf16(wb), mode)
        ws.append(ops.pack_weight(qw) if packed else qw)
    return wl, ws


def _noalloc(x, mode, w, err):
    M = x.shape[0]
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    rc = _lib.load().swiglu_mlp_fp8_noalloc(x.data_ptr(), M, H, I, mode, w[0].as_c(), w[1].as_c(), w[2].as_c(),
                                            y.data_ptr(), err.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _lib.check(rc)
    return y


@pytest.mark.parametrize("mode,packed", [(ops.MLP_BSGEMM, True), (ops.MLP_MXFP8, False)])
def test_noalloc_matches_workspace_entry_point(mode, packed):
    need_gpu()
    wl, w = _weights(mode, packed)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for M in (128, 5):
        log(f"noalloc mode={mode} packed={packed} M={M}")
        xb = inputs.mlp_activations(wl, M, H, extra=300 + M)
        x = to_dev_bf16(xb)
        got = _noalloc(x, mode, w, err)
        want = ops.swiglu_mlp_fp8(x, *w, mode)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert int(err.item()) == 0
    # the last (smaller) call also against the oracle
    from oracle import fp8
    deq = []
    for wb in inputs.mlp_weights(wl, H, I):
        w32 = f32(wb)
        if mode == ops.MLP_BSGEMM:
            q, s = fp8.quant_weight_128x128(w32)
            deq.append(fp8.dequant_block_fp32(q, s, 128, 128))
        else:
            q, s = fp8.quant_mx_1x32(w32)
            deq.append(fp8.dequant_mx_1x32(q, s))
    ref = omlp.swiglu_mlp(f32(xb), *deq, mode)["y"]
    assert max_rel_err(from_dev_bf16(got), ref) <= TOL_FP8_PATH


def test_noalloc_refuses_shapes_beyond_its_scratch():
    need_gpu()
    lib = _lib.load()
    cap = int(lib.swiglu_mlp_fp8_noalloc_max_bytes())
    assert cap == 32 << 20
    assert int(lib.swiglu_mlp_fp8_workspace_size(128, H, I, ops.MLP_BSGEMM)) <= cap
    Ib = 4 * I                                  # inter 38912 at M = 128 needs more than the array
    assert int(lib.swiglu_mlp_fp8_workspace_size(128, H, Ib, ops.MLP_BSGEMM)) > cap
    _, w = _weights(ops.MLP_BSGEMM, False)      # never read: the size check comes first
    x = torch.zeros((128, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((128, H), dtype=torch.bfloat16, device="cuda")
    rc = lib.swiglu_mlp_fp8_noalloc(x.data_ptr(), 128, H, Ib, ops.MLP_BSGEMM, w[0].as_c(), w[1].as_c(),
                                    w[2].as_c(), y.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert rc == -2                             # FP8S_EUNSUPPORTED
