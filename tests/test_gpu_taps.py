"""The fused quantisers, read through the library's debug taps: the codes
and scales each fused kernel hands to its GEMM equal the oracle's activation
quantisation of the GPU's own bf16 input of that step, bit for bit.

  * swiglu_mlp_fp8's x operand: quantised inside the gate/up GEMM (M <= 4)
    or by the x kernel (M > 4), bsgemm and MXFP8;
  * swiglu_mlp_fp8's h operand: h = silu(g) u and its quantisation, formed
    from the gate/up GEMM's g and u in the down GEMM's prologue (M <= 16) or
    in one launch of its own (M > 16);
  * the decode step, every slow layer: the attention kernel's quantised
    output (operand of the output projection) against its bf16 output, and
    the row finisher's quantised MLP input against its RMSNorm rows.  With
    the operands pinned, the output projection and the MLP of each layer are
    then checked on the GPU's own operand (teacher forcing at the operand
    level), which brings back the 4-head batch-24 model: there a rounding
    flip of one attention output moves a residual entry by ~2 % when the
    oracle quantises its own attention output instead."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8, mlp as omlp
from fp8_transformer_step_amd import inputs, model, ops
from _helpers import TOL_FP8_PATH, f32, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _bf16_np(u8):
    """bf16 bytes -> float32 values."""
    return (np.ascontiguousarray(u8).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def _decode_operand(tap, M, K, mode):
    """(codes [M, K], scales) of an operand in the tap layout (see the
    header): fragments [T][KB] with lane l = r + 16 g holding row 16 t + r at
    columns 128 kb + 16 g + 64 half + byte; then the scale slots [T][KB]."""
    T, KB = (M + 15) // 16, K // 128
    nf = T * KB * 2048
    f = tap[:nf].reshape(T, KB, 4, 16, 2, 16)                 # t, kb, g, r, half, byte
    codes = f.transpose(0, 3, 1, 4, 2, 5).reshape(T * 16, K)  # row 16t + r, col 128kb + 64half + 16g + byte
    sc = np.ascontiguousarray(tap[nf:nf + T * KB * 64])
    if mode == omlp.MODE_BSGEMM:
        s = sc.view(np.float32).reshape(T, KB, 16).transpose(0, 2, 1).reshape(T * 16, KB)
    else:
        s = sc.reshape(T, KB, 4, 16).transpose(0, 3, 1, 2).reshape(T * 16, KB * 4)
    return codes[:M], s[:M]


def _operand_bytes(M, K):
    T, KB = (M + 15) // 16, K // 128
    return T * KB * (2048 + 64)


def _check_operand(tap, x_f32, mode, what):
    M, K = x_f32.shape
    codes, s = _decode_operand(tap, M, K, mode)
    q, so, _ = omlp.quant_act(x_f32, mode)
    assert np.array_equal(codes, q), f"{what}: codes differ at {np.argwhere(codes != q)[:4].tolist()}"
    assert np.array_equal(s, so), f"{what}: scales differ"
    return q, so


@pytest.mark.parametrize("mode", [ops.MLP_BSGEMM, ops.MLP_MXFP8])
@pytest.mark.parametrize("M", [1, 3, 4, 8, 37])
def test_mlp_x_operand_tap(mode, M):
    """M <= 4: the gate/up GEMM's in-register quantisation; M > 4: the x kernel."""
    need_gpu()
    H, I = 2560, 9728
    wl = inputs.W_MXFP8 if mode == ops.MLP_MXFP8 else inputs.W_BSGEMM
    w = [ops.quantize_weight(to_dev_bf16(wb), mode) for wb in inputs.mlp_weights(wl, H, I)]
    xb = inputs.mlp_activations(wl, M, H, extra=500 + M)
    tap = torch.zeros(_operand_bytes(M, H), dtype=torch.uint8, device="cuda")
    log(f"x operand tap mode={mode} M={M}")
    ops.set_debug_tap(ops.TAP_MLP_X, tap)
    try:
        ops.swiglu_mlp_fp8(to_dev_bf16(xb), *w, mode)
        torch.cuda.synchronize()
    finally:
        ops.set_debug_tap(ops.TAP_MLP_X, None)
    _check_operand(tap.cpu().numpy(), f32(xb), mode, "x operand")


@pytest.mark.parametrize("mode", [ops.MLP_BSGEMM, ops.MLP_MXFP8])
@pytest.mark.parametrize("M", [1, 4, 5, 16, 29, 37, 64, 128])
def test_mlp_h_operand_tap(mode, M):
    """The kernel that quantises h: h = silu(g) u as it formed it (against
    the oracle's h from the same x operand), and the down GEMM's operand of h
    bit-exact with the oracle's activation quantisation of that h.  M <= 16:
    the down GEMM's own prologue (after the register gate/up kernel at M <= 4,
    the one-tile LDS kernel at 5 and 16); M > 16: the SwiGLU-quantise launch
    (29 two tiles, 37 and 64 four, 128 eight), where the 96 gate/up tiles past
    the first 512 are split over K and their quarters summed."""
    need_gpu()
    H, I = 2560, 9728
    wl = inputs.W_MXFP8 if mode == ops.MLP_MXFP8 else inputs.W_BSGEMM
    wbits = inputs.mlp_weights(wl, H, I)
    w = [ops.quantize_weight(to_dev_bf16(wb), mode) for wb in wbits]
    xb = inputs.mlp_activations(wl, M, H, extra=700 + M)
    nh = M * I * 4
    tap = torch.zeros(nh + _operand_bytes(M, I), dtype=torch.uint8, device="cuda")
    log(f"h operand tap mode={mode} M={M}")
    ops.set_debug_tap(ops.TAP_MLP_H, tap)
    try:
        ops.swiglu_mlp_fp8(to_dev_bf16(xb), *w, mode)
        torch.cuda.synchronize()
    finally:
        ops.set_debug_tap(ops.TAP_MLP_H, None)
    t = tap.cpu().numpy()
    h = np.ascontiguousarray(t[:nh]).view(np.float32).reshape(M, I)
    assert np.all(np.isfinite(h))
    _check_operand(t[nh:], h, mode, "h operand")
    if mode == ops.MLP_MXFP8:
        deq = [fp8.dequant_mx_1x32(*fp8.quant_mx_1x32(f32(b))) for b in wbits]
    else:
        deq = [fp8.dequant_block_fp32(*fp8.quant_weight_128x128(f32(b)), 128, 128) for b in wbits]
    ref = omlp.swiglu_mlp(f32(xb), *deq, mode)["h"].astype(np.float64)
    # fp32 accumulation of 2560 products and the fp32 exp / reciprocal against
    # float64: 1e-3 of max |h| (measured up to 1.4e-4 with the MX outliers),
    # far below the 2^-4 relative step of an e4m3 code
    assert max_rel_err(h.astype(np.float64), ref) <= 1e-3


def test_tap_too_small_is_refused():
    need_gpu()
    H, I = 2560, 9728
    w = [ops.quantize_weight(to_dev_bf16(wb), ops.MLP_BSGEMM) for wb in inputs.mlp_weights(inputs.W_BSGEMM, H, I)]
    x = to_dev_bf16(inputs.mlp_activations(inputs.W_BSGEMM, 2, H, extra=1))
    ops.set_debug_tap(ops.TAP_MLP_X, torch.zeros(_operand_bytes(2, H) - 16, dtype=torch.uint8, device="cuda"))
    try:
        with pytest.raises(Exception):
            ops.swiglu_mlp_fp8(x, *w, ops.MLP_BSGEMM)
    finally:
        ops.set_debug_tap(ops.TAP_MLP_X, None)


@pytest.mark.parametrize("batch,n_heads", [(24, 4), (5, 4), (64, 8)])
def test_step_operand_taps_every_slow_layer(batch, n_heads):
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=batch, n_heads=n_heads))
    c = host.cfg
    B, H, L = c.batch, c.hidden, c.n_slow_layers
    A = c.n_heads * c.head_dim
    T = (B + 15) // 16
    part = B * A * 2 + T * (A // 128) * (2048 + 64) + B * H * 2 + T * (H // 128) * (2048 + 64)
    tap = torch.zeros(L * part, dtype=torch.uint8, device="cuda")
    dm = model.device_model(host)
    kv, _, _ = model.device_kv(host)
    slow = torch.empty((2 * L + 1, B, H), dtype=torch.bfloat16, device="cuda")
    log(f"step taps B={B} heads={n_heads} L={L}")
    ops.set_debug_tap(ops.TAP_STEP_SLOW, tap)
    try:
        ops.dual_ar_decode_step(dm, kv, torch.from_numpy(host.prev_codes).cuda(), slow_taps=slow)
        torch.cuda.synchronize()
    finally:
        ops.set_debug_tap(ops.TAP_STEP_SLOW, None)
    t = tap.cpu().numpy()
    xs = slow.float().cpu().numpy().astype(np.float64)
    for l in range(L):
        o = l * part
        ao = _bf16_np(t[o:o + B * A * 2]).reshape(B, A)
        o += B * A * 2
        op = t[o:o + _operand_bytes(B, A)]
        o += _operand_bytes(B, A)
        xn = _bf16_np(t[o:o + B * H * 2]).reshape(B, H)
        o += B * H * 2
        mp = t[o:o + _operand_bytes(B, H)]
        qo, so = _check_operand(op, ao, omlp.MODE_BSGEMM, f"layer {l} attention operand")
        qm, sm = _check_operand(mp, xn, omlp.MODE_BSGEMM, f"layer {l} MLP operand")
        d = host.slow[l]
        wo = oracle.dequant_weight(f32(d["o"]))[2]
        # the finisher's RMSNorm rows against the oracle's on the GPU's residual
        ref_xn = oracle.rmsnorm(xs[2 * l + 1], f32(d["norm_mlp"]), c.rms_eps)
        assert max_rel_err(xn, ref_xn) <= 2 ** -7
        # output projection + residual on the GPU's own operand
        mid = oracle.round_bf16(xs[2 * l] + omlp.linear_dequant(fp8.dequant_block_fp32(qo, so, 1, 128), wo))
        e1 = max_rel_err(xs[2 * l + 1], mid)
        # MLP + residual on the GPU's own operand (the same bytes the oracle makes from xn)
        p = {k: oracle.dequant_weight(f32(d[k]))[2] for k in ("gate", "up", "down")}
        y = omlp.swiglu_mlp(xn.astype(np.float32), p["gate"], p["up"], p["down"], omlp.MODE_BSGEMM)["y"]
        e2 = max_rel_err(xs[2 * l + 2], oracle.round_bf16(xs[2 * l + 1] + y))
        log(f"  layer {l}: output projection {e1:.3e}, mlp {e2:.3e}")
        assert e1 <= TOL_FP8_PATH and e2 <= TOL_FP8_PATH
