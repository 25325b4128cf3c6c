"""qlinear_quantize on the GPU must equal the oracle bit for bit (bytes and
scales), for all three modes, row-major and K-major scale strides."""

import numpy as np
import pytest
import torch

from oracle import fp8
from fp8_transformer_step_amd import inputs, ops
from _helpers import f32, log, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(bits, mode, k_major=False):
    x = to_dev_bf16(bits)
    q, s = ops.qlinear_quantize(x, mode, k_major=k_major)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _oracle(bits, mode):
    x = f32(bits)
    if mode == ops.Q_ACT_1x128:
        return fp8.quant_act_1x128(x)
    if mode == ops.Q_WGT_128x128:
        return fp8.quant_weight_128x128(x)
    return fp8.quant_mx_1x32(x)


@pytest.mark.parametrize("mode,shape,k_major", [
    (ops.Q_ACT_1x128, (37, 2560), False),
    (ops.Q_ACT_1x128, (128, 2560), True),
    (ops.Q_ACT_1x128, (1, 9728), False),
    (ops.Q_WGT_128x128, (384, 2560), False),
    (ops.Q_WGT_128x128, (2560, 9728), False),
    (ops.Q_MX_1x32, (37, 2560), True),
    (ops.Q_MX_1x32, (5, 9728), False),
    (ops.Q_MX_1x32, (9728, 2560), True),
])
def test_quantize_bit_exact_random(mode, shape, k_major):
    need_gpu()
    log(f"quantize mode={mode} shape={shape} k_major={k_major}")
    bits = inputs.normal_bf16(inputs.W_BSGEMM, 50 + mode, shape, std=0.5)
    # widen the dynamic range: per-row powers of two and sprinkled outliers
    g = np.random.default_rng(1)
    v = f32(bits) * (2.0 ** g.integers(-20, 20, size=(shape[0], 1))).astype(np.float32)
    v[g.random(shape) < 0.01] *= 300.0
    bits = inputs.f32_to_bf16_bits(v)
    q, s = _run(bits, mode, k_major)
    qo, so = _oracle(bits, mode)
    assert np.array_equal(q, qo), f"{np.count_nonzero(q != qo)} bytes differ"
    assert np.array_equal(s, so)


def test_quantize_every_bf16_pattern_unit_scale():
    """Every finite bf16 value passes through the encoder with s = 1: each
    128-group carries 448 so that amax / 448 = 1 exactly."""
    need_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = f32(bits)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    n = len(vals)
    per = 127
    rows = (n + per - 1) // per
    x = np.zeros((rows, 128), np.float32)
    flat = np.zeros(rows * per, np.float32)
    flat[:n] = vals
    x[:, :per] = flat.reshape(rows, per)
    x[:, per] = 448.0
    xb = inputs.f32_to_bf16_bits(x)
    q, s = _run(xb, ops.Q_ACT_1x128)
    qo, so = fp8.quant_act_1x128(x)
    assert np.all(so == 1.0) and np.array_equal(s, so)
    assert np.array_equal(q, qo)


def test_quantize_zero_and_tiny_groups():
    need_gpu()
    x = np.zeros((4, 256), np.float32)
    x[1, 5] = 1e-38          # subnormal-adjacent amax
    x[2, :] = -0.0
    x[3, 7] = -3e-39
    xb = inputs.f32_to_bf16_bits(x)
    for mode in (ops.Q_ACT_1x128, ops.Q_MX_1x32):
        q, s = _run(xb, mode)
        qo, so = _oracle(xb, mode)
        assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_mx_scale_strides_honoured():
    """The same MX quantisation written K-major (stride (1, rows)) and
    row-major must hold the same logical exponents."""
    need_gpu()
    bits = inputs.normal_bf16(inputs.W_MXFP8, 60, (96, 512))
    _, s_k = _run(bits, ops.Q_MX_1x32, k_major=True)
    _, s_r = _run(bits, ops.Q_MX_1x32, k_major=False)
    assert np.array_equal(s_k, s_r)


def test_division_and_lower_clamp_cases_bit_exact():
    """The inputs that pin the oracle's fp32 division (an exact quotient just
    above an e4m3 midpoint whose fp32 rounding lands on it) and the UE8M0
    lower clamp (groups with amax in [2^-133, 2^-119)), through the
    standalone quantiser in all three modes: bytes and scales bit-exact."""
    need_gpu()
    from test_oracle_fp8 import _DIV_CASES
    rows = []
    for amax, x in _DIV_CASES:
        r = np.zeros(256, np.float32)
        r[3], r[77], r[130], r[200] = amax, x, -amax, -x
        rows.append(r)
        rows.append(r * np.float32(2.0 ** -60))
        rows.append(r * np.float32(2.0 ** 40))
    for vals in ([2.0 ** -120], [2.0 ** -133], [1.5 * 2.0 ** -129, -2.0 ** -128], [1.75 * 2.0 ** -120],
                 [2.0 ** -119], [2.0 ** -118, 2.0 ** -133]):
        r = np.zeros(256, np.float32)
        r[:len(vals)] = vals
        r[100:100 + len(vals)] = vals
        rows.append(r)
    while len(rows) % 128:
        rows.append(rows[len(rows) % 12])
    x = np.stack(rows)
    xb = inputs.f32_to_bf16_bits(x)
    assert np.array_equal(f32(xb), x), "the cases must be exact bf16 values"
    for mode in (ops.Q_ACT_1x128, ops.Q_WGT_128x128, ops.Q_MX_1x32):
        q, s = _run(xb, mode)
        qo, so = _oracle(xb, mode)
        assert np.array_equal(q, qo), f"mode {mode}: {np.count_nonzero(q != qo)} bytes differ"
        assert np.array_equal(s, so), f"mode {mode}: scales differ"
