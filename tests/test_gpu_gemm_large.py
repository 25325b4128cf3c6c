"""fp8_gemm_mx (the MXFP8 GEMM for prefill shapes) on the GPU against the
oracle.  Both sides quantise the same bf16 operands on their own (the GPU
with qlinear_quantize mode 2, the oracle with its OCP MX rule; the bytes are
checked equal), then the GPU product is compared with the float64
dequantised product: whole matrices at sizes that span several tiles and a
ragged M, sampled rows at 4096^3, both exponent layouts (row-major and
K-major), and an exact case (small codes, distinct power-of-two exponents per
group) that must match bit for bit and fails on any exponent or operand
index mix-up."""

import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from oracle.dual_ar import round_bf16
from _helpers import TOL_FP8_PATH, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16
from fp8_transformer_step_amd import _lib, inputs, ops

pytestmark = pytest.mark.gpu


def _operands(M, N, K, extra):
    a = inputs.normal_bf16(inputs.W_MXFP8, inputs.T_X, (M, K), 1.0, extra)
    b = inputs.normal_bf16(inputs.W_MXFP8, inputs.T_WG, (N, K), 0.02, extra)
    return a, b


def _gpu_quant(bits, k_major):
    return ops.qlinear_quantize(to_dev_bf16(bits), ops.Q_MX_1x32, k_major=k_major)


def _run(a_bits, b_bits, k_major_a=False, k_major_b=True):
    qa, ea = _gpu_quant(a_bits, k_major_a)
    qb, eb = _gpu_quant(b_bits, k_major_b)
    c = ops.fp8_gemm_mx(qa, ea, qb, eb)
    torch.cuda.synchronize()
    return qa, ea, qb, eb, c


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 512), (1000, 256, 384), (1, 128, 256),
                                   (77, 640, 1280)])
def test_matches_oracle(M, N, K):
    need_gpu()
    a, b = _operands(M, N, K, extra=M + N + K)
    qa, ea, qb, eb, c = _run(a, b)
    oqa, oea = ofp8.quant_mx_1x32(f32(a))
    oqb, oeb = ofp8.quant_mx_1x32(f32(b))
    assert np.array_equal(qa.cpu().numpy(), oqa) and np.array_equal(ea.cpu().numpy(), oea)
    assert np.array_equal(qb.cpu().numpy(), oqb) and np.array_equal(eb.cpu().numpy(), oeb)
    ref = ofp8.dequant_mx_1x32(oqa, oea) @ ofp8.dequant_mx_1x32(oqb, oeb).T
    e = max_rel_err(from_dev_bf16(c), ref)
    log(f"gemm mx {M}x{N}x{K}: max rel err {e:.2e}")
    assert e <= TOL_FP8_PATH


@pytest.mark.parametrize("k_major_a,k_major_b", [(True, True), (False, False)])
def test_exponent_layouts(k_major_a, k_major_b):
    need_gpu()
    M, N, K = 192, 256, 256
    a, b = _operands(M, N, K, extra=7)
    c = _run(a, b, k_major_a, k_major_b)[4]
    oqa, oea = ofp8.quant_mx_1x32(f32(a))
    oqb, oeb = ofp8.quant_mx_1x32(f32(b))
    ref = ofp8.dequant_mx_1x32(oqa, oea) @ ofp8.dequant_mx_1x32(oqb, oeb).T
    assert max_rel_err(from_dev_bf16(c), ref) <= TOL_FP8_PATH


def test_full_size_sampled_rows():
    """4096^3: 48 rows (first, last, a seeded sample) computed by the oracle."""
    need_gpu()
    M = N = K = 4096
    a, b = _operands(M, N, K, extra=4096)
    c = _run(a, b)[4]
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).integers(0, M, 46)]))
    oqb, oeb = ofp8.quant_mx_1x32(f32(b))
    bd = ofp8.dequant_mx_1x32(oqb, oeb)
    oqa, oea = ofp8.quant_mx_1x32(f32(a[rows]))
    ref = ofp8.dequant_mx_1x32(oqa, oea) @ bd.T
    got = from_dev_bf16(c[torch.from_numpy(rows).cuda()])
    e = max_rel_err(got, ref)
    log(f"gemm mx 4096^3 sampled rows: max rel err {e:.2e}")
    assert e <= TOL_FP8_PATH


def test_exact_small_codes_bit_for_bit():
    """Codes of +-{0, 0.5, 1, 1.5, 2} and an exponent in [125, 129] per
    32-group: every product is a multiple of 2^-6 of magnitude at most 64, so
    every partial sum over K = 512 stays below 2^15 and is exact in fp32, and
    C must be the bf16 rounding of the exact product.  A transposed exponent
    or operand index breaks this."""
    need_gpu()
    g = np.random.default_rng(11)
    M, N, K = 160, 256, 512
    codes = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0xB0, 0xB8, 0xBC, 0xC0], np.uint8)
    qa = codes[g.integers(0, len(codes), (M, K))]
    qb = codes[g.integers(0, len(codes), (N, K))]
    ea = g.integers(125, 130, (M, K // 32)).astype(np.uint8)
    eb = g.integers(125, 130, (N, K // 32)).astype(np.uint8)
    ref = round_bf16(ofp8.dequant_mx_1x32(qa, ea) @ ofp8.dequant_mx_1x32(qb, eb).T)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    eb_km = torch.from_numpy(np.ascontiguousarray(eb.T)).cuda().t()          # K-major exponents
    c = ops.fp8_gemm_mx(d(qa), d(ea), d(qb), eb_km)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(c), ref)
    # the same operands with A's exponent rows shuffled must not match
    perm = np.roll(np.arange(M), 1)
    c2 = ops.fp8_gemm_mx(d(qa), d(ea[perm]), d(qb), eb_km)
    torch.cuda.synchronize()
    assert not np.array_equal(from_dev_bf16(c2), ref)


def test_argument_checks():
    need_gpu()
    q = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    e = torch.zeros((128, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        ops.fp8_gemm_mx(q, e, q[:, :128], e)
    with pytest.raises(TypeError):
        ops.fp8_gemm_mx(q.float(), e, q, e)
    qn = torch.zeros((100, 256), dtype=torch.uint8, device="cuda")            # N not a multiple of 128
    en = torch.zeros((100, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.Fp8sError):
        ops.fp8_gemm_mx(q, e, qn, en)


def _packed_reference(q, e):
    """The packed layout written out from its definition (fp8_pack_mx)."""
    R, K = q.shape
    KB, Rp = K // 128, (R + 127) // 128 * 128
    qp = np.zeros((Rp, K), np.uint8)
    qp[:R] = q
    ep = np.full((Rp, K // 32), 127, np.uint8)
    ep[:R] = e
    frags = np.zeros((Rp // 16, KB, 2, 64, 16), np.uint8)
    for l in range(64):
        r, g = l % 16, l // 16
        for half in range(2):
            cols = np.arange(16) + 64 * half + 16 * g
            frags[:, :, half, l, :] = qp.reshape(Rp // 16, 16, KB, 128)[:, r][:, :, cols]
    words = np.zeros((Rp // 64, KB, 64, 4), np.uint8)
    for l in range(64):
        r, g = l % 16, l // 16
        for i in range(4):
            words[:, :, l, i] = ep.reshape(Rp // 64, 64, KB, 4)[:, 16 * i + r, :, g]
    return np.concatenate([frags.reshape(-1), words.reshape(-1)])


def test_packed_layout_bytes():
    need_gpu()
    a, _ = _operands(200, 128, 384, extra=3)
    qa, ea = _gpu_quant(a, True)
    pa = ops.fp8_pack_mx(qa, ea)
    torch.cuda.synchronize()
    want = _packed_reference(qa.cpu().numpy(), ea.cpu().numpy())
    assert np.array_equal(pa.data.cpu().numpy(), want)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (1000, 256, 384), (1, 128, 256), (77, 640, 1280),
                                   (300, 384, 512)])
def test_packed_matches_unpacked_and_oracle(M, N, K):
    need_gpu()
    a, b = _operands(M, N, K, extra=M + N + K)
    qa, ea, qb, eb, c = _run(a, b, True, True)
    cp = ops.fp8_gemm_mx_packed(ops.fp8_pack_mx(qa, ea), ops.fp8_pack_mx(qb, eb))
    torch.cuda.synchronize()
    assert torch.equal(cp.view(torch.int16), c.view(torch.int16))
    oqa, oea = ofp8.quant_mx_1x32(f32(a))
    oqb, oeb = ofp8.quant_mx_1x32(f32(b))
    ref = ofp8.dequant_mx_1x32(oqa, oea) @ ofp8.dequant_mx_1x32(oqb, oeb).T
    assert max_rel_err(from_dev_bf16(cp), ref) <= TOL_FP8_PATH


def test_packed_full_size_sampled_rows():
    need_gpu()
    M = N = K = 4096
    a, b = _operands(M, N, K, extra=4097)
    qa, ea = _gpu_quant(a, True)
    qb, eb = _gpu_quant(b, True)
    c = ops.fp8_gemm_mx_packed(ops.fp8_pack_mx(qa, ea), ops.fp8_pack_mx(qb, eb))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(6).integers(0, M, 46)]))
    oqb, oeb = ofp8.quant_mx_1x32(f32(b))
    oqa, oea = ofp8.quant_mx_1x32(f32(a[rows]))
    ref = ofp8.dequant_mx_1x32(oqa, oea) @ ofp8.dequant_mx_1x32(oqb, oeb).T
    assert max_rel_err(from_dev_bf16(c[torch.from_numpy(rows).cuda()]), ref) <= TOL_FP8_PATH


# ---- bsgemm (128x128 weight blocks, 1x128 activation groups), packed ----

def _bs_run(a_bits, b_bits):
    qa, sa = ops.qlinear_quantize(to_dev_bf16(a_bits), ops.Q_ACT_1x128)
    qb, sb = ops.qlinear_quantize(to_dev_bf16(b_bits), ops.Q_WGT_128x128)
    c = ops.fp8_gemm_bs_packed(ops.fp8_pack_bs(qa, sa, 1), ops.fp8_pack_bs(qb, sb, 128))
    torch.cuda.synchronize()
    return qa, sa, qb, sb, c


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (1000, 256, 384), (1, 128, 256), (77, 640, 1280)])
def test_bs_packed_matches_oracle(M, N, K):
    need_gpu()
    a, b = _operands(M, N, K, extra=500 + M + N + K)
    qa, sa, qb, sb, c = _bs_run(a, b)
    oqa, osa = ofp8.quant_act_1x128(f32(a))
    oqb, osb = ofp8.quant_weight_128x128(f32(b))
    assert np.array_equal(qa.cpu().numpy(), oqa) and np.array_equal(sa.cpu().numpy(), osa)
    assert np.array_equal(qb.cpu().numpy(), oqb) and np.array_equal(sb.cpu().numpy(), osb)
    ref = ofp8.dequant_block_fp32(oqa, osa, 1, 128) @ ofp8.dequant_block_fp32(oqb, osb, 128, 128).T
    e = max_rel_err(from_dev_bf16(c), ref)
    log(f"gemm bs {M}x{N}x{K}: max rel err {e:.2e}")
    assert e <= TOL_FP8_PATH


def test_bs_packed_full_size_sampled_rows():
    need_gpu()
    M = N = K = 4096
    a, b = _operands(M, N, K, extra=4098)
    c = _bs_run(a, b)[4]
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(8).integers(0, M, 46)]))
    oqb, osb = ofp8.quant_weight_128x128(f32(b))
    oqa, osa = ofp8.quant_act_1x128(f32(a[rows]))
    ref = ofp8.dequant_block_fp32(oqa, osa, 1, 128) @ ofp8.dequant_block_fp32(oqb, osb, 128, 128).T
    assert max_rel_err(from_dev_bf16(c[torch.from_numpy(rows).cuda()]), ref) <= TOL_FP8_PATH


def test_bs_exact_small_codes_bit_for_bit():
    """Codes of +-{0, 0.5, 1, 1.5, 2} with a power-of-two scale in [2^-2, 2^2]
    per activation (row, K block) and per weight block: every product is a
    multiple of 2^-6 at most 64 in magnitude, partial sums over K = 512 stay
    below 2^15, so C must be the bf16 rounding of the exact product; a
    wrong row, block or K-block scale index breaks it."""
    need_gpu()
    g = np.random.default_rng(12)
    M, N, K = 160, 256, 512
    codes = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0xB0, 0xB8, 0xBC, 0xC0], np.uint8)
    qa = codes[g.integers(0, len(codes), (M, K))]
    qb = codes[g.integers(0, len(codes), (N, K))]
    sa = np.ldexp(1.0, g.integers(-2, 3, (M, K // 128))).astype(np.float32)
    sb = np.ldexp(1.0, g.integers(-2, 3, (N // 128, K // 128))).astype(np.float32)
    ref = round_bf16(ofp8.dequant_block_fp32(qa, sa, 1, 128) @ ofp8.dequant_block_fp32(qb, sb, 128, 128).T)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    sa_km = torch.from_numpy(np.ascontiguousarray(sa.T)).cuda().t()          # K-major activation scales
    c = ops.fp8_gemm_bs_packed(ops.fp8_pack_bs(d(qa), sa_km, 1), ops.fp8_pack_bs(d(qb), d(sb), 128))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(c), ref)
    c2 = ops.fp8_gemm_bs_packed(ops.fp8_pack_bs(d(qa), d(sa[::-1].copy()), 1), ops.fp8_pack_bs(d(qb), d(sb), 128))
    torch.cuda.synchronize()
    assert not np.array_equal(from_dev_bf16(c2), ref)
