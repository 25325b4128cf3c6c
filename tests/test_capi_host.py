"""CPU-only checks of the C ABI: every symbol declared in include/fp8step.h is
exported by libfp8step.so, and the host-side argument checks return the
documented error codes before anything is launched (no GPU needed)."""

import ctypes
import os
import re
import subprocess

import pytest

from fp8_transformer_step_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8step.h")

EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3
FAKE = 1 << 20            # a 16-byte aligned non-null address that is never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?[\s\*](\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for n in ("qlinear_quantize", "swiglu_mlp_fp8", "gqa_decode_attn", "fp8s_last_error",
              "swiglu_mlp_fp8_workspace_size", "gqa_decode_attn_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(_lib.SIGNATURES) == set(names)


def _q(*args):
    lib = _lib.load()
    return lib.qlinear_quantize(*args)


def test_quantize_argument_checks():
    assert _q(None, 4, 128, 128, 0, FAKE, 128, FAKE, 1, 1, None) == EINVAL
    assert _q(FAKE, 4, 100, 128, 0, FAKE, 128, FAKE, 1, 1, None) == EINVAL          # cols % 128
    assert _q(FAKE, 4, 32, 40, 2, FAKE, 40, FAKE, 1, 1, None) == EINVAL             # ld_q % 16
    assert _q(FAKE, 100, 128, 128, 1, FAKE, 128, FAKE, 1, 1, None) == EINVAL        # rows % 128 (weights)
    assert _q(FAKE, 4, 128, 128, 7, FAKE, 128, FAKE, 1, 1, None) == EINVAL          # mode
    assert _q(FAKE + 2, 4, 128, 128, 0, FAKE, 128, FAKE, 1, 1, None) == EINVAL      # misaligned x
    assert "aligned" in _lib.load().fp8s_last_error().decode()


def _qw():
    return _lib.QWeightC(FAKE, 256, FAKE, 2, 1)


def test_mlp_argument_checks():
    lib = _lib.load()
    ws = lib.swiglu_mlp_fp8_workspace_size(4, 256, 256, 0)
    assert ws > 0
    assert lib.swiglu_mlp_fp8_workspace_size(129, 256, 256, 0) == 0
    assert lib.swiglu_mlp_fp8_workspace_size(4, 200, 256, 0) == 0
    call = lambda M, H, I, mode, wsb: lib.swiglu_mlp_fp8(FAKE, M, H, I, mode, _qw(), _qw(), _qw(), FAKE,
                                                          FAKE, wsb, None, None)
    assert call(129, 256, 256, 0, ws) == EUNSUPPORTED
    assert call(0, 256, 256, 0, ws) == EINVAL
    assert call(4, 200, 256, 0, ws) == EINVAL
    assert call(4, 256, 256, 3, ws) == EINVAL
    assert call(4, 256, 256, 0, ws - 1) == EWORKSPACE
    bad = _lib.QWeightC(FAKE, 100, FAKE, 2, 1)                                      # ld_w < K
    assert lib.swiglu_mlp_fp8(FAKE, 4, 256, 256, 0, bad, _qw(), _qw(), FAKE, FAKE, ws, None, None) == EINVAL


def test_attention_argument_checks():
    lib = _lib.load()
    ws = lib.gqa_decode_attn_workspace_size(2, 32, 128, 400)
    assert ws >= 2 * 32 * 25 * 130 * 4
    call = lambda Hq, Hkv, D, st, wsb: lib.gqa_decode_attn(
        FAKE, FAKE, FAKE, 8 * 32768 * 128, 32768 * 128, st, FAKE, 2, Hq, Hkv, D, 32768, 400,
        ctypes.c_float(0.088), FAKE, FAKE, wsb, None, None)
    assert call(32, 6, 128, 128, ws) == EINVAL              # Hq % Hkv
    assert call(32, 8, 96, 128, ws) == EUNSUPPORTED         # head dim
    assert call(32, 2, 128, 128, ws) == EUNSUPPORTED        # group of 16 query heads
    assert call(32, 8, 128, 100, ws) == EINVAL              # stride_t not a multiple of 8
    assert call(32, 8, 128, 128, 16) == EWORKSPACE


def test_attention_mxkv_argument_checks():
    lib = _lib.load()
    ws = lib.gqa_decode_attn_workspace_size(2, 32, 128, 400)
    call = lambda Hq, Hkv, D, st, sst, wsb: lib.gqa_decode_attn_mxkv(
        FAKE, FAKE, FAKE, FAKE, FAKE, 8 * 32768 * 128, 32768 * 128, st, 8 * 32768 * 4, 32768 * 4, sst, FAKE,
        2, Hq, Hkv, D, 32768, 400, ctypes.c_float(0.088), FAKE, FAKE, wsb, None, None)
    assert call(32, 6, 128, 128, 4, ws) == EINVAL           # Hq % Hkv
    assert call(32, 8, 96, 128, 4, ws) == EUNSUPPORTED      # head dim
    assert call(32, 8, 128, 120, 4, ws) == EINVAL           # byte stride not a multiple of 16
    assert call(32, 8, 128, 128, 3, ws) == EINVAL           # fewer than D/32 exponents per row
    assert call(32, 8, 128, 128, 4, 16) == EWORKSPACE
    assert lib.gqa_decode_attn_mxkv(FAKE, None, FAKE, FAKE, FAKE, 0, 0, 128, 0, 0, 4, FAKE, 2, 32, 8, 128,
                                    32768, 400, ctypes.c_float(0.088), FAKE, FAKE, ws, None, None) == EINVAL


def test_attention_paged_argument_checks():
    lib = _lib.load()
    ws = lib.gqa_decode_attn_workspace_size(2, 32, 128, 4096)
    bf = lambda P, npg, bts, mp, wsb=ws, bt=FAKE, st=128: lib.gqa_decode_attn_paged(
        FAKE, FAKE, FAKE, 8 * P * 128, P * 128, st, npg, P, bt, bts, mp, FAKE, 2, 32, 8, 128, 4096,
        ctypes.c_float(0.088), FAKE, FAKE, wsb, None, None)
    assert bf(8, 100, 256, 256) == EUNSUPPORTED             # page below 16 positions
    assert bf(48, 100, 256, 256) == EUNSUPPORTED            # not a power of two
    assert bf(16, 0, 256, 256) == EINVAL                    # empty pool
    assert bf(16, 100, 255, 256) == EINVAL                  # table row shorter than max pages
    assert bf(16, 100, 256, 0) == EINVAL
    assert bf(16, 100, 256, 256, bt=None) == EINVAL         # no block table
    assert bf(16, 100, 256, 256, st=132) == EINVAL          # slot stride not a multiple of 8
    assert bf(16, 100, 256, 256, wsb=16) == EWORKSPACE
    mx = lambda P, sst: lib.gqa_decode_attn_paged_mxkv(
        FAKE, FAKE, FAKE, FAKE, FAKE, 8 * P * 128, P * 128, 128, 8 * P * 4, P * 4, sst, 100, P, FAKE, 256, 256,
        FAKE, 2, 32, 8, 128, 4096, ctypes.c_float(0.088), FAKE, FAKE, ws, None, None)
    assert mx(24, 4) == EUNSUPPORTED
    assert mx(16, 3) == EINVAL                              # fewer than D/32 exponents per row


def test_gemm_mx_argument_checks():
    lib = _lib.load()
    g = lambda M, N, K, lda=4096, ldc=4096, a=FAKE: lib.fp8_gemm_mx(a, lda, FAKE, 1, M, FAKE, 4096, FAKE, 1, N, M, N,
                                                                    K, FAKE, ldc, None)
    assert g(256, 4000, 4096) == EUNSUPPORTED               # N % 128
    assert g(256, 4096, 4000, lda=4000) == EUNSUPPORTED     # K % 128
    assert g(256, 4096, 4096, lda=4100) == EINVAL           # lda % 16
    assert g(256, 4096, 4096, ldc=4000) == EINVAL           # ldc < N
    assert g(256, 4096, 4096, a=None) == EINVAL
    assert lib.fp8_mx_packed_bytes(200, 384) == 256 * 384 + 256 * 12
    assert lib.fp8_mx_packed_bytes(200, 100) == 0
    assert lib.fp8_pack_mx(FAKE, 384, FAKE, 1, 200, 200, 384, FAKE, 16, None) == EWORKSPACE
    assert lib.fp8_pack_mx(FAKE, 380, FAKE, 1, 200, 200, 384, FAKE, 1 << 20, None) == EINVAL
    assert lib.fp8_gemm_mx_packed(FAKE, FAKE, 256, 4000, 4096, FAKE, 4096, None) == EUNSUPPORTED
    assert lib.fp8_gemm_mx_packed(None, FAKE, 256, 4096, 4096, FAKE, 4096, None) == EINVAL


def test_sampling_and_window_argument_checks():
    lib = _lib.load()
    f = ctypes.c_float
    smp = lambda V, ld, T, k, p, lg=FAKE: lib.sample_top_k_top_p(lg, 4, V, ld, f(T), k, f(p), FAKE, FAKE, 1, None)
    assert smp(8193, 8193, 0.8, 30, 0.8) == EUNSUPPORTED    # above the largest vocabulary
    assert smp(4096, 4000, 0.8, 30, 0.8) == EINVAL          # row stride below V
    assert smp(4096, 4096, 0.0, 30, 0.8) == EINVAL          # temperature
    assert smp(4096, 4096, float("inf"), 30, 0.8) == EINVAL
    assert smp(4096, 4096, 0.8, 30, 0.0) == EINVAL          # top_p
    assert smp(4096, 4096, 0.8, 30, 1.5) == EINVAL
    assert smp(4096, 4096, 0.8, 30, 0.8, lg=None) == EINVAL
    assert lib.prev_tokens_shift_inplace(None, FAKE, 2, 4, 10, None) == EINVAL
    assert lib.prev_tokens_shift_inplace(FAKE, FAKE, 2, 0, 10, None) == EINVAL
    assert lib.prev_tokens_shift_inplace(FAKE, FAKE, 0, 4, 10, None) == EINVAL


@pytest.mark.parametrize("M,H,I", [(1, 2560, 9728), (128, 2560, 9728), (1, 256, 1024)])
def test_mlp_workspace_is_small(M, H, I):
    n = _lib.load().swiglu_mlp_fp8_workspace_size(M, H, I, 0)
    assert 0 < n < 32 * 2 ** 20


def test_qlinear_argument_checks():
    lib = _lib.load()
    ws = lib.qlinear_fp8_workspace_size(64, 6144, 2560)
    assert ws > 0
    assert lib.qlinear_fp8_workspace_size(129, 6144, 2560) == 0
    assert lib.qlinear_fp8_workspace_size(64, 6100, 2560) == 0
    assert lib.qlinear_fp8_workspace_size(64, 6144, 2500) == 0
    w = _lib.QWeightC(FAKE, 2560, FAKE, 20, 1)
    call = lambda M, K, N, out, wsb, res=None, norm=None, ldx=2560: lib.qlinear_fp8(
        FAKE, M, K, ldx, norm, ctypes.c_float(1e-6), w, N, res, N, out, FAKE, N, FAKE, wsb, None)
    assert call(0, 2560, 6144, 0, ws) == EINVAL
    assert call(129, 2560, 6144, 0, ws) == EUNSUPPORTED
    assert call(64, 2500, 6144, 0, ws) == EINVAL              # K % 128
    assert call(64, 2560, 6100, 0, ws) == EINVAL              # N % 32
    assert call(64, 2560, 6144, 2, ws) == EINVAL              # out dtype
    assert call(64, 2560, 6144, 1, ws, res=FAKE) == EINVAL    # residual needs bf16 output
    assert call(64, 2560, 6144, 0, ws, norm=FAKE + 2) == EINVAL
    assert call(64, 2560, 6144, 0, ws, ldx=2564) == EINVAL    # ld_x % 8
    assert call(64, 2560, 6144, 0, ws - 1) == EWORKSPACE


def test_qkv_append_argument_checks():
    lib = _lib.load()
    w = _lib.QWeightC(FAKE, 2560, FAKE, 20, 1)
    ws = lib.qlinear_fp8_workspace_size(64, 6144, 2560)
    call = lambda Hq, Hkv, D, kvl=FAKE, cap=32768: lib.qkv_proj_kv_append(
        FAKE, 64, 2560, 2560, None, ctypes.c_float(1e-6), w, Hq, Hkv, D, FAKE, FAKE, FAKE,
        8 * 32768 * 128, 32768 * 128, 128, kvl, cap, FAKE, ws, None, None)
    assert call(32, 6, 128) == EINVAL                         # Hq % Hkv
    assert call(32, 8, 96) == EUNSUPPORTED                    # head dim
    assert call(32, 8, 128, kvl=None) == EINVAL
    assert call(32, 8, 128, cap=0) == EINVAL
    assert call(64, 16, 128) == EWORKSPACE                    # N = 12288 needs a larger workspace


def test_embed_and_argmax_argument_checks():
    lib = _lib.load()
    tabs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert lib.embed_sum_bf16(tabs, 0, 4096, 2560, FAKE, 10, 64, None, FAKE, None, None) == EUNSUPPORTED
    assert lib.embed_sum_bf16(tabs, 17, 4096, 2560, FAKE, 17, 64, None, FAKE, None, None) == EUNSUPPORTED
    assert lib.embed_sum_bf16(tabs, 2, 4096, 2564, FAKE, 10, 64, None, FAKE, None, None) == EINVAL
    assert lib.embed_sum_bf16(tabs, 2, 4096, 2560, FAKE, 1, 64, None, FAKE, None, None) == EINVAL
    assert lib.embed_sum_bf16(tabs, 2, 4096, 2560, None, 10, 64, None, FAKE, None, None) == EINVAL
    assert lib.argmax_rows_f32(FAKE, 64, 4096, 4000, FAKE, 10, None) == EINVAL
    assert lib.argmax_rows_f32(None, 64, 4096, 4096, FAKE, 10, None) == EINVAL


def _model(**kw):
    f = dict(hidden=2560, inter=9728, codebook_size=4096, n_heads=32, n_kv_heads=8, head_dim=128,
             n_codebooks=10, n_slow_layers=2, n_fast_layers=1, rms_eps=1e-6)
    f.update(kw)
    blk = _lib.BlockWeightsC(_qw(), _qw(), _qw(), _qw(), _qw(), FAKE, FAKE)
    slow = (_lib.BlockWeightsC * 2)(blk, blk)
    fast = (_lib.BlockWeightsC * 1)(blk)
    emb = (ctypes.c_void_p * 16)(*([FAKE] * 16))
    heads = (_lib.QWeightC * 16)(*([_qw()] * 16))
    m = _lib.DualArModelC(f["hidden"], f["inter"], f["codebook_size"], f["n_heads"], f["n_kv_heads"],
                          f["head_dim"], f["n_codebooks"], f["n_slow_layers"], f["n_fast_layers"],
                          f["rms_eps"], slow, fast, FAKE, FAKE, emb, heads)
    m._keep = (slow, fast, emb, heads)
    return m


def test_dual_ar_step_argument_checks():
    lib = _lib.load()
    m = _model()
    ws = lib.dual_ar_decode_step_workspace_size(ctypes.byref(m), 64, 4096)
    assert ws > 0
    assert lib.dual_ar_decode_step_workspace_size(ctypes.byref(m), 129, 4096) == 0
    for bad in (dict(n_codebooks=1), dict(n_codebooks=17), dict(head_dim=96), dict(codebook_size=4004),
                dict(n_kv_heads=6), dict(hidden=2500)):
        assert lib.dual_ar_decode_step_workspace_size(ctypes.byref(_model(**bad)), 64, 4096) == 0, bad
    caches = (ctypes.c_void_p * 2)(FAKE, FAKE)
    kv = _lib.KvStateC(caches, caches, 8 * 32768 * 128, 32768 * 128, 128, 32768, FAKE, 4096)
    call = lambda mm, B, wsb, prev=FAKE: lib.dual_ar_decode_step(
        ctypes.byref(mm), B, prev, ctypes.byref(kv), FAKE, None, None, None, FAKE, wsb, None, None)
    assert call(m, 0, ws) == EUNSUPPORTED
    assert call(m, 64, ws, prev=None) == EINVAL
    assert call(_model(n_codebooks=1), 64, ws) == EUNSUPPORTED
    assert call(m, 64, ws - 1) == EWORKSPACE
    assert "workspace" in lib.fp8s_last_error().decode()
