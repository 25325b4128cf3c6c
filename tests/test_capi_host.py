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


@pytest.mark.parametrize("M,H,I", [(1, 2560, 9728), (128, 2560, 9728), (1, 256, 1024)])
def test_mlp_workspace_is_small(M, H, I):
    n = _lib.load().swiglu_mlp_fp8_workspace_size(M, H, I, 0)
    assert 0 < n < 32 * 2 ** 20
