"""FP8 e4m3 codec and the two block-scaling rules, in float64 NumPy.

Test infrastructure only (see the package header).

What is computed, and where it comes from:

* e4m3 -- the "FP8" of both quantisation schemes on the page "How We Made Our
  Text-to-Speech API Free" (section "FP8 Quantization Strategy").  The page
  names the OCP standard for the MX path; we read both paths as the OCP E4M3
  encoding (bias 7, no infinities, 0x7F/0xFF are NaN, largest finite 448,
  subnormals m * 2^-9).  Rounding is round-to-nearest-even and values beyond
  448 saturate to 448 (the OCP "satfinite" conversion and the clamp rule of the
  OCP MX specification).  The sign is kept, so a negative value that rounds to
  zero encodes as 0x80.

* bsgemm block scaling ("128x128 block-scaled FP8" for weights, 1x128 groups
  for activations: same page, "FP8 Quantization Strategy" and "What's Open
  Source").  The page gives no formula; we take the plainest one: per group,
  amax = max |x|, the fp32 dequantisation scale s = amax / 448 (fp32, correctly
  rounded), s = 1 when amax = 0, and q = e4m3(x / s) with the division done in
  fp32, correctly rounded.  x ~= q * s.

* MX 1x32 with OCP UE8M0 shared exponents (same page, "FP8 Quantization
  Strategy").  OCP MX rule: per group of 32 along K, the shared exponent is
  floor(log2 amax) - 8 (8 = largest exponent of E4M3), stored biased by 127 as
  an unsigned byte, clamped to [0, 254]; amax = 0 stores 0.  q = e4m3(x / X)
  with X = 2^(E - 127); this division is exact.

Pins (tests/test_oracle_fp8.py): the decoder against torch's float8_e4m3fn
view-cast for all 256 codes; the encoder against a brute-force nearest-code
search over every finite bf16 pattern and a dense fp32 boundary set, and against
torch's cast where that cast is defined (|v| <= 448); OCP table values in
tests/golden; scale round-trip of exactly representable blocks; the UE8M0
closed form.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3_MAX = 448.0
_CHUNK = 1 << 20            # elementwise work is done in chunks of this size


def _chunked(fn, v, out_dtype):
    """Apply the elementwise function fn to v in chunks (on a few threads).

    Purely a traversal order: every element is computed by the same fn as an
    unchunked call would, so the result is identical; it only keeps the
    float64 temporaries of large tensors in cache."""
    flat = np.ascontiguousarray(v).reshape(-1)
    if flat.size <= _CHUNK:
        return fn(flat).reshape(np.shape(v))
    out = np.empty(flat.size, dtype=out_dtype)
    starts = range(0, flat.size, _CHUNK)

    def run(i):
        out[i:i + _CHUNK] = fn(flat[i:i + _CHUNK])
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(run, starts))
    return out.reshape(np.shape(v))
_MIN_NORMAL_EXP = -6        # smallest normal exponent of E4M3
_MANT_BITS = 3


def e4m3_encode(v):
    """Encode finite values (float64 holding the exact input) as e4m3 bytes.

    NaN encodes as 0x7F with its sign bit; infinities are rejected.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isinf(v).any():
        raise ValueError("e4m3_encode: infinities are not accepted")
    return _chunked(_encode, v, np.uint8)


def _encode(v):
    sign = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)

    # Exponent of |v|, floored at the subnormal exponent; quantum of that binade.
    _, e = np.frexp(a)                         # a = f * 2^e, f in [0.5, 1)
    e = np.maximum(e - 1, _MIN_NORMAL_EXP)     # floor(log2 a), or -6
    quantum = np.ldexp(1.0, e - _MANT_BITS)
    n = np.rint(a / quantum)                   # exact scaling, round half to even
    val = np.minimum(n * quantum, E4M3_MAX)    # saturate

    # Bit pattern of the (representable) magnitude val.
    sub = val < np.ldexp(1.0, _MIN_NORMAL_EXP)
    code_sub = np.rint(val / np.ldexp(1.0, _MIN_NORMAL_EXP - _MANT_BITS))
    _, ev = np.frexp(np.where(sub, 1.0, val))
    ev = ev - 1
    mant = np.rint((np.where(sub, 1.0, val) / np.ldexp(1.0, ev) - 1.0) * 8.0)
    code_norm = (ev + 7) * 8 + mant
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(b):
    """Decode e4m3 bytes to float64 (exact).  0x7F/0xFF decode to NaN."""
    return _chunked(_decode, np.asarray(b, dtype=np.uint8), np.float64)


def _decode(b):
    b = b.astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    ef = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(ef == 0,
                   m * 2.0 ** -9,
                   (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    mag = np.where((ef == 15) & (m == 7), np.nan, mag)
    return s * mag


def _blocks(x, gr, gc):
    """View a [R, C] array as [R/gr, gr, C/gc, gc]."""
    r, c = x.shape
    if r % gr or c % gc:
        raise ValueError(f"shape {x.shape} is not a multiple of the {gr}x{gc} group")
    return x.reshape(r // gr, gr, c // gc, gc)


def quant_block_fp32(x, gr, gc):
    """bsgemm quantisation of x (fp32 values) in gr x gc groups.

    Returns (q uint8 [R, C], s float32 [R/gr, C/gc]) with x ~= q * s.
    """
    x = np.asarray(x, dtype=np.float32)
    xb = _blocks(x, gr, gc)
    amax = np.abs(xb).max(axis=(1, 3)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    # fp32 division, correctly rounded (NumPy float32 arithmetic is IEEE single).
    scaled = (xb / s[:, None, :, None]).astype(np.float32)
    q = e4m3_encode(scaled.astype(np.float64)).reshape(x.shape)
    return q, s


def quant_act_1x128(x):
    """Activation quantisation, 1x128 groups along K: s is [M, K/128]."""
    return quant_block_fp32(x, 1, 128)


def quant_weight_128x128(w):
    """Weight quantisation, 128x128 blocks: s is [N/128, K/128]."""
    return quant_block_fp32(w, 128, 128)


def dequant_block_fp32(q, s, gr, gc):
    """Exact float64 value of a bsgemm-quantised tensor."""
    v = e4m3_decode(q)
    vb = _blocks(v, gr, gc)
    return (vb * np.asarray(s, np.float64)[:, None, :, None]).reshape(v.shape)


def ue8m0_exponent(amax):
    """OCP MX shared exponent (biased UE8M0 byte) for E4M3 elements."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    e = e - 1                                   # floor(log2 amax)
    biased = np.clip(e - 8 + 127, 0, 254)
    return np.where(amax > 0, biased, 0).astype(np.uint8)


def quant_mx_1x32(x):
    """MX quantisation in 1x32 groups along K.

    Returns (q uint8 [R, C], E uint8 [R, C/32]); logical layout, row-major.
    x ~= q * 2^(E - 127).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    xb = _blocks(x, 1, 32)
    amax = np.abs(xb).max(axis=(1, 3))
    E = ue8m0_exponent(amax)
    X = np.ldexp(1.0, E.astype(np.int64) - 127)
    q = e4m3_encode(xb / X[:, None, :, None]).reshape(x.shape)
    return q, E


def dequant_mx_1x32(q, E):
    """Exact float64 value of an MX-quantised tensor (E is [R, C/32])."""
    v = e4m3_decode(q)
    vb = _blocks(v, 1, 32)
    X = np.ldexp(1.0, np.asarray(E).astype(np.int64) - 127)
    return (vb * X[:, None, :, None]).reshape(v.shape)
