"""Pins of the oracle's e4m3 codec and scaling rules against things other than
itself: torch's float8_e4m3fn, a brute-force nearest-code search, the OCP
table values in tests/golden, and closed forms of the scale rules."""

import os

import numpy as np
import pytest
import torch

from oracle import fp8
from fp8_transformer_step_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _brute_force_encode(v):
    """Nearest of the 127 finite non-negative codes by exhaustive search.

    Ties go to the code with an even mantissa (even code); magnitudes above
    448 saturate to 448; the sign bit is copied.
    """
    v = np.asarray(v, np.float64)
    table = _torch_decode_all()[:127]            # 0x00..0x7E, increasing
    a = np.abs(v)[:, None]
    d = np.abs(a - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even code
    even = (np.arange(127) % 2 == 0)[None, :]
    pick_even = (cand & even).any(axis=1)
    code = np.where(pick_even, np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    code = np.where(np.abs(v) > 448.0, 0x7E, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def test_decode_all_codes_matches_torch():
    ref = _torch_decode_all()
    got = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_golden_ocp_table():
    rows = []
    with open(os.path.join(GOLDEN, "ocp_e4m3_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code = line.split()[:2]
            rows.append((float(val), int(code, 16)))
    vals = np.array([r[0] for r in rows])
    codes = np.array([r[1] for r in rows], np.uint8)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)
    dec = fp8.e4m3_decode(codes)
    for v, d in zip(vals, dec):
        if np.isnan(v):
            assert np.isnan(d)
        else:
            assert v == d and np.signbit(v) == np.signbit(d)


def test_encode_every_bf16_pattern_bruteforce():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = inputs.bf16_bits_to_f32(bits).astype(np.float64)
    finite = np.isfinite(vals)
    v = vals[finite]
    got = fp8.e4m3_encode(v)
    ref = np.concatenate([_brute_force_encode(c) for c in np.array_split(v, 16)])
    assert np.array_equal(got, ref)


def test_encode_fp32_boundaries_bruteforce():
    table = _torch_decode_all()[:127]
    mids = (table[:-1] + table[1:]) / 2.0
    pts = np.concatenate([table, mids, [456.0, 460.0, 463.9, 464.0, 464.1, 480.0, 1e6]])
    pts32 = pts.astype(np.float32)
    nbr = np.concatenate([pts32,
                          np.nextafter(pts32, np.float32(np.inf)),
                          np.nextafter(pts32, np.float32(0))])
    nbr = np.concatenate([nbr, -nbr]).astype(np.float64)
    assert np.array_equal(fp8.e4m3_encode(nbr), _brute_force_encode(nbr))


def test_encode_matches_torch_cast_in_range():
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.uniform(-448, 448, 20000),
        g.standard_normal(20000) * 2.0 ** g.integers(-14, 8, 20000),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(v.astype(np.float64)), ref)


def test_bsgemm_scale_round_trip_of_representable_blocks():
    """A block of e4m3 values times 2^k whose amax is 448 * 2^k has s = 2^k
    exactly and dequant(quant(x)) == x."""
    g = np.random.default_rng(11)
    table = _torch_decode_all()[:127]
    for gr, gc in ((1, 128), (128, 128)):
        R, C = (4 * gr, 3 * gc)
        x = np.empty((R, C), np.float64)
        ks = g.integers(-20, 20, size=(R // gr, C // gc))
        for bi in range(R // gr):
            for bj in range(C // gc):
                blk = table[g.integers(0, 127, size=(gr, gc))] * np.where(
                    g.random((gr, gc)) < 0.5, -1.0, 1.0)
                blk[g.integers(gr), g.integers(gc)] = 448.0
                x[bi * gr:(bi + 1) * gr, bj * gc:(bj + 1) * gc] = blk * 2.0 ** ks[bi, bj]
        q, s = fp8.quant_block_fp32(x.astype(np.float32), gr, gc)
        assert np.array_equal(s.astype(np.float64), 2.0 ** ks)
        assert np.array_equal(fp8.dequant_block_fp32(q, s, gr, gc), x)


def test_bsgemm_zero_block_scale_is_one():
    q, s = fp8.quant_act_1x128(np.zeros((2, 256), np.float32))
    assert np.all(s == 1.0) and np.all(q == 0)


def test_bsgemm_scale_is_fp32_amax_over_448():
    g = np.random.default_rng(3)
    x = (g.standard_normal((5, 256)) * 3).astype(np.float32)
    _, s = fp8.quant_act_1x128(x)
    amax = np.abs(x.reshape(5, 2, 128)).max(axis=2).astype(np.float64)
    # fp32 correctly rounded quotient: the exact quotient rounded once
    assert np.array_equal(s, (amax / 448.0).astype(np.float32))


def test_ue8m0_closed_form_and_saturation():
    for j in range(-100, 120, 7):
        for mant in (1.0, 1.5, 1.75, 1.999):
            amax = mant * 2.0 ** j
            E = int(fp8.ue8m0_exponent(np.array([amax]))[0])
            assert E == j + 119
            x = np.zeros((1, 32), np.float32)
            x[0, 5] = amax
            x[0, 9] = -amax / 4
            q, e = fp8.quant_mx_1x32(x)
            assert int(e[0, 0]) == j + 119
            top = int(q[0, 5])
            if mant > 1.75:
                assert top == 0x7E          # block max saturates to 448
            else:
                assert fp8.dequant_mx_1x32(q, e)[0, 5] == np.float32(amax)


def test_mx_round_trip_of_representable_blocks():
    g = np.random.default_rng(5)
    table = _torch_decode_all()[:127]
    R, C = 6, 256
    x = np.empty((R, C))
    ks = g.integers(-30, 30, size=(R, C // 32))
    for r in range(R):
        for b in range(C // 32):
            blk = table[g.integers(0, 127, 32)] * np.where(g.random(32) < 0.5, -1, 1)
            blk[g.integers(32)] = table[g.integers(120, 127)]   # amax in [256, 448]
            x[r, b * 32:(b + 1) * 32] = blk * 2.0 ** ks[r, b]
    q, e = fp8.quant_mx_1x32(x.astype(np.float32))
    assert np.array_equal(e.astype(np.int64) - 127, ks)
    assert np.array_equal(fp8.dequant_mx_1x32(q, e), x)


def test_mx_zero_block():
    q, e = fp8.quant_mx_1x32(np.zeros((1, 64), np.float32))
    assert np.all(e == 0) and np.all(q == 0)


def test_negative_underflow_keeps_sign():
    q, _ = fp8.quant_act_1x128(np.array([[448.0] + [-1e-6] * 127], np.float32))
    assert q[0, 1] == 0x80


@pytest.mark.parametrize("gr,gc", [(1, 100), (96, 128)])
def test_group_must_divide_shape(gr, gc):
    with pytest.raises(ValueError):
        fp8.quant_block_fp32(np.zeros((128, 256), np.float32), gr, gc)
