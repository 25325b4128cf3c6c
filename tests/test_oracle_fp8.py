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


# ---- exact-arithmetic pins of the bsgemm division and the UE8M0 lower clamp ----
# These rebuild each rounding step with fractions.Fraction (exact rationals),
# so they do not rely on NumPy's float32 arithmetic.

from fractions import Fraction  # noqa: E402


def _round_binary(q, mant_bits, min_exp):
    """Round the exact rational q to the nearest value with mant_bits stored
    mantissa bits and exponent >= min_exp (subnormals below), ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                  # now 2^e <= a < 2^(e+1)
    e = max(e, min_exp)
    quantum = Fraction(2) ** (e - mant_bits)
    n, r = divmod(a, quantum)
    n = int(n)
    if r * 2 > quantum or (r * 2 == quantum and n % 2 == 1):
        n += 1
    return sign * n * quantum


def _fp32(q):
    return _round_binary(q, 23, -126)


def _e4m3(q):
    v = _round_binary(q, 3, -6)
    return max(min(v, Fraction(448)), Fraction(-448))


# (amax, x): bf16 values for which e4m3(fp32(x / s)), s = fp32(amax / 448),
# differs from both e4m3 of the exact quotient and e4m3(fp32(x * fp32(1 / s))).
# Found by a search over bf16 pairs; each is checked below with exact rationals.
_DIV_CASES = [(1.078125, 0.10107421875), (1.59375, 0.07470703125), (1.625, 0.3046875),
              (1.296875, 0.97265625)]


def _division_readings(amax, x):
    s = _fp32(Fraction(amax) / 448)
    fp32_div = _e4m3(_fp32(Fraction(x) / s))
    exact = _e4m3(Fraction(x) / s)
    recip = _e4m3(_fp32(Fraction(x) * _fp32(1 / s)))
    return s, fp32_div, exact, recip


def test_bsgemm_division_is_fp32_correctly_rounded():
    """The bsgemm rule divides in fp32 (correctly rounded) before the e4m3
    rounding.  Each case is built so that the exact quotient lies just above
    an e4m3 rounding midpoint and its fp32 rounding lands on it (a tie that
    goes to the even code), so dividing exactly, in fp64, or multiplying by
    an fp32 reciprocal each give a different code: all three readings are
    computed here in exact arithmetic and the oracle must give the first."""
    for amax, x in _DIV_CASES:
        s, want, exact, recip = _division_readings(amax, x)
        assert want != exact and want != recip, "the case does not tell the readings apart"
        for shape, fn, slot in (((1, 128), fp8.quant_act_1x128, (0, 77)),
                                ((128, 128), fp8.quant_weight_128x128, (93, 5))):
            blk = np.zeros(shape, np.float32)
            blk[0, 0] = amax
            blk[slot] = x
            blk[slot[0], (slot[1] + 1) % 128] = -x
            q, sc = fn(blk)
            assert Fraction(float(sc.reshape(-1)[0])) == s
            got = Fraction(float(fp8.e4m3_decode(q[slot])))
            assert got == want
            assert Fraction(float(fp8.e4m3_decode(q[slot[0], (slot[1] + 1) % 128]))) == -want
            assert Fraction(float(fp8.e4m3_decode(q[0, 0]))) == _e4m3(_fp32(Fraction(amax) / s))


def test_bsgemm_division_cases_reach_the_fp64_path():
    """The fp64 quotient also rounds to the exact reading's code here, so an
    oracle that divided in float64 would fail the pin above."""
    for amax, x in _DIV_CASES:
        s, want, exact, _ = _division_readings(amax, x)
        q64 = fp8.e4m3_encode(np.float64(x) / np.float64(float(s)))
        assert Fraction(float(fp8.e4m3_decode(q64))) == exact != want


def test_ue8m0_lower_clamp():
    """Blocks whose largest magnitude lies in [2^-133, 2^-119) (bf16
    subnormals included) have floor(log2 amax) - 8 + 127 < 0: the shared
    exponent clamps to 0, X = 2^-127, and the codes are e4m3(x * 2^127),
    written out here by hand."""
    # (values of one 32-group, expected exponent byte, expected codes)
    cases = [
        ([2.0 ** -120], 0, [0x70]),                          # 2^7 = 128: exp 14, mant 0
        ([2.0 ** -133], 0, [0x08]),                          # 2^-6, smallest normal e4m3
        ([1.5 * 2.0 ** -129, -2.0 ** -128], 0, [0x2C, 0xB0]),  # 0.375, -0.5
        ([1.75 * 2.0 ** -120], 0, [0x76]),                   # 224: exp 14, mant 6
        ([1.0 * 2.0 ** -119], 0, [0x78]),                    # amax = 2^-119 -> E = 0, 256 (exp 15, mant 0)
        ([2.0 ** -118], 1, [0x78]),                          # first exponent above the clamp: 2^-118 / 2^-126
    ]
    for vals, e_want, codes in cases:
        blk = np.zeros((1, 32), np.float32)
        blk[0, :len(vals)] = vals
        q, E = fp8.quant_mx_1x32(blk)
        assert int(E[0, 0]) == e_want
        assert list(q[0, :len(vals)]) == codes
        assert not q[0, len(vals):].any()
    assert int(fp8.ue8m0_exponent(np.float64(2.0 ** -133))) == 0
    assert int(fp8.ue8m0_exponent(np.float64(2.0 ** -119 * 1.99))) == 0
