"""sample_top_k_top_p and prev_tokens_shift_inplace on the GPU against the
oracle.  The sampler decides integers from fp32 masses, the oracle from
float64 ones: a code must equal the oracle's unless u, or the top-p cut,
lies within fp32 rounding of a cumulative-mass boundary, and then it must be
one of the draws on the other side of that boundary.  Cases: the pages' setting
(temperature 0.8, top_p 0.8, top_k 30) on a 64 x 4096 head, top_k = 1
(greedy), equal logits (an exact case), ties at the top-k threshold, NaN
entries and rows, ragged and maximal vocabularies, and the empirical law of
one row over a grid of uniforms.  The window shift is bit-exact."""

import numpy as np
import pytest
import torch

from oracle import sampling as osmp
from _helpers import log, need_gpu
from fp8_transformer_step_amd import ops

pytestmark = pytest.mark.gpu

BOUNDARY = 2e-5                    # relative fp32 slack on a cumulative mass


def _u(seed, B):
    return np.random.default_rng(seed).random(B).astype(np.float32)


def _run(logits, u, T, k, p):
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    out = ops.sample_top_k_top_p(lg, torch.from_numpy(u).cuda(), T, k, p)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _allowed(row, T, k, p, u):
    """Indices a correct fp32 evaluation may return: the exact draw, and
    where the top-p cut or u lies within BOUNDARY of a cumulative mass, the
    draws on the other side of that boundary."""
    row = np.asarray(row, np.float64)
    order = osmp.rank_order(row)
    n_valid = int(np.count_nonzero(~np.isnan(row)))
    kk = min(len(row) if k <= 0 else k, n_valid)
    z = row[order[:kk]] / T
    c = np.cumsum(np.exp(z - z[0]))
    tot = c[-1]
    cuts = [n for n in range(1, kk + 1)
            if c[n - 1] >= p * tot * (1 - BOUNDARY) and (n == 1 or c[n - 2] < p * tot * (1 + BOUNDARY))]
    out = set()
    for n in cuts:
        cdf = c[:n] / c[n - 1]
        r = min(int(np.searchsorted(cdf, u, side="right")), n - 1)
        out.add(int(order[r]))
        if r + 1 < n and abs(cdf[r] - u) <= BOUNDARY:
            out.add(int(order[r + 1]))
        if r > 0 and abs(cdf[r - 1] - u) <= BOUNDARY:
            out.add(int(order[r - 1]))
    return out


def _check(logits, u, T, k, p, got):
    """Every code is the oracle's or one of the draws across a boundary
    within fp32 rounding; returns how many rows took such a draw."""
    loose = 0
    for b in range(logits.shape[0]):
        ref = osmp.sample_row(logits[b], T, k, p, float(u[b]))[0]
        if int(got[b]) == ref:
            continue
        assert int(got[b]) in _allowed(logits[b], T, k, p, float(u[b])), (b, int(got[b]), ref, float(u[b]))
        loose += 1
    return loose


def test_pages_setting_on_a_codebook_head():
    need_gpu()
    g = np.random.default_rng(101)
    x = (g.standard_normal((64, 4096)) * 3.0).astype(np.float32)
    u = _u(102, 64)
    got = _run(x, u, 0.8, 30, 0.8)
    loose = _check(x, u, 0.8, 30, 0.8, got)
    log(f"sample 64x4096 T0.8 k30 p0.8: {loose} rows at a boundary")
    assert loose <= 2


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 0.95), (0.5, 200, 1.0), (2.0, 4096, 0.5), (0.8, 7, 0.999)])
def test_other_settings(T, k, p):
    need_gpu()
    g = np.random.default_rng(110 + k)
    x = (g.standard_normal((32, 4096)) * 2.0).astype(np.float32)
    u = _u(111 + k, 32)
    assert _check(x, u, T, k, p, _run(x, u, T, k, p)) <= 2


def test_top_k_one_is_greedy():
    need_gpu()
    g = np.random.default_rng(120)
    x = g.standard_normal((16, 4096)).astype(np.float32)
    x[3, [5, 900]] = 10.0                        # a tie: the lower index
    x[4, :100] = np.nan                          # NaN never chosen
    u = _u(121, 16)
    got = _run(x, u, 0.8, 1, 0.8)
    ref = np.array([np.nanargmax(r) for r in x])
    assert np.array_equal(got, ref)
    assert got[3] == 5


def test_equal_logits_draw_floor_u_times_v():
    need_gpu()
    V = 4096
    x = np.full((V, V), 1.25, np.float32)
    u = ((np.arange(V) + 0.5) / V).astype(np.float32)
    assert np.array_equal(_run(x, u, 0.8, 0, 1.0), np.arange(V))


def test_ties_at_the_top_k_threshold():
    need_gpu()
    g = np.random.default_rng(130)
    x = g.integers(-3, 4, size=(48, 4096)).astype(np.float32)     # many equal values
    u = _u(131, 48)
    got = _run(x, u, 1.0, 30, 1.0)
    assert _check(x, u, 1.0, 30, 1.0, got) <= 2
    # with 30 kept among hundreds of equal maxima, the kept ones are the 30 lowest indices
    for b in range(48):
        top = np.flatnonzero(x[b] == x[b].max())
        assert got[b] in top[:30]


def test_nan_entries_and_nan_rows():
    need_gpu()
    g = np.random.default_rng(140)
    x = g.standard_normal((8, 1000)).astype(np.float32)
    x[:, ::3] = np.nan
    x[5] = np.nan
    u = _u(141, 8)
    got = _run(x, u, 0.8, 0, 1.0)
    assert got[5] == 0
    for b in range(8):
        if b != 5:
            assert not np.isnan(x[b, got[b]])
    keep = [b for b in range(8) if b != 5]
    assert _check(x[keep], u[keep], 0.8, 0, 1.0, got[keep]) <= 1


@pytest.mark.parametrize("V", [1, 37, 255, 257, 8192])
def test_ragged_and_maximal_vocabularies(V):
    need_gpu()
    g = np.random.default_rng(150 + V)
    x = (g.standard_normal((12, V)) * 2.0).astype(np.float32)
    u = _u(151 + V, 12)
    for T, k, p in ((0.8, 30, 0.8), (1.0, 0, 1.0)):
        assert _check(x, u, T, k, p, _run(x, u, T, k, p)) <= 1


def test_empirical_law_of_one_row():
    """4096 draws of one row over a grid of u: the share of every entry is
    its oracle probability to the grid step (boundaries within fp32)."""
    need_gpu()
    N = 4096
    row = (np.random.default_rng(160).standard_normal(4096) * 3.0).astype(np.float32)
    x = np.tile(row, (N, 1))
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    got = _run(x, u, 0.8, 30, 0.8)
    ref = np.array([osmp.sample_row(row.astype(np.float64), 0.8, 30, 0.8, float(v))[0] for v in u])
    assert np.count_nonzero(got != ref) <= 2


def test_window_shift_bit_exact():
    need_gpu()
    g = np.random.default_rng(170)
    for bs, W, cw in ((64, 16, 10), (3, 1, 10), (5, 7, 1), (1000, 4, 9)):
        prev = g.integers(-2**31, 2**31 - 1, size=(bs, W, cw), dtype=np.int64).astype(np.int32)
        nxt = g.integers(0, 4096, size=(bs, cw)).astype(np.int32)
        p = torch.from_numpy(prev).cuda()
        ops.prev_tokens_shift_inplace(p, torch.from_numpy(nxt).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(p.cpu().numpy(), osmp.prev_tokens_shift(prev, nxt)), (bs, W, cw)


def test_window_after_w_shifts_and_contract():
    need_gpu()
    g = np.random.default_rng(171)
    bs, W, cw = 64, 8, 10
    p = torch.from_numpy(g.integers(0, 4096, (bs, W, cw)).astype(np.int32)).cuda()
    frames = [g.integers(0, 4096, (bs, cw)).astype(np.int32) for _ in range(W + 3)]
    for f in frames:
        ops.prev_tokens_shift_inplace(p, torch.from_numpy(f).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), np.stack(frames[-W:], axis=1))
    nxt = torch.zeros((bs, cw), dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        ops.prev_tokens_shift_inplace(p.long(), nxt)
    with pytest.raises(TypeError):
        ops.prev_tokens_shift_inplace(p, nxt.long())
    with pytest.raises(ValueError):
        ops.prev_tokens_shift_inplace(p, nxt.unsqueeze(1))
    with pytest.raises(ValueError):
        ops.prev_tokens_shift_inplace(p[:, :, :5], nxt[:, :5])
