"""Pins of the oracle's top-k / top-p sampling and previous-tokens window
shift: argmax special cases, an exact uniform case, the empirical law over a
fine grid of uniforms against scipy's softmax on an argsort-selected set, a
hand-computed top-p cut, NaN handling, and the window shift."""

import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sampling


def _logits(seed, B, V, scale=3.0):
    return np.random.default_rng(seed).standard_normal((B, V)) * scale


def test_top_k_one_and_tiny_top_p_are_argmax():
    x = _logits(1, 8, 300)
    x[3, [10, 20]] = x[3].max() + 1.0          # a tie: the lower index wins
    for u in (0.0, 0.3, 0.999):
        uu = np.full(8, u)
        assert np.array_equal(sampling.sample_top_k_top_p(x, 0.8, 1, 0.8, uu), np.argmax(x, axis=1))
        assert np.array_equal(sampling.sample_top_k_top_p(x, 0.8, 30, 1e-9, uu), np.argmax(x, axis=1))
    assert sampling.sample_top_k_top_p(x, 0.8, 1, 1.0, np.zeros(8))[3] == 10


def test_equal_logits_draw_floor_u_times_v():
    V = 64
    for j in range(V):
        u = (j + 0.5) / V
        assert sampling.sample_row(np.full(V, 2.5), 0.8, 0, 1.0, u)[0] == j
        assert sampling.sample_row(np.full(V, 2.5), 0.8, 0, 1.0, j / V)[0] == j


@pytest.mark.parametrize("T,k,p", [(0.8, 30, 0.8), (1.0, 0, 1.0), (0.5, 100, 0.95), (2.0, 7, 0.3)])
def test_empirical_law_matches_softmax_of_kept_set(T, k, p):
    """Over u on a grid of N points, the share of each entry is its
    probability under the kept (top-k then top-p) distribution, to 1/N."""
    V, N = 200, 20000
    row = _logits(2, 1, V)[0]
    order = np.argsort(-row, kind="stable")
    kk = V if k <= 0 else k
    probs = softmax(row[order[:kk]] / T)
    cum = np.cumsum(probs)
    n = int(np.argmax(cum >= p * cum[-1] - 1e-15)) + 1 if p < 1 else kk
    law = np.zeros(V)
    law[order[:n]] = probs[:n] / probs[:n].sum()
    counts = np.zeros(V)
    for i in range(N):
        counts[sampling.sample_row(row, T, k, p, (i + 0.5) / N)[0]] += 1
    assert np.abs(counts / N - law).max() <= 1.0 / N + 1e-12
    assert set(np.flatnonzero(counts)) <= set(order[:n])


def test_hand_computed_top_p_cut():
    # probabilities 0.5, 0.3, 0.2 at T = 1 (logits = log p); top_p 0.75 keeps two
    row = np.log([0.2, 0.5, 0.3])
    idx, n, cdf = sampling.sample_row(row, 1.0, 0, 0.75, 0.0)
    assert n == 2 and idx == 1
    assert np.allclose(cdf, [0.625, 1.0], rtol=1e-15)
    assert sampling.sample_row(row, 1.0, 0, 0.75, 0.6249)[0] == 1
    assert sampling.sample_row(row, 1.0, 0, 0.75, 0.6251)[0] == 2
    # top_p 0.81 needs the third entry; temperature 0.5 squares and renormalises
    assert sampling.sample_row(row, 1.0, 0, 0.81, 0.0)[1] == 3
    sq = np.array([0.25, 0.09, 0.04]) / 0.38
    assert np.allclose(sampling.sample_row(row, 0.5, 0, 1.0, 0.0)[2], np.cumsum(sq), rtol=1e-14)


def test_nan_never_drawn():
    row = np.array([np.nan, 1.0, np.nan, 1.0 + math.log(3.0), np.nan])
    picks = {sampling.sample_row(row, 1.0, 0, 1.0, u)[0] for u in np.linspace(0, 0.999, 101)}
    assert picks == {1, 3}
    assert sampling.sample_row(row, 1.0, 0, 1.0, 0.74)[0] == 3   # p = 3/4 for index 3
    assert sampling.sample_row(row, 1.0, 0, 1.0, 0.76)[0] == 1


def test_parameter_checks():
    row = np.zeros(4)
    for T, p, u in ((0.0, 0.5, 0.1), (1.0, 0.0, 0.1), (1.0, 1.1, 0.1), (1.0, 0.5, 1.0)):
        with pytest.raises(ValueError):
            sampling.sample_row(row, T, 0, p, u)


def test_window_shift_example():
    prev = np.arange(2 * 3 * 4, dtype=np.int32).reshape(2, 3, 4)
    nxt = np.array([[100, 101, 102, 103], [200, 201, 202, 203]], np.int32)
    out = sampling.prev_tokens_shift(prev, nxt)
    assert out.tolist() == [[[4, 5, 6, 7], [8, 9, 10, 11], [100, 101, 102, 103]],
                            [[16, 17, 18, 19], [20, 21, 22, 23], [200, 201, 202, 203]]]
    assert prev[0, 0, 0] == 0                  # the input is untouched


def test_window_after_w_shifts_holds_the_w_newest_frames():
    g = np.random.default_rng(3)
    bs, W, cw = 3, 5, 10
    win = g.integers(0, 4096, (bs, W, cw)).astype(np.int32)
    frames = [g.integers(0, 4096, (bs, cw)).astype(np.int32) for _ in range(W + 2)]
    for f in frames:
        win = sampling.prev_tokens_shift(win, f)
    assert np.array_equal(win, np.stack(frames[-W:], axis=1))


def test_window_shift_contract():
    prev = np.zeros((2, 3, 4), np.int32)
    with pytest.raises(TypeError):
        sampling.prev_tokens_shift(prev.astype(np.int64), np.zeros((2, 4), np.int32))
    with pytest.raises(ValueError):
        sampling.prev_tokens_shift(prev, np.zeros((2, 1, 4), np.int32))
    with pytest.raises(ValueError):
        sampling.prev_tokens_shift(prev, np.zeros((4, 2), np.int32))
