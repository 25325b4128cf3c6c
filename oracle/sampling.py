"""Seeded top-k / top-p sampling of a codebook head, and the sliding window
of previous tokens of the Dual-AR decoder.

Test infrastructure only (see the package header).

Sources, by page title and section:
  * "Fish Speech KV Cache 推理优化记录" (Fish Speech KV-cache optimisation
    notes), section 6 (benchmark conditions): generation samples with
    temperature 0.8, top_p 0.8, top_k 30 and a fixed seed; section 7: the
    generation regression uses top_k = 1 (deterministic) and checks tokens.
  * "How We Made Our Text-to-Speech API Free: The Inference Engineering
    Behind S2.1 Pro" (and its Chinese original), section "Continuous
    Batching for Autoregressive TTS", part "DualAR: S2-Specific Batching
    Constraints": a sliding window of previous tokens conditions every step;
    its in-place shift takes prev int32 [bs, W, cw] and next_tokens int32
    [bs, cw] under a strict shape and dtype contract.

Readings where the pages are silent:
  * Sampling order: logits / temperature, then top-k, then top-p over the
    softmax of the surviving logits, then one draw.  Entries are ranked by
    (logit descending, index ascending), so ties are decided by the lower
    index and the kept sets are unique.  NaN logits rank last and are never
    drawn.  top-p keeps the shortest ranked prefix whose probability mass is
    at least top_p times the top-k mass (never fewer than one entry).  The
    draw takes a uniform u in [0, 1) from the caller (random numbers are
    inputs) and returns the first ranked entry whose cumulative mass exceeds
    u times the kept mass (inverse CDF in ranked order).
  * The window shift: frame w + 1 moves to frame w for w < W - 1, and the
    new tokens become frame W - 1 (the newest); frame 0 (the oldest) drops.

Pins (tests/test_oracle_sampling.py): top_k = 1 and a vanishing top_p give
numpy's argmax for every u; equal logits give floor(u * V) exactly; the
fraction of a fine grid of u that lands on each entry matches scipy's
softmax over the kept set (itself found with numpy's argsort) to the grid
step; a hand-computed three-entry top-p example; NaN never drawn; the window
shift against a hand-written example and W successive shifts leaving exactly
the W newest frames.
"""

import numpy as np


def rank_order(row):
    """Indices of a logit row ranked by (value descending, index ascending),
    NaN entries last (in index order)."""
    row = np.asarray(row, np.float64)
    nan = np.isnan(row)
    key = np.where(nan, 0.0, -row)
    return np.lexsort((np.arange(row.size), key, nan))


def sample_row(row, temperature, top_k, top_p, u):
    """One draw from a logit row.  Returns (index, kept count after top-p,
    cumulative masses of the ranked kept prefix, normalised to 1)."""
    row = np.asarray(row, np.float64)
    V = row.size
    if not temperature > 0:
        raise ValueError("temperature must be positive")
    if not 0 < top_p <= 1:
        raise ValueError("top_p must lie in (0, 1]")
    if not 0 <= u < 1:
        raise ValueError("u must lie in [0, 1)")
    k = V if top_k <= 0 else min(int(top_k), V)
    order = rank_order(row)
    n_valid = int(np.count_nonzero(~np.isnan(row)))
    k = max(1, min(k, n_valid)) if n_valid else 1
    kept = order[:k]
    if n_valid == 0:
        return int(kept[0]), 1, np.ones(1)
    z = row[kept] / temperature
    p = np.exp(z - z[0])                       # z[0] is the largest
    c = np.cumsum(p)
    n = int(np.searchsorted(c, top_p * c[-1], side="left")) + 1    # shortest prefix with mass >= top_p
    n = min(max(n, 1), k)
    cdf = c[:n] / c[n - 1]
    i = int(np.searchsorted(cdf, u, side="right"))                  # first with cdf > u
    return int(kept[min(i, n - 1)]), n, cdf


def sample_top_k_top_p(logits, temperature, top_k, top_p, u):
    """Codes int32 [B] drawn from logits [B, V] with uniforms u [B]."""
    logits = np.asarray(logits)
    return np.array([sample_row(logits[b], temperature, top_k, top_p, float(u[b]))[0]
                     for b in range(logits.shape[0])], np.int32)


def prev_tokens_shift(prev, next_tokens):
    """The window after one step: prev int32 [bs, W, cw], next_tokens int32
    [bs, cw]; returns a new array (the input is not modified)."""
    prev = np.asarray(prev)
    nt = np.asarray(next_tokens)
    if prev.dtype != np.int32 or nt.dtype != np.int32:
        raise TypeError("prev and next_tokens must be int32")
    if prev.ndim != 3 or nt.shape != (prev.shape[0], prev.shape[2]):
        raise ValueError("shapes must be prev [bs, W, cw] and next_tokens [bs, cw]")
    out = np.empty_like(prev)
    out[:, :-1] = prev[:, 1:]
    out[:, -1] = nt
    return out
