"""The range arithmetic of the balanced attention split, checked on the CPU.

The split kernel concatenates the valid prefixes of a batch (T positions per
KV head), cuts them into W = min(S * K, T) equal ranges, K = ceil(T / (S *
1024)), S the workgroups per KV head, and piece (range v, sequence b) writes
record v + b; the merge reads records first(b) .. first(b) + count(b) - 1
with first(b) = owner(p0) + b, count(b) = owner(p0 + L - 1) - owner(p0) + 1,
owner(x) = ((x + 1) W - 1) // T.  The merge is only right if every record it
reads is one a piece wrote, and no two pieces write the same record.  The
rule is restated here in integers and checked exhaustively on small batches
and on random large ones (the device uses the same integer formulas)."""

import numpy as np

MAX_CHUNK = 1024


def plan(lengths, S):
    pre = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(pre[-1])
    K = max(1, -(-T // (S * MAX_CHUNK)))
    W = min(S * K, T)
    return pre, T, K, W


def owner(x, T, W):
    return ((x + 1) * W - 1) // T


def written_records(lengths, S):
    """Records the pieces write, with the positions each piece covers."""
    pre, T, K, W = plan(lengths, S)
    recs = {}
    for v in range(W):
        R0, R1 = v * T // W, (v + 1) * T // W
        assert R1 - R0 <= MAX_CHUNK
        for b in range(len(lengths)):
            s0, s1 = max(R0, pre[b]), min(R1, pre[b + 1])
            if s1 > s0:
                assert v + b not in recs, "two pieces write one record"
                recs[v + b] = (b, s0 - pre[b], s1 - pre[b])
    return recs


def merge_reads(lengths, S):
    pre, T, K, W = plan(lengths, S)
    out = []
    for b in range(len(lengths)):
        L = int(lengths[b])
        if L == 0:
            out.append(range(0))
            continue
        w0, w1 = owner(pre[b], T, W), owner(pre[b] + L - 1, T, W)
        out.append(range(w0 + b, w1 + b + 1))
    return out


def check(lengths, S):
    lengths = np.asarray(lengths, np.int64)
    if lengths.sum() == 0:
        return
    recs = written_records(lengths, S)
    reads = merge_reads(lengths, S)
    seen = set()
    for b, rr in enumerate(reads):
        covered = []
        for r in rr:
            assert r in recs, f"sequence {b} reads record {r} that no piece wrote"
            assert recs[r][0] == b, "a sequence reads another sequence's record"
            covered.append(recs[r][1:])
            seen.add(r)
        # the pieces of b tile its prefix [0, L) in order
        pos = 0
        for lo, hi in covered:
            assert lo == pos
            pos = hi
        assert pos == lengths[b]
    assert seen == set(recs), "a written record is never merged"
    _, T, _, W = plan(lengths, S)
    # records stay inside the workspace the host sizes for them
    B = len(lengths)
    assert max(recs) < W + B


def test_more_workgroups_than_positions():
    """The case that once left unwritten records: fewer positions than ranges."""
    for S in (1, 2, 7, 128, 160, 256):
        for B in (1, 2, 3, 16, 64):
            for L in (1, 2, 5, 37):
                check([L] * B, S)


def test_exhaustive_small_batches():
    rng = np.random.default_rng(7)
    for S in (1, 2, 3, 5, 8):
        for B in range(1, 7):
            for _ in range(40):
                check(rng.integers(0, 9, B), S)


def test_invalid_sequences_count_zero():
    check([0, 5, 0, 0, 3, 0], 4)
    check([0, 0, 1], 128)


def test_large_random_batches():
    rng = np.random.default_rng(11)
    for S in (128, 160, 256):
        for B, lo, hi in ((16, 234, 400), (64, 234, 4096), (64, 234, 8192), (64, 1, 3), (1024, 1, 64)):
            check(rng.integers(lo, hi + 1, B), S)
