"""Pins of the oracle's GQA decode attention: closed forms, an explicit
repeat_interleave expansion, torch's float64 SDPA over the full cache with a
narrowed mask, tail invariance, and the kv_len schedule of the page."""

import os

import numpy as np
import torch

from oracle import attention, fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, B=3, Hq=8, Hkv=2, D=16, cap=40):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Hq, D))
    k = g.standard_normal((B, Hkv, cap, D))
    v = g.standard_normal((B, Hkv, cap, D))
    L = g.integers(1, cap + 1, size=B)
    return q, k, v, L


def test_kv_len_one_returns_first_value():
    q, k, v, _ = _case(1)
    out = attention.gqa_decode_attention(q, k, v, np.ones(3, int))
    G = 8 // 2
    for h in range(8):
        assert np.array_equal(out[:, h], v[:, h // G, 0])


def test_zero_query_gives_mean_of_prefix():
    q, k, v, L = _case(2)
    out = attention.gqa_decode_attention(np.zeros_like(q), k, v, L)
    for b in range(3):
        for h in range(8):
            assert np.allclose(out[b, h], v[b, h // 4, :L[b]].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_gqa_equals_explicit_repeat_interleave():
    q, k, v, L = _case(3)
    G = 4
    kr = np.repeat(k, G, axis=1)          # repeat_interleave along the head axis
    vr = np.repeat(v, G, axis=1)
    out = attention.gqa_decode_attention(q, k, v, L)
    for b in range(3):
        s = np.einsum("hd,htd->ht", q[b], kr[b, :, :L[b]]) / np.sqrt(16)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ref = np.einsum("ht,htd->hd", p, vr[b, :, :L[b]])
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_active_prefix_equals_full_cache_with_mask_sdpa():
    """Section 7 of the KV-cache page: active-prefix output equals the full
    cache with a narrowed mask, within rtol 1e-5 / atol 1e-6."""
    q, k, v, L = _case(4, B=2, Hq=32, Hkv=8, D=128, cap=300)
    out = attention.gqa_decode_attention(q, k, v, L)
    kt = torch.from_numpy(k).repeat_interleave(4, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(4, dim=1)
    qt = torch.from_numpy(q)[:, :, None, :]
    mask = torch.arange(300)[None, None, None, :] < torch.from_numpy(L)[:, None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    assert np.allclose(out, ref[:, :, 0].numpy(), rtol=1e-5, atol=1e-6)


def test_tail_is_never_read():
    q, k, v, L = _case(5)
    k2, v2 = k.copy(), v.copy()
    for b in range(3):
        k2[b, :, L[b]:] = np.nan
        v2[b, :, L[b]:] = np.inf
    assert np.array_equal(attention.gqa_decode_attention(q, k, v, L),
                          attention.gqa_decode_attention(q, k2, v2, L))


def test_softmax_scale_default_is_inverse_sqrt_d():
    q, k, v, L = _case(6, D=64)
    a = attention.gqa_decode_attention(q, k, v, L)
    b = attention.gqa_decode_attention(q, k, v, L, scale=1 / 8.0)
    assert np.array_equal(a, b)


def test_invalid_kv_len_rejected():
    q, k, v, _ = _case(7)
    for bad in (0, 41):
        try:
            attention.gqa_decode_attention(q, k, v, np.array([1, bad, 1]))
        except ValueError:
            continue
        raise AssertionError("kv_len outside [1, cap] must be rejected")


def test_golden_kv_len_schedule():
    with open(os.path.join(GOLDEN, "kv_len_schedule.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for phase, idx, kv in rows:
        idx = int(idx)
        got = attention.kv_len_schedule(234, None if idx < 0 else idx)
        assert got == int(kv), (phase, idx)


def _mx_representable(g, shape):
    """Rows of 32-groups built from e4m3 codes and UE8M0 exponents such that
    every group holds a code of the top binade (256..448), so the OCP rule
    returns the very exponent, and dividing by it the very codes."""
    D = shape[-1]
    n_groups = int(np.prod(shape[:-1])) * (D // 32)
    codes = g.integers(0, 256, size=(n_groups, 32)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] &= 0xF7                    # no NaN codes
    top = g.integers(0x78, 0x7F, size=n_groups).astype(np.uint8) | (g.integers(0, 2, size=n_groups) << 7).astype(np.uint8)
    codes[np.arange(n_groups), g.integers(0, 32, size=n_groups)] = top
    exps = g.integers(110, 140, size=n_groups).astype(np.uint8)
    vals = fp8.e4m3_decode(codes) * np.ldexp(1.0, exps.astype(np.int64) - 127)[:, None]
    return (vals.reshape(shape), codes.reshape(shape),
            exps.reshape(tuple(shape[:-1]) + (D // 32,)))


def test_mxkv_equals_plain_attention_on_representable_rows():
    g = np.random.default_rng(11)
    B, Hq, Hkv, D, T = 2, 8, 2, 64, 50
    q = g.standard_normal((B, Hq, D))
    kval, kc, ke = _mx_representable(g, (B, Hkv, T, D))
    vval, vc, ve = _mx_representable(g, (B, Hkv, T, D))
    # the OCP quantiser gives back the codes and exponents the rows came from
    qk, ek = fp8.quant_mx_1x32(kval.reshape(-1, D).astype(np.float32))
    assert np.array_equal(qk, kc.reshape(-1, D)) and np.array_equal(ek, ke.reshape(-1, D // 32))
    L = np.array([50, 13])
    out = attention.gqa_decode_attention_mxkv(q, kc, ke, vc, ve, L)
    ref = attention.gqa_decode_attention(q, kval, vval, L)
    assert np.allclose(out, ref, rtol=1e-12, atol=0)


def test_mxkv_kv_len_one_returns_dequantised_first_value():
    g = np.random.default_rng(12)
    B, Hq, Hkv, D, T = 2, 4, 1, 64, 9
    q = g.standard_normal((B, Hq, D))
    _, kc, ke = _mx_representable(g, (B, Hkv, T, D))
    vval, vc, ve = _mx_representable(g, (B, Hkv, T, D))
    out = attention.gqa_decode_attention_mxkv(q, kc, ke, vc, ve, np.ones(B, int))
    for h in range(Hq):
        assert np.array_equal(out[:, h], vval[:, 0, 0])


def test_mx_kv_store_is_identity_on_representable_rows():
    """A row whose 32-groups are MX-representable is stored as it is."""
    g = np.random.default_rng(13)
    vals, _, _ = _mx_representable(g, (3, 2, 128))
    assert np.array_equal(attention.mx_kv_store(vals), vals)
    assert np.array_equal(attention.mx_kv_store(np.zeros((2, 64))), np.zeros((2, 64)))


def test_mx_kv_store_brute_force_nearest_grid_point():
    """Each stored value is the e4m3 grid point (times the group's power of
    two 2^(floor(log2 amax) - 8)) nearest to the input, found by a search
    over all 254 finite codes; inputs are drawn off the rounding midpoints."""
    g = np.random.default_rng(14)
    rows = g.standard_normal((4, 64)) * np.ldexp(1.0, g.integers(-6, 7, size=(4, 1)))
    got = attention.mx_kv_store(rows)
    grid = fp8.e4m3_decode(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8))
    for r in range(rows.shape[0]):
        for k in range(0, 64, 32):
            grp = rows[r, k:k + 32]
            X = np.ldexp(1.0, int(np.floor(np.log2(np.abs(grp).max()))) - 8)
            for i, x in enumerate(grp):
                d = np.abs(grid * X - x)
                assert np.sort(d)[1] - d.min() > 1e-12 * abs(x)   # not a tie
                assert got[r, k + i] == grid[np.argmin(d)] * X


def _scatter_pages(g, cache, P, spare=3):
    """A pool [pages, Hkv, P, D] holding a contiguous cache [B, Hkv, cap, D]
    (cap a multiple of P) on shuffled pages, plus `spare` NaN pages no
    sequence names, and the block table [B, cap / P]."""
    B, Hkv, cap, D = cache.shape
    n = B * cap // P
    order = g.permutation(n + spare)
    pool = np.full((n + spare, Hkv, P, D), np.nan)
    table = np.zeros((B, cap // P), np.int64)
    for b in range(B):
        for i in range(cap // P):
            pg = order[b * (cap // P) + i]
            table[b, i] = pg
            pool[pg] = cache[b, :, i * P:(i + 1) * P]
    return pool, table


def test_paged_equals_contiguous_on_shuffled_pages():
    g = np.random.default_rng(21)
    q, k, v, L = _case(21, cap=48)
    for P in (1, 4, 16):
        kp, table = _scatter_pages(g, k, P)
        vp = np.zeros_like(kp)
        for b in range(3):
            for i in range(48 // P):
                vp[table[b, i]] = v[b, :, i * P:(i + 1) * P]
        out = attention.gqa_decode_attention_paged(q, kp, vp, table, L, P)
        assert np.isfinite(out).all()
        assert np.array_equal(out, attention.gqa_decode_attention(q, k, v, L)), P


def test_paged_kv_len_one_returns_first_slot_of_first_page():
    g = np.random.default_rng(22)
    q = g.standard_normal((2, 4, 8))
    pool_k, pool_v = g.standard_normal((2, 5, 2, 4, 8))
    table = np.array([[3, 0], [1, 4]])
    out = attention.gqa_decode_attention_paged(q, pool_k, pool_v, table, [1, 1], 4)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], pool_v[table[b, 0], h // 2, 0])


def test_paged_brute_force_scalar_loop():
    """Tiny pool, every value from direct indexing and math.exp."""
    import math
    g = np.random.default_rng(23)
    B, Hq, Hkv, D, P, n_pages = 2, 4, 2, 3, 2, 7
    q = g.standard_normal((B, Hq, D))
    pk, pv = g.standard_normal((2, n_pages, Hkv, P, D))
    table = [[5, 2, 6], [0, 3, 1]]
    L = [5, 3]
    out = attention.gqa_decode_attention_paged(q, pk, pv, table, L, P, scale=0.7)
    for b in range(B):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            rows = [(table[b][t // P], t % P) for t in range(L[b])]
            s = [0.7 * sum(q[b, h, d] * pk[pg, kvh, sl, d] for d in range(D)) for pg, sl in rows]
            w = [math.exp(x - max(s)) for x in s]
            ref = [sum(w[i] * pv[pg, kvh, sl, d] for i, (pg, sl) in enumerate(rows)) / sum(w) for d in range(D)]
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-14)


def test_paged_out_of_pool_page_rejected():
    g = np.random.default_rng(24)
    q = g.standard_normal((1, 2, 8))
    pool = g.standard_normal((3, 1, 4, 8))
    for bad in (3, -1):
        try:
            attention.gqa_decode_attention_paged(q, pool, pool, [[0, bad]], [6], 4)
        except ValueError:
            continue
        raise AssertionError(f"page id {bad} accepted")
    # the same entry past kv_len is never read
    attention.gqa_decode_attention_paged(q, pool, pool, [[0, 99]], [4], 4)


def test_paged_mxkv_equals_paged_plain_on_dequantised_pool():
    g = np.random.default_rng(25)
    B, Hq, Hkv, D, P = 2, 8, 2, 64, 16
    q = g.standard_normal((B, Hq, D))
    kval, kc, ke = _mx_representable(g, (6, Hkv, P, D))
    vval, vc, ve = _mx_representable(g, (6, Hkv, P, D))
    table = np.array([[4, 1, 5], [0, 2, 3]])
    L = [40, 17]
    out = attention.gqa_decode_attention_paged_mxkv(q, kc, ke, vc, ve, table, L, P)
    ref = attention.gqa_decode_attention_paged(q, kval, vval, table, L, P)
    assert np.allclose(out, ref, rtol=1e-12, atol=0)


def _extend_case(seed, T, L, Hq=8, Hkv=2, D=16, cap=48):
    """Queries for T[b] new tokens and caches with kv_len L[b] (NaN past it)."""
    g = np.random.default_rng(seed)
    B = len(T)
    q_start = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    q = g.standard_normal((int(q_start[-1]), Hq, D))
    k = g.standard_normal((B, Hkv, cap, D))
    v = g.standard_normal((B, Hkv, cap, D))
    for b in range(B):
        k[b, :, L[b]:] = np.nan
        v[b, :, L[b]:] = np.nan
    return q, k, v, q_start


def test_extend_one_token_equals_decode():
    L = [30, 1, 48]
    q, k, v, qs = _extend_case(31, [1, 1, 1], L)
    out = attention.extend_attention(q, k, v, qs, L)
    assert np.array_equal(out, attention.gqa_decode_attention(q, k, v, np.array(L)))


def test_prefill_equals_torch_causal_sdpa():
    T = [20, 7]
    q, k, v, qs = _extend_case(32, T, T)
    out = attention.extend_attention(q, k, v, qs, T)
    for b in range(2):
        qt = torch.from_numpy(q[qs[b]:qs[b + 1]]).transpose(0, 1)                 # [Hq, T, D]
        kt = torch.from_numpy(k[b, :, :T[b]]).repeat_interleave(4, dim=0)
        vt = torch.from_numpy(v[b, :, :T[b]]).repeat_interleave(4, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        assert np.allclose(out[qs[b]:qs[b + 1]], ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)


def test_extend_equals_last_rows_of_full_prefill():
    L = [40, 25]
    T = [9, 25]
    qfull, k, v, qs_full = _extend_case(33, L, L)
    full = attention.extend_attention(qfull, k, v, qs_full, L)
    rows = np.concatenate([np.arange(qs_full[b + 1] - T[b], qs_full[b + 1]) for b in range(2)])
    qs = np.concatenate([[0], np.cumsum(T)])
    out = attention.extend_attention(qfull[rows], k, v, qs, L)
    assert np.array_equal(out, full[rows])


def test_extend_brute_force_scalar_loop():
    import math
    T, L = [3, 2], [5, 2]
    q, k, v, qs = _extend_case(34, T, L, Hq=2, Hkv=1, D=3, cap=6)
    out = attention.extend_attention(q, k, v, qs, L, scale=0.6)
    for b in range(2):
        for t in range(T[b]):
            p = L[b] - T[b] + t
            for h in range(2):
                qv = q[qs[b] + t, h]
                s = [0.6 * sum(qv[d] * k[b, 0, j, d] for d in range(3)) for j in range(p + 1)]
                w = [math.exp(x - max(s)) for x in s]
                ref = [sum(w[j] * v[b, 0, j, d] for j in range(p + 1)) / sum(w) for d in range(3)]
                assert np.allclose(out[qs[b] + t, h], ref, rtol=1e-12, atol=1e-14)


def test_extend_rejects_bad_lengths_and_allows_empty():
    q, k, v, qs = _extend_case(35, [2, 0], [3, 4])
    out = attention.extend_attention(q, k, v, qs, [3, 4])
    assert out.shape == (2, 8, 16) and np.isfinite(out).all()
    try:
        attention.extend_attention(q, k, v, qs, [1, 4])          # T > kv_len
    except ValueError:
        return
    raise AssertionError("T > kv_len accepted")
