"""Pins of the Dual-AR decode-step oracle (oracle/dual_ar.py) against
closed forms, brute force and library routines; no GPU."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import dual_ar as da

H, I, HQ, HKV, D = 256, 384, 4, 2, 64
G = HQ // HKV


def _rand_layer(rs, zero_out=False):
    def w(n, k, std=0.05):
        return rs.standard_normal((n, k)).astype(np.float32) * np.float32(std)
    raw = {"qkv": w((HQ + 2 * HKV) * D, H), "o": w(H, HQ * D), "gate": w(I, H), "up": w(I, H), "down": w(H, I)}
    if zero_out:
        raw["o"][:] = 0
        raw["down"][:] = 0
    p = {k: da.dequant_weight(oracle.round_bf16(v))[2] for k, v in raw.items()}
    p["norm_attn"] = oracle.round_bf16(1 + 0.1 * rs.standard_normal(H))
    p["norm_mlp"] = oracle.round_bf16(1 + 0.1 * rs.standard_normal(H))
    return p


def _cache(rs, B, slots):
    return (oracle.round_bf16(rs.standard_normal((B, HKV, slots, D))),
            oracle.round_bf16(rs.standard_normal((B, HKV, slots, D))))


# ---- bf16 rounding ----------------------------------------------------------------
def test_round_bf16_matches_torch_cast_on_fp32_values():
    rs = np.random.default_rng(0)
    x = np.concatenate([rs.standard_normal(100000) * np.exp(rs.uniform(-90, 90, 100000)),
                        np.ldexp(1.0 + np.arange(256) / 256.0 + 1.0 / 512, 3),    # exact ties
                        np.ldexp(rs.uniform(1, 2, 1000), -130)]).astype(np.float32)  # bf16 subnormals
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_is_nearest_with_ties_to_even_by_search():
    # every positive finite bf16 value, ascending
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    rs = np.random.default_rng(1)
    x = np.abs(rs.standard_normal(20000)) * np.exp(rs.uniform(-80, 80, 20000))
    x = np.concatenate([x, (vals[1:200] + vals[:199]) / 2])           # midpoints (ties)
    i = np.clip(np.searchsorted(vals, x), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = (hi - x < x - lo) | ((hi - x == x - lo) & (bits[i] % 2 == 0))
    want = np.where(pick_hi, hi, lo)
    got = oracle.round_bf16(x)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(oracle.round_bf16(-x), -want)


# ---- RMSNorm ----------------------------------------------------------------------
def test_rmsnorm_matches_torch_rms_norm():
    rs = np.random.default_rng(2)
    x = oracle.round_bf16(rs.standard_normal((7, H)) * 3)
    w = oracle.round_bf16(1 + 0.1 * rs.standard_normal(H))
    ref = F.rms_norm(torch.from_numpy(x), (H,), torch.from_numpy(w), eps=oracle.RMS_EPS).numpy()
    np.testing.assert_array_equal(oracle.rmsnorm(x, w), oracle.round_bf16(ref))


def test_rmsnorm_constant_row_closed_form():
    c = np.array([[0.5] * H, [-3.0] * H, [1e-3] * H])
    w = np.full(H, 1.25)
    want = oracle.round_bf16(c / np.sqrt(c * c + oracle.RMS_EPS) * 1.25)
    np.testing.assert_array_equal(oracle.rmsnorm(c, w), want)


# ---- the block -----------------------------------------------------------------------
def test_layer_with_zero_output_projections_is_identity_and_appends_kv():
    rs = np.random.default_rng(3)
    B, slots = 3, 16
    p = _rand_layer(rs, zero_out=True)
    kc, vc = _cache(rs, B, slots)
    k0, v0 = kc.copy(), vc.copy()
    kv_len = np.array([1, 9, 16])
    x = oracle.round_bf16(rs.standard_normal((B, H)))
    out, it = oracle.decoder_layer(x, p, kc, vc, kv_len, HQ, HKV, D)
    np.testing.assert_array_equal(out, x)
    for b in range(B):
        t = kv_len[b] - 1
        np.testing.assert_array_equal(kc[b, :, t], it["k"][b])
        np.testing.assert_array_equal(vc[b, :, t], it["v"][b])
        keep = np.arange(slots) != t
        np.testing.assert_array_equal(kc[b][:, keep], k0[b][:, keep])
        np.testing.assert_array_equal(vc[b][:, keep], v0[b][:, keep])


def test_single_slot_attention_returns_the_appended_value():
    rs = np.random.default_rng(4)
    B = 2
    p = _rand_layer(rs)
    kc, vc = _cache(rs, B, 8)
    out, it = oracle.decoder_layer(oracle.round_bf16(rs.standard_normal((B, H))), p, kc, vc,
                                   np.array([1, 1]), HQ, HKV, D)
    for h in range(HQ):
        np.testing.assert_array_equal(it["attn"][:, h * D:(h + 1) * D], it["v"][:, h // G])


def test_layer_matches_a_torch_composition():
    """The block rebuilt from torch's rms_norm, silu and
    scaled_dot_product_attention (GQA by repeat_interleave over the prefix,
    with a -inf mask on the tail) around the pinned FP8 linear."""
    rs = np.random.default_rng(5)
    B, slots = 3, 24
    p = _rand_layer(rs)
    kc, vc = _cache(rs, B, slots)
    kv_len = np.array([5, 24, 13])
    x = oracle.round_bf16(rs.standard_normal((B, H)) * 2)
    kc_t, vc_t = torch.from_numpy(kc.copy()), torch.from_numpy(vc.copy())
    out, _ = oracle.decoder_layer(x, p, kc, vc, kv_len, HQ, HKV, D)

    def lin(a, w):
        return torch.from_numpy(oracle.fp8_linear(a.numpy(), w))

    def bf(t):
        return torch.from_numpy(oracle.round_bf16(t.numpy()))

    xt = torch.from_numpy(x)
    xn = bf(F.rms_norm(xt, (H,), torch.from_numpy(p["norm_attn"]), eps=oracle.RMS_EPS))
    qkv = bf(lin(xn, p["qkv"]))
    q, k, v = qkv.split([HQ * D, HKV * D, HKV * D], dim=1)
    q = q.view(B, HQ, D)
    rows = torch.arange(B)
    kc_t[rows, :, torch.from_numpy(kv_len - 1)] = k.view(B, HKV, D)
    vc_t[rows, :, torch.from_numpy(kv_len - 1)] = v.view(B, HKV, D)
    mask = torch.arange(slots)[None, :] < torch.from_numpy(kv_len)[:, None]          # [B, slots]
    attn_mask = torch.zeros(B, 1, 1, slots, dtype=torch.float64).masked_fill(~mask[:, None, None, :], float("-inf"))
    o = F.scaled_dot_product_attention(q[:, :, None, :], kc_t.repeat_interleave(G, dim=1),
                                       vc_t.repeat_interleave(G, dim=1), attn_mask=attn_mask)
    attn = bf(o.reshape(B, HQ * D))
    x_mid = bf(xt + lin(attn, p["o"]))
    xn2 = bf(F.rms_norm(x_mid, (H,), torch.from_numpy(p["norm_mlp"]), eps=oracle.RMS_EPS))
    g, u = lin(xn2, p["gate"]), lin(xn2, p["up"])
    hdn = (F.silu(g) * u).to(torch.float32).to(torch.float64)
    y = lin(hdn, p["down"])
    ref = bf(x_mid + y).numpy()
    # a float64 difference in softmax order may move a value across a bf16
    # rounding boundary somewhere upstream: allow a few bf16 steps
    err = np.abs(out - ref).max() / np.abs(ref).max()
    assert err < 2e-2
    assert np.mean(out == ref) > 0.95


# ---- the codebook chain -------------------------------------------------------------
def test_codebook_chain_follows_the_closed_form():
    """Embeddings E_c[k] = e_{pi_c(k)}, head 0 = identity, head p+1 rows
    e_{pi_p(rho_p(j))}, zero output projections, a slow norm weight that keeps
    one coordinate j*.  Then code 0 = j*, code 1 = rho_0^-1(pi_0^-1(j*))
    (h is added at the first micro-step only) and code p+1 = rho_p^-1(code p)."""
    rs = np.random.default_rng(6)
    C, V, B = 10, H, 2
    pis = [rs.permutation(V) for _ in range(C)]
    rhos = [rs.permutation(V) for _ in range(C - 1)]
    eye = np.eye(V)
    embed = [eye[pi] for pi in pis]                       # row k = e_{pi(k)}
    heads = [da.dequant_weight(eye)[2]] + [da.dequant_weight(eye[pis[p][rhos[p]]])[2] for p in range(C - 1)]
    prev = np.stack([rs.permutation(V)[:C] for _ in range(B)]).astype(np.int32)
    # make the ten slow-input coordinates distinct per row
    for b in range(B):
        while len({int(pis[c][prev[b, c]]) for c in range(C)}) < C:
            prev[b] = rs.permutation(V)[:C]
    jstar = np.array([pis[3][prev[b, 3]] for b in range(B)])
    model = {"slow": [_rand_layer(rs, zero_out=True)], "fast": [_rand_layer(rs, zero_out=True)],
             "embed": embed, "heads": heads, "fast_norm": np.ones(H),
             "n_heads": HQ, "n_kv_heads": HKV, "head_dim": D}
    kc, vc = _cache(rs, B, 4)
    kv_len = np.array([2, 4])
    for b in range(B):
        slow_w = np.zeros(H)
        slow_w[jstar[b]] = 10.0
        model["slow_norm"] = slow_w
        r = oracle.dual_ar_step(model, prev[b:b + 1], [kc[b:b + 1].copy()], [vc[b:b + 1].copy()], kv_len[b:b + 1])
        inv = [np.argsort(pi) for pi in pis]
        rinv = [np.argsort(rho) for rho in rhos]
        want = [int(jstar[b]), int(rinv[0][inv[0][jstar[b]]])]
        for p in range(1, C - 1):
            want.append(int(rinv[p][want[p]]))
        assert r["codes"][0].tolist() == want
        # adding h at every micro-step (a plausible slip) would give other codes
        wrong = [int(rinv[p][inv[p][jstar[b]]]) for p in range(1, C - 1)]
        assert wrong != want[2:]


def test_teacher_forcing_with_its_own_outputs_changes_nothing():
    rs = np.random.default_rng(7)
    C, V, B = 10, 128, 3
    model = {"slow": [_rand_layer(rs) for _ in range(2)], "fast": [_rand_layer(rs)],
             "embed": [oracle.round_bf16(0.05 * rs.standard_normal((V, H))) for _ in range(C)],
             "heads": [da.dequant_weight(oracle.round_bf16(0.05 * rs.standard_normal((V, H))))[2] for _ in range(C)],
             "slow_norm": oracle.round_bf16(1 + 0.1 * rs.standard_normal(H)),
             "fast_norm": oracle.round_bf16(1 + 0.1 * rs.standard_normal(H)),
             "n_heads": HQ, "n_kv_heads": HKV, "head_dim": D}
    prev = rs.integers(0, V, (B, C)).astype(np.int32)
    kv_len = np.array([3, 12, 7])
    caches = [_cache(rs, B, 12) for _ in range(2)]
    free = oracle.dual_ar_step(model, prev, [c[0].copy() for c in caches], [c[1].copy() for c in caches], kv_len)
    force = {"slow_x": free["slow_x"], "codes": free["codes"], "fast_x": free["fast_x"]}
    forced = oracle.dual_ar_step(model, prev, [c[0].copy() for c in caches], [c[1].copy() for c in caches],
                                 kv_len, force=force)
    np.testing.assert_array_equal(forced["codes"], free["codes"])
    for a, b in zip(forced["slow_x"], free["slow_x"]):
        np.testing.assert_array_equal(a, b)
    for p in range(C - 1):
        for a, b in zip(forced["fast_x"][p], free["fast_x"][p]):
            np.testing.assert_array_equal(a, b)


def test_kv_len_out_of_range_raises():
    rs = np.random.default_rng(8)
    p = _rand_layer(rs)
    kc, vc = _cache(rs, 1, 4)
    with pytest.raises(ValueError):
        oracle.decoder_layer(np.zeros((1, H)), p, kc, vc, np.array([5]), HQ, HKV, D)
    with pytest.raises(ValueError):
        oracle.decoder_layer(np.zeros((1, H)), p, kc, vc, np.array([0]), HQ, HKV, D)
