"""The full Dual-AR decode step on the GPU against the oracle, teacher forced:
the output of every half-block (attention half, MLP half) of every layer and
micro-step is compared with the oracle applied to the GPU's own input of that
half-block, so FP8 re-quantisation flips and argmax near-ties cannot
compound.  The codes must be the exact argmax of
the GPU's logits, and those logits must match the oracle's.

A small model with the same structure is checked on every layer, row and
micro-step; the full model (36 slow layers, 4 fast layers, batch 64, caches
of 32768 slots, kv_len up to 4096) on sampled layers and rows."""

import numpy as np
import pytest
import torch

import oracle
from fp8_transformer_step_amd import model, ops
from _helpers import TOL_FP8_PATH, f32, log, max_rel_err, need_gpu

pytestmark = pytest.mark.gpu
# An MXFP8 cache row against the bf16 row it stores: up to 1/8 of a group's
# largest magnitude (saturation at 448 of a group scaled into [256, 512)),
# plus the bf16 path's own tolerance for the row itself.
MX_KV_TOL = 1 / 8 + TOL_FP8_PATH


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _oracle_block(d):
    p = {k: oracle.dequant_weight(f32(d[k]))[2] for k in ("qkv", "o", "gate", "up", "down")}
    p["norm_attn"] = f32(d["norm_attn"]).astype(np.float64)
    p["norm_mlp"] = f32(d["norm_mlp"]).astype(np.float64)
    return p


def _prefix_cache(host, s, rows):
    """The oracle's copy of physical set s for the given rows (initial content)."""
    c = host.cfg
    Lmax = int(max(host.kv_len[b] for b in rows))
    k = np.zeros((len(rows), c.n_kv_heads, Lmax, c.head_dim), np.float32)
    v = np.zeros_like(k)
    for i, b in enumerate(rows):
        kp, vp = host.kv_prefix(s, b)
        k[i, :, :kp.shape[1]] = f32(kp)
        v[i, :, :vp.shape[1]] = f32(vp)
    return k, v


def _prefix_cache_mx(host, s, rows):
    """_prefix_cache as an MXFP8 cache holds it (the oracle's MX store of
    every prefix row)."""
    k, v = _prefix_cache(host, s, rows)
    return oracle.mx_kv_store(k), oracle.mx_kv_store(v)


def _dequant_mx(cache, b, t):
    """The values of an MxKvCache at sequence b, slot t: [Hkv, D] float64."""
    from oracle import attention as oattn
    return oattn.dequant_mx_rows(cache.q[b, :, t].cpu().numpy(), cache.e[b, :, t].cpu().numpy())


def _ulp_close(got, want):
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(want), 1e-30))[1] - 8)
    return bool(np.all(np.abs(got - want) <= ulp))


def _clone(c):
    return ops.MxKvCache(c.q.clone(), c.e.clone()) if isinstance(c, ops.MxKvCache) else c.clone()


def _run_step(host, mx=False):
    c = host.cfg
    dm = model.device_model(host)
    kv, ks, vs = model.device_kv(host, mx=mx)
    k0 = [_clone(k) for k in ks]
    v0 = [_clone(v) for v in vs]
    B, H, C, V = c.batch, c.hidden, c.n_codebooks, c.codebook_size
    slow_taps = torch.empty((2 * c.n_slow_layers + 1, B, H), dtype=torch.bfloat16, device="cuda")
    fast_taps = torch.empty((C - 1, 2 * c.n_fast_layers + 1, B, H), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((C, B, V), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    log(f"dual-AR step B={B} L={c.n_slow_layers} F={c.n_fast_layers} H={H} V={V}")
    codes = ops.dual_ar_decode_step(dm, kv, torch.from_numpy(host.prev_codes).cuda(), slow_taps=slow_taps,
                                    fast_taps=fast_taps, logits_tap=logits, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    out = {"codes": codes.cpu().numpy(), "slow": _np(slow_taps), "fast": _np(fast_taps),
           "logits": logits.cpu().numpy().astype(np.float64), "ks": ks, "vs": vs, "k0": k0, "v0": v0}
    # the codes are the exact greedy decisions on the GPU's logits
    np.testing.assert_array_equal(out["codes"], np.argmax(out["logits"], axis=2).T)
    # a second call on the same inputs gives the same codes (deterministic reductions)
    codes2 = ops.dual_ar_decode_step(dm, kv, torch.from_numpy(host.prev_codes).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes2.cpu().numpy(), out["codes"])
    return out


@pytest.mark.parametrize("batch,n_heads", [(5, 4), (24, 8), (100, 8)])
def test_small_model_every_layer_teacher_forced(batch, n_heads):
    """Batch 5, 24 and 100 take the one-, two- and eight-tile (16 rows per
    tile) variants of every projection and of the split-partial finisher.

    The larger batches use 8 query heads here: with 4 heads of 64 the output
    projection contracts over only 256 values, so one e4m3 rounding flip of
    an attention output moves a residual entry by about 2 % of the tensor's
    maximum when the oracle quantises its own attention output.  The 4-head
    batch-24 model is checked in test_gpu_taps instead, on the GPU's own
    operand bytes (themselves checked bit-exact against the oracle's
    quantisation of the GPU's attention output)."""
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=batch, n_heads=n_heads))
    c = host.cfg
    g = _run_step(host)
    C, F, L = c.n_codebooks, c.n_fast_layers, c.n_slow_layers
    om = {"slow": [_oracle_block(d) for d in host.slow], "fast": [_oracle_block(d) for d in host.fast],
          "slow_norm": f32(host.slow_norm).astype(np.float64), "fast_norm": f32(host.fast_norm).astype(np.float64),
          "embed": [f32(t) for t in host.embed], "heads": [oracle.dequant_weight(f32(h))[2] for h in host.heads],
          "n_heads": c.n_heads, "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim, "eps": c.rms_eps}
    rows = list(range(c.batch))
    caches = [_prefix_cache(host, l % c.kv_sets, rows) for l in range(L)]
    force = {"slow_x": list(g["slow"]), "codes": g["codes"], "fast_x": [list(g["fast"][p]) for p in range(C - 1)]}
    r = oracle.dual_ar_step(om, host.prev_codes, [k for k, _ in caches], [v for _, v in caches], host.kv_len,
                            force=force)
    assert _ulp_close(g["slow"][0], r["slow_x"][0])
    for i in range(1, 2 * L + 1):
        e = max_rel_err(g["slow"][i], r["slow_x"][i])
        log(f"  slow layer {(i - 1) // 2} {'attention' if i % 2 else 'mlp'} half: {e:.3e}")
        assert e <= TOL_FP8_PATH
    for cb in range(C):
        e = max_rel_err(g["logits"][cb], r["logits"][cb])
        log(f"  head {cb}: {e:.3e}, codes equal to the oracle's argmax: "
            f"{np.mean(g['codes'][:, cb] == r['codes'][:, cb]):.2f}")
        assert e <= TOL_FP8_PATH
    for p in range(C - 1):
        assert max_rel_err(g["fast"][p][0], r["fast_x"][p][0]) <= 2 ** -7
        for i in range(1, 2 * F + 1):
            e = max_rel_err(g["fast"][p][i], r["fast_x"][p][i])
            assert e <= TOL_FP8_PATH, (p, i, e)
    # caches: the last layer on each set left its K/V at kv_len - 1, nothing else changed
    for s in range(c.kv_sets):
        last = max(l for l in range(L) if l % c.kv_sets == s)
        kk, vv = r["slow_kv"][last]
        kg, vg = g["ks"][s], g["vs"][s]
        for b in rows:
            t = int(host.kv_len[b]) - 1
            assert max_rel_err(_np(kg[b, :, t]), kk[b]) <= TOL_FP8_PATH
            assert max_rel_err(_np(vg[b, :, t]), vv[b]) <= TOL_FP8_PATH
            keep = torch.arange(c.cap, device="cuda") != t
            assert torch.equal(kg[b][:, keep].view(torch.int16), g["k0"][s][b][:, keep].view(torch.int16))
            assert torch.equal(vg[b][:, keep].view(torch.int16), g["v0"][s][b][:, keep].view(torch.int16))


def test_small_model_mxfp8_kv_teacher_forced():
    """The step with MXFP8 slow-layer caches: every half-block against the
    oracle whose slow caches hold the MX store of their rows (prefix and
    appended row); the appended rows dequantise to the oracle's bf16 K/V
    within the MX rounding: the OCP rule scales a group's largest magnitude
    into [256, 512) and e4m3 saturates at 448, so an element can lose up to
    1/8 of the group's largest magnitude (half an e4m3 step, 1/16, below
    that); no other cache byte changes."""
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=24, n_heads=8))
    c = host.cfg
    g = _run_step(host, mx=True)
    C, F, L = c.n_codebooks, c.n_fast_layers, c.n_slow_layers
    om = {"slow": [_oracle_block(d) for d in host.slow], "fast": [_oracle_block(d) for d in host.fast],
          "slow_norm": f32(host.slow_norm).astype(np.float64), "fast_norm": f32(host.fast_norm).astype(np.float64),
          "embed": [f32(t) for t in host.embed], "heads": [oracle.dequant_weight(f32(h))[2] for h in host.heads],
          "n_heads": c.n_heads, "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim, "eps": c.rms_eps}
    rows = list(range(c.batch))
    caches = [_prefix_cache_mx(host, l % c.kv_sets, rows) for l in range(L)]
    force = {"slow_x": list(g["slow"]), "codes": g["codes"], "fast_x": [list(g["fast"][p]) for p in range(C - 1)]}
    r = oracle.dual_ar_step(om, host.prev_codes, [k for k, _ in caches], [v for _, v in caches], host.kv_len,
                            force=force, slow_kv_store=oracle.mx_kv_store)
    for i in range(1, 2 * L + 1):
        e = max_rel_err(g["slow"][i], r["slow_x"][i])
        log(f"  slow layer {(i - 1) // 2} {'attention' if i % 2 else 'mlp'} half: {e:.3e}")
        assert e <= TOL_FP8_PATH
    for cb in range(C):
        assert max_rel_err(g["logits"][cb], r["logits"][cb]) <= TOL_FP8_PATH
    for p in range(C - 1):
        for i in range(1, 2 * F + 1):
            assert max_rel_err(g["fast"][p][i], r["fast_x"][p][i]) <= TOL_FP8_PATH, (p, i)
    for s in range(c.kv_sets):
        last = max(l for l in range(L) if l % c.kv_sets == s)
        kk, vv = r["slow_kv"][last]
        kg, vg, k0, v0 = g["ks"][s], g["vs"][s], g["k0"][s], g["v0"][s]
        for b in rows:
            t = int(host.kv_len[b]) - 1
            for got, want in ((_dequant_mx(kg, b, t), kk[b]), (_dequant_mx(vg, b, t), vv[b])):
                assert max_rel_err(got, want) <= MX_KV_TOL
            keep = torch.arange(c.cap, device="cuda") != t
            for now, before in ((kg, k0), (vg, v0)):
                assert torch.equal(now.q[b][:, keep], before.q[b][:, keep])
                assert torch.equal(now.e[b][:, keep], before.e[b][:, keep])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mx", [False, True], ids=["bf16_kv", "mxfp8_kv"])
def test_full_model_sampled_layers_teacher_forced(mx):
    need_gpu()
    host = model.HostModel(model.FULL)
    c = host.cfg
    g = _run_step(host, mx=mx)
    C, F, L = c.n_codebooks, c.n_fast_layers, c.n_slow_layers
    rows = sorted({0, 13, 29, 47, c.batch - 1, int(np.argmax(host.kv_len)), int(np.argmin(host.kv_len))})
    log(f"  sampled rows {rows}, kv_len {[int(host.kv_len[b]) for b in rows]}")
    D = c.head_dim
    for l in (0, 17, L - 1):
        p = _oracle_block(host.slow[l])
        k, v = (_prefix_cache_mx if mx else _prefix_cache)(host, l % c.kv_sets, rows)
        mid, it = oracle.attention_block(g["slow"][2 * l][rows], p, k, v, host.kv_len[rows], c.n_heads,
                                         c.n_kv_heads, D, c.rms_eps, oracle.mx_kv_store if mx else None)
        out, _ = oracle.mlp_block(g["slow"][2 * l + 1][rows], p, c.rms_eps)
        e1 = max_rel_err(g["slow"][2 * l + 1][rows], mid)
        e2 = max_rel_err(g["slow"][2 * l + 2][rows], out)
        log(f"  slow layer {l}: attention half {e1:.3e}, mlp half {e2:.3e}")
        assert e1 <= TOL_FP8_PATH and e2 <= TOL_FP8_PATH
        if l == L - 1:           # the last layer on its set: its K/V row is what the cache holds now
            s = l % c.kv_sets
            for i, b in enumerate(rows):
                t = int(host.kv_len[b]) - 1
                if mx:
                    assert max_rel_err(_dequant_mx(g["ks"][s], b, t), it["k"][i]) <= MX_KV_TOL
                    assert max_rel_err(_dequant_mx(g["vs"][s], b, t), it["v"][i]) <= MX_KV_TOL
                else:
                    assert max_rel_err(_np(g["ks"][s][b, :, t]), it["k"][i]) <= TOL_FP8_PATH
                    assert max_rel_err(_np(g["vs"][s][b, :, t]), it["v"][i]) <= TOL_FP8_PATH
    heads = [oracle.dequant_weight(f32(h))[2] for h in host.heads]
    h = oracle.rmsnorm(g["slow"][2 * L][rows], f32(host.slow_norm))
    lg, _ = oracle.greedy_code(h, heads[0])
    e = max_rel_err(g["logits"][0][rows], lg)
    log(f"  head 0: {e:.3e}")
    assert e <= TOL_FP8_PATH
    fast = [_oracle_block(d) for d in host.fast]
    fk = [np.zeros((len(rows), c.n_kv_heads, C - 1, D)) for _ in range(F)]
    fv = [np.zeros((len(rows), c.n_kv_heads, C - 1, D)) for _ in range(F)]
    for p in range(C - 1):
        z = oracle.embed_sum([f32(host.embed[p])], g["codes"][rows, p:p + 1], add=h if p == 0 else None)
        assert max_rel_err(g["fast"][p][0][rows], z) <= 2 ** -7
        steps = np.full(len(rows), p + 1)
        for f in range(F):
            mid, _ = oracle.attention_block(g["fast"][p][2 * f][rows], fast[f], fk[f], fv[f], steps, c.n_heads,
                                            c.n_kv_heads, D, c.rms_eps)
            out, _ = oracle.mlp_block(g["fast"][p][2 * f + 1][rows], fast[f], c.rms_eps)
            e1 = max_rel_err(g["fast"][p][2 * f + 1][rows], mid)
            e2 = max_rel_err(g["fast"][p][2 * f + 2][rows], out)
            assert e1 <= TOL_FP8_PATH and e2 <= TOL_FP8_PATH, (p, f, e1, e2)
        zn = oracle.rmsnorm(g["fast"][p][2 * F][rows], f32(host.fast_norm))
        lg, _ = oracle.greedy_code(zn, heads[p + 1])
        e = max_rel_err(g["logits"][p + 1][rows], lg)
        log(f"  micro-step {p}: head {p + 1} {e:.3e}")
        assert e <= TOL_FP8_PATH


def test_packed_weights_give_the_same_step():
    """Fragment-packed weights (the layout device_model uses by default) and
    row-major ones give the same logits and codes, bit for bit, on the
    4-head batch-24 model."""
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=24, n_heads=4))
    out = []
    for packed in (False, True):
        dm = model.device_model(host, packed=packed)
        kv, _, _ = model.device_kv(host)
        logits = torch.empty((host.cfg.n_codebooks, host.cfg.batch, host.cfg.codebook_size), dtype=torch.float32,
                             device="cuda")
        log(f"dual-AR step packed={packed}")
        codes = ops.dual_ar_decode_step(dm, kv, torch.from_numpy(host.prev_codes).cuda(), logits_tap=logits)
        torch.cuda.synchronize()
        out.append((codes.cpu().numpy(), logits.cpu().numpy()))
    np.testing.assert_array_equal(out[0][0], out[1][0])
    np.testing.assert_array_equal(out[0][1], out[1][1])


def test_out_of_range_previous_code_is_reported_and_skipped():
    """A previous-frame code outside [0, codebook_size) sets
    FP8S_DEV_CODE_RANGE and adds nothing to its row's input embedding; the
    other rows and codes are untouched."""
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=5, n_heads=4))
    c = host.cfg
    B, H, C, V = c.batch, c.hidden, c.n_codebooks, c.codebook_size
    dm = model.device_model(host)
    kv, _, _ = model.device_kv(host)
    prev = host.prev_codes.copy()
    prev[2, 3] = V
    prev[4, 0] = -1
    slow_taps = torch.empty((2 * c.n_slow_layers + 1, B, H), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.dual_ar_decode_step(dm, kv, torch.from_numpy(prev).cuda(), slow_taps=slow_taps, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == ops.DEV_CODE_RANGE
    got = _np(slow_taps[0])
    tables = [f32(t) for t in host.embed]
    for b in range(B):
        keep = [t for t in range(C) if 0 <= prev[b, t] < V]
        want = oracle.embed_sum([tables[t] for t in keep], prev[b:b + 1, keep])[0]
        assert _ulp_close(got[b], want), b
