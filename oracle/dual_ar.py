"""The full batched Dual-AR decode step (slow AR over the layers, then the
fast AR over the codebooks), in float64 NumPy.

Test infrastructure only (see the package header).

What the step is, from the pages:
  * "Fish Speech KV Cache 推理优化记录", section 2 (how Fish Speech turns text
    into speech): a frame of audio is one token per codebook of a 10-codebook
    RVQ; the slow AR advances in time, predicts the frame's main semantic
    token and hands its hidden state on; the fast AR then generates the
    remaining codebook tokens of the frame one after another, conditioned on
    it; the frame's tokens become context for the next slow step.
  * The same page, sections 4-5: the slow AR's layers attend over a KV cache
    pre-allocated at full capacity, reading only the kv_len prefix; the new
    token's K/V is written at kv_len - 1 before the query attends.
  * "How We Made Our Text-to-Speech API Free", "Why cuBLAS Wasn't Enough" and
    "Kernel Benchmark Results": every projection is an FP8 GEMM with
    block-scaled weights and on-the-fly activation quantisation; the MLP is
    the SwiGLU MLP of oracle.mlp.
  * "How We Made Our Text-to-Speech API Free", "DualAR: S2-Specific Batching
    Constraints": coarse codebook first, then the fine codebooks, per step.
  * "How Fish Audio Keeps a GPU Busy: Continuous Batching for Streaming
    Speech", section "Where speech makes it harder": the slow AR predicts a
    semantic code and a smaller fast AR fills in the remaining nine codebook
    tokens.

Readings of what the pages leave open (each also listed in the design notes):
  * Block: pre-norm, x += O(attn(RMSNorm(x))); x += MLP(RMSNorm(x)).  RMSNorm
    is x / sqrt(mean(x^2) + eps) * w with eps = 1e-6.  No rotary embedding
    and no q/k norm (not described on the pages; they move no weight bytes).
  * QKV is one FP8 GEMM whose output columns are [q heads | k heads | v heads],
    head-major, head_dim contiguous.
  * Activations between operations are bf16 (the dtype the pages' model runs
    in): the residual stream, RMSNorm outputs, q/k/v, the attention output.
    Each is rounded to nearest-even bf16 from the float64 result here.
  * Slow-AR input: the sum over codebooks of the previous frame's code
    embeddings, E_c[prev_code_c] (the frame's tokens as context).
  * After the last slow layer: h = RMSNorm(x) with its own weight; code 0 =
    argmax of the FP8 head 0 applied to h (greedy).
  * Fast AR: the same block shape, its own layers, its own small cache
    (one slot per micro-step); micro-step p = 0..C-2 takes
    z = bf16(h + E_0[code_0]) when p = 0 and z = E_p[code_p] after that,
    runs the fast layers with kv_len = p + 1, and picks code p+1 = argmax of
    head p+1 applied to RMSNorm(z) (fast final norm).  The embedding tables
    are shared by the slow-AR input and the fast AR.
  * argmax ties go to the lowest index (greedy decoding).

Pins (tests/test_oracle_dual_ar.py): bf16 rounding against torch's cast and
a brute-force nearest search; RMSNorm against torch.nn.functional.rms_norm
and a closed form; a layer with zero output projections is the identity and
writes its K/V row; a single-slot cache returns the appended value; the layer
against a composition built on torch's scaled_dot_product_attention; a code
chain with permutation-structured embeddings and heads whose codes follow in
closed form.
"""

import numpy as np

from .attention import gqa_decode_attention
from .fp8 import dequant_block_fp32, quant_weight_128x128
from .mlp import MODE_BSGEMM, linear_dequant, quant_act, swiglu_mlp

RMS_EPS = 1e-6


def round_bf16(x):
    """Round float64 values to the nearest bf16 value (ties to even).

    bf16 keeps 8 significant bits; below 2^-126 the step is fixed at 2^-133.
    Values beyond the bf16 range are not expected here (finite activations).
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, e = np.frexp(np.where(a > 0, a, 1.0))          # a in [2^(e-1), 2^e)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(a / step) * step                      # exact in float64
    return np.where(a > 0, np.copysign(r, x), x)


def rmsnorm(x, w, eps=RMS_EPS):
    """bf16(x / sqrt(mean(x^2) + eps) * w) row-wise, in float64."""
    x = np.asarray(x, np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return round_bf16(x / r * np.asarray(w, np.float64))


def fp8_linear(x, w_deq):
    """x [M, K] (bf16 values) quantised 1x128 / fp32 scale, times a dequantised
    128x128 block-scaled weight [N, K]: float64 [M, N]."""
    _, _, xd = quant_act(np.asarray(x, np.float32), MODE_BSGEMM)
    return linear_dequant(xd, w_deq)


def dequant_weight(w_bf16_values):
    """Quantise a weight [N, K] with 128x128 fp32 block scales and return
    (q, s, exact float64 dequantised value)."""
    q, s = quant_weight_128x128(np.asarray(w_bf16_values, np.float32))
    return q, s, dequant_block_fp32(q, s, 128, 128)


def attention_block(x, p, k_cache, v_cache, kv_len, n_heads, n_kv_heads, head_dim, eps=RMS_EPS, kv_store=None):
    """First half of a pre-norm block: x + O(attn(qkv(RMSNorm(x)))).

    x        : [B, H] bf16 values
    p        : dict with dequantised 'qkv' [(Hq+2Hkv)D, H], 'o' [H, Hq D] and
               the bf16 RMSNorm weight 'norm_attn' [H]
    k_cache, v_cache : [B, Hkv, slots, D] arrays (the values the cache
               holds), written at kv_len[b] - 1 (the new token) and read over
               [0, kv_len[b])
    kv_store : the values a cache holds for the new bf16 K/V rows [Hkv, D]
               (None: the rows themselves, a bf16 cache; attention.mx_kv_store
               for an MXFP8 cache)
    Returns (x_mid, dict of the intermediates; 'k', 'v' are the bf16 rows).
    """
    x = np.asarray(x, np.float64)
    B = x.shape[0]
    Hq, Hkv, D = n_heads, n_kv_heads, head_dim
    xn = rmsnorm(x, p["norm_attn"], eps)
    qkv = round_bf16(fp8_linear(xn, p["qkv"]))
    q = qkv[:, :Hq * D].reshape(B, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(B, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(B, Hkv, D)
    for b in range(B):
        t = int(kv_len[b]) - 1
        if not 0 <= t < k_cache.shape[2]:
            raise ValueError(f"kv_len[{b}] = {t + 1} outside [1, {k_cache.shape[2]}]")
        k_cache[b, :, t, :] = k[b] if kv_store is None else kv_store(k[b])
        v_cache[b, :, t, :] = v[b] if kv_store is None else kv_store(v[b])
    attn = round_bf16(gqa_decode_attention(q, k_cache, v_cache, kv_len)).reshape(B, Hq * D)
    x_mid = round_bf16(x + fp8_linear(attn, p["o"]))
    return x_mid, {"xn": xn, "q": q, "k": k, "v": v, "attn": attn}


def mlp_block(x_mid, p, eps=RMS_EPS):
    """Second half of a pre-norm block: x_mid + MLP(RMSNorm(x_mid)), with the
    dequantised 'gate', 'up' [I, H], 'down' [H, I] and 'norm_mlp' [H] of p."""
    x_mid = np.asarray(x_mid, np.float64)
    xn2 = rmsnorm(x_mid, p["norm_mlp"], eps)
    y = swiglu_mlp(xn2, p["gate"], p["up"], p["down"], MODE_BSGEMM)["y"]
    return round_bf16(x_mid + y), {"xn2": xn2, "y": y}


def decoder_layer(x, p, k_cache, v_cache, kv_len, n_heads, n_kv_heads, head_dim, eps=RMS_EPS):
    """One pre-norm block at decode: the attention half, then the MLP half.
    Returns (x_out, dict of the intermediates, x_mid included)."""
    x_mid, it = attention_block(x, p, k_cache, v_cache, kv_len, n_heads, n_kv_heads, head_dim, eps)
    out, it2 = mlp_block(x_mid, p, eps)
    return out, {**it, "x_mid": x_mid, **it2}


def embed_sum(tables, codes, add=None):
    """bf16(add + sum_c tables[c][codes[:, c]]) in float64 (codebook order)."""
    codes = np.asarray(codes)
    acc = np.zeros((codes.shape[0], np.asarray(tables[0]).shape[1]), np.float64) if add is None \
        else np.array(add, np.float64)
    for c in range(codes.shape[1]):
        acc = acc + np.asarray(tables[c], np.float64)[codes[:, c]]
    return round_bf16(acc)


def greedy_code(z_normed, head_deq):
    """(logits float64 [B, V], argmax codes with ties to the lowest index)."""
    logits = fp8_linear(z_normed, head_deq)
    return logits, np.argmax(logits, axis=1).astype(np.int32)


def dual_ar_step(model, prev_codes, slow_k, slow_v, kv_len, force=None, slow_kv_store=None):
    """One batched Dual-AR decode step.

    model : dict with
        'slow', 'fast' : lists of layer dicts (see attention_block, mlp_block)
        'slow_norm', 'fast_norm' : bf16 [H] final norm weights
        'embed' : list of C bf16 tables [V, H];  'heads' : list of C
                  dequantised FP8 heads [V, H]
        'n_heads', 'n_kv_heads', 'head_dim', 'eps'
    prev_codes : int [B, C], the previous frame's codes
    slow_k, slow_v : per slow layer, [B, Hkv, slots, D] prefix arrays (the
        caller's copies; row kv_len-1 is overwritten with the new K/V)
    kv_len : int [B], includes this step's token
    force  : optional teacher forcing, a dict with
        'slow_x' : [2L+1][B, H]  the residual stream at every half-block
                   boundary: entry 2l is the input of slow layer l, 2l+1 its
                   stream after the attention half, 2L the last output
        'codes'  : [B, C]        the codes fed onward
        'fast_x' : [C-1][2F+1][B, H] the same for the fast layers, per
                   micro-step
      Each half-block then starts from the forced input instead of the
      oracle's own previous output, and each micro-step embeds the forced code
      (FP8 re-quantisation flips and argmax near-ties cannot compound).
    slow_kv_store : the kv_store of the slow layers' caches (see
      attention_block; slow_k, slow_v then hold the values those caches
      hold); the fast AR's own cache is bf16.
    Returns a dict with slow_x [2L+1], h, logits [C], codes [B, C], fast_x
    [C-1][2F+1] (each entry the oracle's output given its (forced) input), and
    the K/V rows written per layer ('slow_kv', 'fast_kv').
    """
    Hq, Hkv, D = model["n_heads"], model["n_kv_heads"], model["head_dim"]
    eps = model.get("eps", RMS_EPS)
    C = len(model["embed"])
    B = prev_codes.shape[0]
    L, F = len(model["slow"]), len(model["fast"])

    def stream_in(own, forced, i):
        return own[i] if forced is None else np.asarray(forced[i], np.float64)

    def run_layers(xs, forced, layers, ks, vs, lens, kv_out, store=None):
        for l, p in enumerate(layers):
            x_mid, it = attention_block(stream_in(xs, forced, 2 * l), p, ks[l], vs[l], lens, Hq, Hkv, D, eps, store)
            xs.append(x_mid)
            out, _ = mlp_block(stream_in(xs, forced, 2 * l + 1), p, eps)
            xs.append(out)
            kv_out.append((it["k"], it["v"]))

    slow_x = [embed_sum(model["embed"], prev_codes)]
    slow_kv = []
    run_layers(slow_x, None if force is None else force["slow_x"], model["slow"], slow_k, slow_v, kv_len, slow_kv,
               slow_kv_store)
    h = rmsnorm(stream_in(slow_x, None if force is None else force["slow_x"], 2 * L), model["slow_norm"], eps)
    logits = [None] * C
    codes = np.zeros((B, C), np.int32)
    logits[0], codes[:, 0] = greedy_code(h, model["heads"][0])
    fed = codes if force is None else np.asarray(force["codes"], np.int32)

    slots = C - 1
    fk = [np.zeros((B, Hkv, slots, D)) for _ in range(F)]
    fv = [np.zeros((B, Hkv, slots, D)) for _ in range(F)]
    fast_x, fast_kv = [], []
    for p in range(C - 1):
        xs = [embed_sum([model["embed"][p]], fed[:, p:p + 1], add=h if p == 0 else None)]
        kvs = []
        forced = None if force is None else force["fast_x"][p]
        run_layers(xs, forced, model["fast"], fk, fv, np.full(B, p + 1, np.int32), kvs)
        zn = rmsnorm(stream_in(xs, forced, 2 * F), model["fast_norm"], eps)
        logits[p + 1], codes[:, p + 1] = greedy_code(zn, model["heads"][p + 1])
        if force is None:
            fed = codes
        fast_x.append(xs)
        fast_kv.append(kvs)
    return {"slow_x": slow_x, "h": h, "logits": logits, "codes": codes, "fast_x": fast_x,
            "slow_kv": slow_kv, "fast_kv": fast_kv}
