"""Grouped-query decode attention over the active prefix of a KV cache.

Test infrastructure only (see the package header).

Follows the page "Fish Speech KV Cache 推理优化记录" (Fish Speech KV-cache
optimisation notes):
  * section 4 -- the cache is pre-allocated at full capacity (32768 slots in
    the page's S2-Pro setup), 32 query heads share 8 KV heads, head dim 128;
  * section 5 -- keep the capacity, read only K[:, :, :kv_len] and
    V[:, :, :kv_len]; the KV heads are expanded with repeat_interleave by
    n_head // n_kv_head along the head axis, so query head h reads KV head
    h // G; attention is PyTorch scaled_dot_product_attention with the mask
    narrowed to the prefix, i.e. softmax(q k^T / sqrt(D)) v over t < kv_len;
  * section 5, table of kv_len: prefill T, first decode T + 1, i-th decode
    (from 0) T + i + 1 -- the new token's K/V is already in the cache when the
    decode query attends, so the query sees every position in [0, kv_len).

The loop below never touches cache positions t >= kv_len[b].

The MXFP8-cache variant (gqa_decode_attention_mxkv) is the pages' FP8/MX
decode attention (page "How We Made Our Text-to-Speech API Free", sections
"What's Open Source" and "FP8 Quantization Strategy"): each cache row is held
as e4m3 codes with one OCP UE8M0 exponent per 32 consecutive d, and the
attention is the one above over the dequantised rows.

The paged variants (gqa_decode_attention_paged, ..._paged_mxkv) are the
pages' paged decode attention (same section "What's Open Source"): the cache
rows live in a pool of fixed-size pages, and position t of sequence b is slot
t % P of page block_table[b][t // P].  The pages give no page size or pool
layout; the pool here is [pages, Hkv, P, D] and the attention is the one
above over the rows the table names.

The extend / prefill variant (extend_attention) is the pages' prefill and
paged-prefill ("extend") attention (page "How We Made Our Text-to-Speech API
Free", section "What's Open Source"; the KV-cache page's section 5 table:
prefill writes T positions, kv_len = T): the T new tokens of a sequence are
the last T of its kv_len cached positions, and the new token at position p
attends causally to positions 0 .. p.  Prefill is T = kv_len.

Pins (tests/test_oracle_attention.py): kv_len = 1 returns v_0; q = 0 returns
the mean of the V prefix; equality with an explicit np.repeat expansion of the
heads; torch's float64 scaled_dot_product_attention on the expanded heads;
active-prefix equals full-cache-plus-mask within rtol 1e-5 / atol 1e-6 (the
tolerance of the page's section 7 test); the kv_len schedule of section 5.
MXFP8 variant: on caches built from MX-representable rows (so that the OCP
rule gives back the codes and exponents they were built from) it equals the
plain attention over those rows, and kv_len = 1 returns the dequantised v_0.
Paged variants: a contiguous cache scattered over shuffled pages gives the
contiguous result exactly; pages the table does not name (NaN-filled) never
enter; kv_len = 1 returns slot 0 of the first named page; a brute-force
scalar loop on a tiny pool; an out-of-pool page id is refused.
Extend: one new token per sequence equals the decode attention exactly; a
prefill equals torch's float64 causal scaled_dot_product_attention on the
repeat_interleave'd heads; an extend equals the last rows of the prefill of
the whole sequence exactly; a brute-force scalar loop on a tiny case; cache
positions at or past kv_len (NaN-filled) never enter.
"""

import numpy as np

from . import fp8


def kv_len_schedule(prompt_len, decode_index=None):
    """kv_len at prefill (decode_index None) or at the i-th decode (from 0)."""
    if decode_index is None:
        return prompt_len
    return prompt_len + decode_index + 1


def gqa_decode_attention(q, k_cache, v_cache, kv_len, scale=None):
    """Decode attention for one query token per sequence.

    q        : [B, Hq, D]
    k_cache  : [B, Hkv, cap, D]   (only t < kv_len[b] is read)
    v_cache  : [B, Hkv, cap, D]
    kv_len   : [B] ints in [1, cap]
    scale    : softmax scale, default 1/sqrt(D)
    Returns float64 [B, Hq, D].
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        L = int(kv_len[b])
        if not 1 <= L <= k_cache.shape[2]:
            raise ValueError(f"kv_len[{b}] = {L} outside [1, cap]")
        for h in range(Hq):
            kvh = h // G
            K = np.asarray(k_cache[b, kvh, :L], np.float64)
            V = np.asarray(v_cache[b, kvh, :L], np.float64)
            s = (K @ np.asarray(q[b, h], np.float64)) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h] = p @ V
    return out


def dequant_mx_rows(codes, exps):
    """Exact float64 values of MX rows: codes [..., D] uint8 (OCP e4m3) and
    exps [..., D/32] uint8 (UE8M0, one per 32 consecutive entries)."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    flat = fp8.dequant_mx_1x32(codes.reshape(-1, D), np.asarray(exps).reshape(-1, D // 32))
    return flat.reshape(codes.shape)


def mx_kv_store(rows):
    """The values an MXFP8 KV cache holds for bf16 rows [..., D]: each row
    quantised in 1x32 groups with UE8M0 shared exponents (OCP MX, the MXFP8
    attention variant of "How We Made Our Text-to-Speech API Free", "What's
    Open Source", and its "FP8 Quantization Strategy" groups), then
    dequantised exactly."""
    rows = np.asarray(rows, np.float64)
    D = rows.shape[-1]
    q, e = fp8.quant_mx_1x32(rows.reshape(-1, D))
    return fp8.dequant_mx_1x32(q, e).reshape(rows.shape)


def gqa_decode_attention_mxkv(q, k_codes, k_exps, v_codes, v_exps, kv_len, scale=None):
    """gqa_decode_attention over MXFP8 caches: k_codes, v_codes [B, Hkv, T, D]
    e4m3 bytes, k_exps, v_exps [B, Hkv, T, D/32] UE8M0 bytes.  Only rows
    t < kv_len[b] enter the result (the dequantisation is elementwise)."""
    k = dequant_mx_rows(k_codes, k_exps)
    v = dequant_mx_rows(v_codes, v_exps)
    return gqa_decode_attention(q, k, v, kv_len, scale)


def gather_paged(pool, block_table, kv_len, page_size):
    """The contiguous cache [B, Hkv, max(kv_len), ...] that a paged pool
    [pages, Hkv, P, ...] describes: row t < kv_len[b] of sequence b is slot
    t % P of page block_table[b][t // P].  Rows past kv_len[b] stay zero; no
    other page is read.  A named page outside the pool raises ValueError."""
    pool = np.asarray(pool)
    P = int(page_size)
    if pool.shape[2] != P:
        raise ValueError("pool slot axis must equal page_size")
    B = len(kv_len)
    Lmax = int(max(int(x) for x in kv_len))
    out = np.zeros((B, pool.shape[1], Lmax) + pool.shape[3:], pool.dtype)
    for b in range(B):
        L = int(kv_len[b])
        for i in range((L + P - 1) // P):
            pg = int(block_table[b][i])
            if not 0 <= pg < pool.shape[0]:
                raise ValueError(f"block_table[{b}][{i}] = {pg} outside the pool")
            n = min(P, L - i * P)
            out[b, :, i * P:i * P + n] = pool[pg, :, :n]
    return out


def gqa_decode_attention_paged(q, k_pool, v_pool, block_table, kv_len, page_size, scale=None):
    """gqa_decode_attention over paged caches k_pool, v_pool [pages, Hkv, P, D]."""
    k = gather_paged(k_pool, block_table, kv_len, page_size)
    v = gather_paged(v_pool, block_table, kv_len, page_size)
    return gqa_decode_attention(q, k, v, kv_len, scale)


def gqa_decode_attention_paged_mxkv(q, k_codes, k_exps, v_codes, v_exps, block_table, kv_len, page_size,
                                    scale=None):
    """gqa_decode_attention_mxkv over paged MXFP8 pools: codes [pages, Hkv,
    P, D], exponents [pages, Hkv, P, D/32]."""
    g = lambda pool: gather_paged(pool, block_table, kv_len, page_size)
    return gqa_decode_attention_mxkv(q, g(k_codes), g(k_exps), g(v_codes), g(v_exps), kv_len, scale)

def extend_attention(q, k_cache, v_cache, q_start, kv_len, scale=None):
    """Causal attention of the new tokens of every sequence over its cache.

    q        : [total, Hq, D]; sequence b owns rows q_start[b] .. q_start[b+1]-1,
               T_b = q_start[b+1] - q_start[b] new tokens (T_b may be 0)
    k_cache  : [B, Hkv, cap, D]; the new tokens are the last T_b of the
    v_cache    kv_len[b] valid positions (only t < kv_len[b] is read)
    Token t of sequence b sits at position p = kv_len[b] - T_b + t and
    attends to positions 0 .. p.  Returns float64 [total, Hq, D].
    """
    q = np.asarray(q)
    total, Hq, D = q.shape
    B, Hkv = k_cache.shape[0], k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((total, Hq, D), np.float64)
    for b in range(B):
        q0, q1 = int(q_start[b]), int(q_start[b + 1])
        T, L = q1 - q0, int(kv_len[b])
        if not 0 <= T <= L <= k_cache.shape[2]:
            raise ValueError(f"sequence {b}: need 0 <= T <= kv_len <= cap")
        for t in range(T):
            p = L - T + t
            for h in range(Hq):
                kvh = h // G
                K = np.asarray(k_cache[b, kvh, :p + 1], np.float64)
                V = np.asarray(v_cache[b, kvh, :p + 1], np.float64)
                s = (K @ np.asarray(q[q0 + t, h], np.float64)) * scale
                w = np.exp(s - s.max())
                w /= w.sum()
                out[q0 + t, h] = w @ V
    return out
