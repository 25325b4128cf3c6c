"""Thin torch-facing wrappers over the C ABI of libfp8step.so.

Each function only checks tensor placement and dtypes, allocates outputs with
torch when the caller does not pass them, and forwards raw device pointers and
sizes to the library on the current HIP stream.  All arithmetic runs in the
HIP kernels.
"""

import math
from dataclasses import dataclass

import torch

from . import _lib

# Quantisation and MLP modes (include/fp8step.h).
Q_ACT_1x128, Q_WGT_128x128, Q_MX_1x32 = 0, 1, 2
MLP_BSGEMM, MLP_MXFP8 = 0, 1
DEV_KVLEN_RANGE, DEV_CODE_RANGE, DEV_PAGE_RANGE = 1, 3, 4
TAP_MLP_X, TAP_STEP_SLOW, TAP_MLP_H = 1, 2, 3
OUT_BF16, OUT_F32 = 0, 1


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fp8step operates on GPU tensors only")


def _bits(t):
    """bf16 tensor -> its storage pointer (the library reads uint16 bits)."""
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected a bfloat16 tensor, got {t.dtype}")
    return t.data_ptr()


def qlinear_quantize(x, mode, q=None, scale=None, k_major=None):
    """Quantise a 2-D bf16 tensor; returns (q uint8, scale).

    Scale tensors: mode 0 -> fp32 [rows, cols/128]; mode 1 -> fp32
    [rows/128, cols/128]; mode 2 -> uint8 [rows, cols/32].  With
    k_major=True (the MX default) the scale tensor is allocated as a K-major
    view (stride (1, rows)).
    """
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if k_major is None:
        k_major = mode == Q_MX_1x32
    if scale is None:
        if mode == Q_ACT_1x128:
            shape, dt = (rows, cols // 128), torch.float32
        elif mode == Q_WGT_128x128:
            shape, dt = (rows // 128, cols // 128), torch.float32
        else:
            shape, dt = (rows, cols // 32), torch.uint8
        if k_major:
            scale = torch.empty((shape[1], shape[0]), dtype=dt, device=x.device).t()
        else:
            scale = torch.empty(shape, dtype=dt, device=x.device)
    _lib.check(_lib.load().qlinear_quantize(
        _bits(x), rows, cols, x.stride(0), mode, q.data_ptr(), q.stride(0),
        scale.data_ptr(), scale.stride(0), scale.stride(1), _stream()))
    return q, scale


@dataclass
class QWeight:
    """An e4m3 weight [N, K] with its block scales (see fp8s_qweight).
    packed: w holds the bytes in the fragment-packed layout of
    fp8s_pack_weight (passed with ld_w = 0)."""
    w: torch.Tensor
    scale: torch.Tensor
    packed: bool = False

    def as_c(self):
        return _lib.QWeightC(self.w.data_ptr(), 0 if self.packed else self.w.stride(0), self.scale.data_ptr(),
                             self.scale.stride(0), self.scale.stride(1))


def pack_weight(qw):
    """Load-time copy of a QWeight into the fragment-packed layout (same
    scales, same results from every consumer)."""
    if qw.packed:
        return qw
    N, K = qw.w.shape
    if int(_lib.load().fp8s_packed_weight_bytes(N, K)) == 0:
        raise ValueError(f"cannot pack a [{N}, {K}] weight (N % 16, K % 128)")
    out = torch.empty((N, K), dtype=torch.uint8, device=qw.w.device)
    _lib.check(_lib.load().fp8s_pack_weight(qw.w.data_ptr(), qw.w.stride(0), N, K, out.data_ptr(), _stream()))
    return QWeight(out, qw.scale, True)


def quantize_weight(w_bf16, mlp_mode):
    """Quantise a bf16 weight for the given MLP path (load-time step)."""
    if mlp_mode == MLP_BSGEMM:
        q, s = qlinear_quantize(w_bf16, Q_WGT_128x128)
    else:
        q, s = qlinear_quantize(w_bf16, Q_MX_1x32, k_major=True)
    return QWeight(q, s)


def mlp_workspace_bytes(M, hidden, inter, mode):
    return int(_lib.load().swiglu_mlp_fp8_workspace_size(M, hidden, inter, mode))


def new_mlp_workspace(M, hidden, inter, mode, device="cuda"):
    """A zero-filled workspace (the library keeps it zeroed between calls)."""
    n = mlp_workspace_bytes(M, hidden, inter, mode)
    if n == 0:
        raise ValueError("unsupported MLP shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def swiglu_mlp_fp8(x, gate, up, down, mode, y=None, workspace=None, err=None):
    """y = SwiGLU MLP of x [M, hidden] bf16 with FP8 weights; returns y bf16."""
    _require_cuda(x)
    if not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous [M, hidden] tensor")
    M, H = x.shape
    I = gate.w.shape[0]
    if y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = new_mlp_workspace(M, H, I, mode, x.device)
    _lib.check(_lib.load().swiglu_mlp_fp8(
        _bits(x), M, H, I, mode, gate.as_c(), up.as_c(), down.as_c(), _bits(y),
        workspace.data_ptr(), workspace.numel(), err.data_ptr() if err is not None else None,
        _stream()))
    return y


def attn_workspace_bytes(B, Hq, D, max_kv_len):
    return int(_lib.load().gqa_decode_attn_workspace_size(B, Hq, D, max_kv_len))


def new_attn_workspace(B, Hq, D, max_kv_len, device="cuda"):
    """A zero-filled attention workspace (its split counters stay zeroed)."""
    return torch.zeros(max(attn_workspace_bytes(B, Hq, D, max_kv_len), 16), dtype=torch.uint8, device=device)


def gqa_decode_attn(q, k_cache, v_cache, kv_len, max_kv_len_hint, softmax_scale=None,
                    out=None, workspace=None, err=None):
    """Decode attention of q [B, Hq, D] over caches [B, Hkv, cap, D] (any
    strides with unit stride along D) for positions < kv_len[b]."""
    _require_cuda(q, k_cache, v_cache, kv_len)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    B, Hq, D = q.shape
    _, Hkv, cap, _ = k_cache.shape
    if k_cache.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    hint = min(int(max_kv_len_hint), cap)
    if workspace is None:
        workspace = new_attn_workspace(B, Hq, D, hint, q.device)
    _lib.check(_lib.load().gqa_decode_attn(
        _bits(q.contiguous()), _bits(k_cache), _bits(v_cache), k_cache.stride(0), k_cache.stride(1),
        k_cache.stride(2), kv_len.data_ptr(), B, Hq, Hkv, D, cap, hint, float(softmax_scale),
        _bits(out), workspace.data_ptr(), workspace.numel(),
        err.data_ptr() if err is not None else None, _stream()))
    return out


@dataclass
class MxKvCache:
    """An MXFP8 KV cache: e4m3 bytes q [B, Hkv, cap, D] and UE8M0 exponents
    e [B, Hkv, cap, D/32] (one per 32 consecutive d)."""
    q: torch.Tensor
    e: torch.Tensor


def quantize_kv_mx(cache_bf16):
    """Quantise a bf16 cache [B, Hkv, cap, D] (contiguous) row by row in 1x32
    groups (qlinear_quantize mode 2, row-major exponents)."""
    if not cache_bf16.is_contiguous():
        raise ValueError("the cache must be contiguous")
    B, Hkv, cap, D = cache_bf16.shape
    rows = cache_bf16.view(B * Hkv * cap, D)
    e = torch.empty((B * Hkv * cap, D // 32), dtype=torch.uint8, device=cache_bf16.device)
    q, e = qlinear_quantize(rows, Q_MX_1x32, scale=e)
    return MxKvCache(q.view(B, Hkv, cap, D), e.view(B, Hkv, cap, D // 32))


def gqa_decode_attn_mxkv(q, k, v, kv_len, max_kv_len_hint, softmax_scale=None,
                         out=None, workspace=None, err=None):
    """Decode attention of q [B, Hq, D] over MXFP8 caches k, v (MxKvCache)."""
    _require_cuda(q, k.q, k.e, v.q, v.e, kv_len)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if k.q.stride() != v.q.stride() or k.e.stride() != v.e.stride() or k.q.shape != v.q.shape:
        raise ValueError("k and v must share shapes and strides")
    B, Hq, D = q.shape
    _, Hkv, cap, _ = k.q.shape
    if k.q.stride(3) != 1 or k.e.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    hint = min(int(max_kv_len_hint), cap)
    if workspace is None:
        workspace = new_attn_workspace(B, Hq, D, hint, q.device)
    _lib.check(_lib.load().gqa_decode_attn_mxkv(
        _bits(q.contiguous()), k.q.data_ptr(), k.e.data_ptr(), v.q.data_ptr(), v.e.data_ptr(),
        k.q.stride(0), k.q.stride(1), k.q.stride(2), k.e.stride(0), k.e.stride(1), k.e.stride(2),
        kv_len.data_ptr(), B, Hq, Hkv, D, cap, hint, float(softmax_scale),
        _bits(out), workspace.data_ptr(), workspace.numel(),
        err.data_ptr() if err is not None else None, _stream()))
    return out


def _check_block_table(block_table, B):
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")


def gqa_decode_attn_paged(q, k_pool, v_pool, block_table, kv_len, max_kv_len_hint, softmax_scale=None,
                          out=None, workspace=None, err=None):
    """Decode attention of q [B, Hq, D] over paged bf16 caches: k_pool,
    v_pool are indexed (page, kv head, slot, d) (any strides with unit stride
    along d; a [pages, slot, head, d] pool is passed as .permute(0, 2, 1, 3));
    position t of sequence b is slot t % P of page block_table[b, t // P]."""
    _require_cuda(q, k_pool, v_pool, block_table, kv_len)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if k_pool.stride() != v_pool.stride() or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must share shape and strides")
    B, Hq, D = q.shape
    n_pages, Hkv, P, _ = k_pool.shape
    if k_pool.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    _check_block_table(block_table, B)
    max_pages = block_table.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    hint = min(int(max_kv_len_hint), max_pages * P)
    if workspace is None:
        workspace = new_attn_workspace(B, Hq, D, hint, q.device)
    _lib.check(_lib.load().gqa_decode_attn_paged(
        _bits(q.contiguous()), _bits(k_pool), _bits(v_pool), k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        n_pages, P, block_table.data_ptr(), block_table.stride(0), max_pages, kv_len.data_ptr(), B, Hq, Hkv, D,
        hint, float(softmax_scale), _bits(out), workspace.data_ptr(), workspace.numel(),
        err.data_ptr() if err is not None else None, _stream()))
    return out


def gqa_decode_attn_paged_mxkv(q, k, v, block_table, kv_len, max_kv_len_hint, softmax_scale=None,
                               out=None, workspace=None, err=None):
    """gqa_decode_attn_paged over MXFP8 page pools k, v (MxKvCache whose q
    is [pages, Hkv, P, D] e4m3 and e [pages, Hkv, P, D/32] UE8M0)."""
    _require_cuda(q, k.q, k.e, v.q, v.e, block_table, kv_len)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if k.q.stride() != v.q.stride() or k.e.stride() != v.e.stride() or k.q.shape != v.q.shape:
        raise ValueError("k and v must share shapes and strides")
    B, Hq, D = q.shape
    n_pages, Hkv, P, _ = k.q.shape
    if k.q.stride(3) != 1 or k.e.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    _check_block_table(block_table, B)
    max_pages = block_table.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    hint = min(int(max_kv_len_hint), max_pages * P)
    if workspace is None:
        workspace = new_attn_workspace(B, Hq, D, hint, q.device)
    _lib.check(_lib.load().gqa_decode_attn_paged_mxkv(
        _bits(q.contiguous()), k.q.data_ptr(), k.e.data_ptr(), v.q.data_ptr(), v.e.data_ptr(),
        k.q.stride(0), k.q.stride(1), k.q.stride(2), k.e.stride(0), k.e.stride(1), k.e.stride(2),
        n_pages, P, block_table.data_ptr(), block_table.stride(0), max_pages, kv_len.data_ptr(), B, Hq, Hkv, D,
        hint, float(softmax_scale), _bits(out), workspace.data_ptr(), workspace.numel(),
        err.data_ptr() if err is not None else None, _stream()))
    return out


def fp8_gemm_mx(qa, ea, qb, eb, c=None):
    """C bf16 [M, N] = dequant(qa, ea) . dequant(qb, eb)^T for MXFP8
    operands: qa uint8 [M, K], ea uint8 [M, K/32] (any strides), qb uint8
    [N, K], eb uint8 [N, K/32]."""
    _require_cuda(qa, ea, qb, eb)
    for t in (qa, ea, qb, eb):
        if t.dtype != torch.uint8 or t.dim() != 2:
            raise TypeError("operands and exponents must be 2-D uint8")
    M, K = qa.shape
    N = qb.shape[0]
    if qb.shape[1] != K or tuple(ea.shape) != (M, K // 32) or tuple(eb.shape) != (N, K // 32):
        raise ValueError("shapes must be qa [M, K], ea [M, K/32], qb [N, K], eb [N, K/32]")
    if qa.stride(1) != 1 or qb.stride(1) != 1:
        raise ValueError("operand rows must be contiguous")
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    _lib.check(_lib.load().fp8_gemm_mx(
        qa.data_ptr(), qa.stride(0), ea.data_ptr(), ea.stride(0), ea.stride(1),
        qb.data_ptr(), qb.stride(0), eb.data_ptr(), eb.stride(0), eb.stride(1),
        M, N, K, _bits(c), c.stride(0), _stream()))
    return c


def extend_attn(q, q_start, k_cache, v_cache, kv_len, max_new_hint, softmax_scale=None, out=None, err=None):
    """Causal attention of new tokens q [total, Hq, D] (sequence b owns rows
    q_start[b] .. q_start[b+1]-1, int32 [B+1] on the device) over caches
    [B, Hkv, cap, D] holding them as the last rows of kv_len[b]."""
    _require_cuda(q, q_start, k_cache, v_cache, kv_len)
    if q_start.dtype != torch.int32 or kv_len.dtype != torch.int32:
        raise TypeError("q_start and kv_len must be int32")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape or k_cache.stride(3) != 1:
        raise ValueError("k_cache and v_cache must share shape and strides, D contiguous")
    total, Hq, D = q.shape
    B, Hkv, cap, _ = k_cache.shape
    if q_start.shape != (B + 1,) or kv_len.shape != (B,):
        raise ValueError("q_start must be [B + 1] and kv_len [B]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _lib.check(_lib.load().extend_attn(
        _bits(q.contiguous()), q_start.data_ptr(), total, _bits(k_cache), _bits(v_cache), k_cache.stride(0),
        k_cache.stride(1), k_cache.stride(2), kv_len.data_ptr(), B, Hq, Hkv, D, cap, int(max_new_hint),
        float(softmax_scale), _bits(out), err.data_ptr() if err is not None else None, _stream()))
    return out


def extend_attn_paged(q, q_start, k_pool, v_pool, block_table, kv_len, max_new_hint, softmax_scale=None, out=None,
                      err=None):
    """extend_attn over paged caches: k_pool, v_pool indexed (page, kv
    head, slot, d) as in gqa_decode_attn_paged."""
    _require_cuda(q, q_start, k_pool, v_pool, block_table, kv_len)
    if q_start.dtype != torch.int32 or kv_len.dtype != torch.int32:
        raise TypeError("q_start and kv_len must be int32")
    if k_pool.stride() != v_pool.stride() or k_pool.shape != v_pool.shape or k_pool.stride(3) != 1:
        raise ValueError("k_pool and v_pool must share shape and strides, D contiguous")
    total, Hq, D = q.shape
    n_pages, Hkv, P, _ = k_pool.shape
    B = kv_len.shape[0]
    _check_block_table(block_table, B)
    if q_start.shape != (B + 1,):
        raise ValueError("q_start must be [B + 1]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _lib.check(_lib.load().extend_attn_paged(
        _bits(q.contiguous()), q_start.data_ptr(), total, _bits(k_pool), _bits(v_pool), k_pool.stride(0),
        k_pool.stride(1), k_pool.stride(2), n_pages, P, block_table.data_ptr(), block_table.stride(0),
        block_table.shape[1], kv_len.data_ptr(), B, Hq, Hkv, D, int(max_new_hint), float(softmax_scale), _bits(out),
        err.data_ptr() if err is not None else None, _stream()))
    return out


@dataclass
class PackedMx:
    """An MXFP8 operand [rows, K] in the packed layout of fp8_pack_mx."""
    data: torch.Tensor
    rows: int
    K: int


def fp8_pack_mx(q, e):
    """Pack codes q uint8 [R, K] and exponents e uint8 [R, K/32] (any
    strides) for fp8_gemm_mx_packed."""
    _require_cuda(q, e)
    R, K = q.shape
    if q.dtype != torch.uint8 or e.dtype != torch.uint8 or tuple(e.shape) != (R, K // 32) or q.stride(1) != 1:
        raise ValueError("need q uint8 [R, K] with contiguous rows and e uint8 [R, K/32]")
    n = int(_lib.load().fp8_mx_packed_bytes(R, K))
    if n == 0:
        raise ValueError("K must be a positive multiple of 128")
    out = torch.empty(n, dtype=torch.uint8, device=q.device)
    _lib.check(_lib.load().fp8_pack_mx(q.data_ptr(), q.stride(0), e.data_ptr(), e.stride(0), e.stride(1), R, K,
                                       out.data_ptr(), n, _stream()))
    return PackedMx(out, R, K)


def fp8_gemm_mx_packed(pa, pb, c=None):
    """C bf16 [M, N] = dequant(A) . dequant(B)^T from packed operands."""
    if pa.K != pb.K:
        raise ValueError("operands must share K")
    M, N, K = pa.rows, pb.rows, pa.K
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=pa.data.device)
    _lib.check(_lib.load().fp8_gemm_mx_packed(pa.data.data_ptr(), pb.data.data_ptr(), M, N, K, _bits(c),
                                              c.stride(0), _stream()))
    return c


def fp8_pack_bs(q, s, rows_per_scale):
    """Pack bsgemm codes q uint8 [R, K] with fp32 scales s (activation:
    [R, K/128], rows_per_scale 1; weight: [R/128, K/128], rows_per_scale
    128; any strides) for fp8_gemm_bs_packed."""
    _require_cuda(q, s)
    R, K = q.shape
    if q.dtype != torch.uint8 or s.dtype != torch.float32 or q.stride(1) != 1:
        raise ValueError("need q uint8 [R, K] with contiguous rows and fp32 scales")
    if tuple(s.shape) != ((R + rows_per_scale - 1) // rows_per_scale, K // 128):
        raise ValueError("scale shape does not match rows_per_scale")
    n = int(_lib.load().fp8_bs_packed_bytes(R, K))
    if n == 0:
        raise ValueError("K must be a positive multiple of 128")
    out = torch.empty(n, dtype=torch.uint8, device=q.device)
    _lib.check(_lib.load().fp8_pack_bs(q.data_ptr(), q.stride(0), s.data_ptr(), s.stride(0), s.stride(1),
                                       int(rows_per_scale), R, K, out.data_ptr(), n, _stream()))
    return PackedMx(out, R, K)


def fp8_gemm_bs_packed(pa, pb, c=None):
    """C bf16 [M, N] from bsgemm operands packed by fp8_pack_bs."""
    if pa.K != pb.K:
        raise ValueError("operands must share K")
    M, N, K = pa.rows, pb.rows, pa.K
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=pa.data.device)
    _lib.check(_lib.load().fp8_gemm_bs_packed(pa.data.data_ptr(), pb.data.data_ptr(), M, N, K, _bits(c),
                                              c.stride(0), _stream()))
    return c


def swiglu_mlp_fp8_large(x, gate_up, down, mode, y=None, workspace=None):
    """y bf16 [M, hidden] = SwiGLU MLP of x bf16 [M, hidden] (any M) with
    packed weights: gate_up = PackedMx of [Wg; Wu] ([2 inter, hidden]), down
    = PackedMx of Wd ([hidden, inter]), both from fp8_pack_bs (mode
    MLP_BSGEMM) or fp8_pack_mx (MLP_MXFP8)."""
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16 [M, hidden] with unit column stride")
    M, H = x.shape
    I = gate_up.rows // 2
    if gate_up.K != H or down.rows != H or down.K != I or gate_up.rows != 2 * I:
        raise ValueError("weights do not match x: gate_up [2 inter, hidden], down [hidden, inter]")
    n = int(_lib.load().swiglu_mlp_fp8_large_workspace_size(M, H, I, mode))
    if n == 0:
        raise ValueError("need M >= 1, hidden and inter multiples of 128, a known mode")
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _lib.check(_lib.load().swiglu_mlp_fp8_large(_bits(x), x.stride(0), M, H, I, mode, gate_up.data.data_ptr(),
                                                down.data.data_ptr(), _bits(y), y.stride(0), workspace.data_ptr(),
                                                workspace.numel(), _stream()))
    return y


def sample_top_k_top_p(logits, uniforms, temperature=0.8, top_k=30, top_p=0.8, codes=None):
    """One token per row of fp32 logits [B, V] (unit stride along V) with
    the caller's uniforms [B] fp32 in [0, 1); returns int32 codes [B]."""
    _require_cuda(logits, uniforms)
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be float32 [B, V] with unit stride along V")
    B, V = logits.shape
    if uniforms.dtype != torch.float32 or uniforms.shape != (B,) or not uniforms.is_contiguous():
        raise ValueError("uniforms must be contiguous float32 [B]")
    if codes is None:
        codes = torch.empty(B, dtype=torch.int32, device=logits.device)
    _lib.check(_lib.load().sample_top_k_top_p(
        logits.data_ptr(), B, V, logits.stride(0), float(temperature), int(top_k), float(top_p),
        uniforms.data_ptr(), codes.data_ptr(), codes.stride(0), _stream()))
    return codes


def prev_tokens_shift_inplace(prev, next_tokens):
    """prev int32 [bs, W, cw] <- its frames 1..W-1 then next_tokens int32
    [bs, cw], in place.  The contract is strict: no dtype conversion, no
    reshaping or broadcasting (a mismatch raises)."""
    _require_cuda(prev, next_tokens)
    if prev.dtype != torch.int32 or next_tokens.dtype != torch.int32:
        raise TypeError("prev and next_tokens must be int32")
    if prev.dim() != 3 or next_tokens.dim() != 2 or tuple(next_tokens.shape) != (prev.shape[0], prev.shape[2]):
        raise ValueError("shapes must be prev [bs, W, cw] and next_tokens [bs, cw]")
    if not prev.is_contiguous() or not next_tokens.is_contiguous():
        raise ValueError("prev and next_tokens must be contiguous")
    bs, W, cw = prev.shape
    _lib.check(_lib.load().prev_tokens_shift_inplace(prev.data_ptr(), next_tokens.data_ptr(), bs, W, cw, _stream()))
    return prev


def _opt_ptr(t):
    return t.data_ptr() if t is not None else None


def qlinear_workspace_bytes(M, N, K):
    return int(_lib.load().qlinear_fp8_workspace_size(M, N, K))


def new_qlinear_workspace(M, N, K, device="cuda"):
    """A zero-filled workspace (the library keeps its control words zeroed)."""
    n = qlinear_workspace_bytes(M, N, K)
    if n == 0:
        raise ValueError("unsupported qlinear shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def qlinear_fp8(x, w, norm_w=None, eps=1e-6, residual=None, out_dtype=OUT_BF16, y=None, workspace=None):
    """y = [residual +] quant(norm(x)) . W^T for x [M, K] bf16 and a bsgemm
    QWeight W [N, K]; y is bf16 or fp32 [M, N]."""
    _require_cuda(x, norm_w, residual)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    N = w.w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device=x.device)
    if workspace is None:
        workspace = new_qlinear_workspace(M, N, K, x.device)
    _lib.check(_lib.load().qlinear_fp8(
        _bits(x), M, K, x.stride(0), _opt_ptr(norm_w), float(eps), w.as_c(), N,
        _opt_ptr(residual), residual.stride(0) if residual is not None else 0, out_dtype,
        y.data_ptr(), y.stride(0), workspace.data_ptr(), workspace.numel(), _stream()))
    return y


def qkv_proj_kv_append(x, w_qkv, Hq, Hkv, D, k_cache, v_cache, kv_len, norm_w=None, eps=1e-6,
                       q_out=None, workspace=None, err=None):
    """q = query part of quant(norm(x)) . W_qkv^T ([M, Hq*D] bf16); the key and
    value parts are written into the caches [B, Hkv, cap, D] at kv_len - 1."""
    _require_cuda(x, k_cache, v_cache, kv_len)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape or k_cache.stride(3) != 1:
        raise ValueError("k_cache and v_cache must share shape and strides, D contiguous")
    M, K = x.shape
    N = (Hq + 2 * Hkv) * D
    if q_out is None:
        q_out = torch.empty((M, Hq * D), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = new_qlinear_workspace(M, N, K, x.device)
    _lib.check(_lib.load().qkv_proj_kv_append(
        _bits(x), M, K, x.stride(0), _opt_ptr(norm_w), float(eps), w_qkv.as_c(), Hq, Hkv, D, _bits(q_out),
        _bits(k_cache), _bits(v_cache), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        kv_len.data_ptr(), k_cache.shape[2], workspace.data_ptr(), workspace.numel(), _opt_ptr(err), _stream()))
    return q_out


def qkv_proj_kv_append_mxkv(x, w_qkv, Hq, Hkv, D, k, v, kv_len, norm_w=None, eps=1e-6,
                            q_out=None, workspace=None, err=None):
    """qkv_proj_kv_append into MXFP8 caches k, v (MxKvCache): the new rows'
    e4m3 bytes and UE8M0 exponents are written at kv_len - 1."""
    _require_cuda(x, k.q, k.e, v.q, v.e, kv_len)
    if k.q.stride() != v.q.stride() or k.e.stride() != v.e.stride() or k.q.shape != v.q.shape:
        raise ValueError("k and v must share shapes and strides")
    if k.q.stride(3) != 1 or k.e.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    M, K = x.shape
    N = (Hq + 2 * Hkv) * D
    if q_out is None:
        q_out = torch.empty((M, Hq * D), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = new_qlinear_workspace(M, N, K, x.device)
    _lib.check(_lib.load().qkv_proj_kv_append_mxkv(
        _bits(x), M, K, x.stride(0), _opt_ptr(norm_w), float(eps), w_qkv.as_c(), Hq, Hkv, D, _bits(q_out),
        k.q.data_ptr(), k.e.data_ptr(), v.q.data_ptr(), v.e.data_ptr(),
        k.q.stride(0), k.q.stride(1), k.q.stride(2), k.e.stride(0), k.e.stride(1), k.e.stride(2),
        kv_len.data_ptr(), k.q.shape[2], workspace.data_ptr(), workspace.numel(), _opt_ptr(err), _stream()))
    return q_out


def embed_sum(tables, codes, add=None, out=None, err=None):
    """out[b] = bf16(add[b] + sum_c tables[c][codes[b, c]]); codes int32 [B, >= len(tables)]."""
    import ctypes
    _require_cuda(codes, add, *tables)
    B = codes.shape[0]
    V, H = tables[0].shape
    if out is None:
        out = torch.empty((B, H), dtype=torch.bfloat16, device=codes.device)
    arr = (ctypes.c_void_p * len(tables))(*[t.data_ptr() for t in tables])
    _lib.check(_lib.load().embed_sum_bf16(arr, len(tables), V, H, codes.data_ptr(), codes.stride(0), B,
                                          _opt_ptr(add), _bits(out), _opt_ptr(err), _stream()))
    return out


def argmax_rows(logits, codes=None):
    """Greedy codes of fp32 logits [B, N] (ties to the lowest index); int32 [B]
    or into column 0 of the given int32 codes view."""
    _require_cuda(logits)
    B, N = logits.shape
    if codes is None:
        codes = torch.empty((B, 1), dtype=torch.int32, device=logits.device)
    _lib.check(_lib.load().argmax_rows_f32(logits.data_ptr(), B, N, logits.stride(0), codes.data_ptr(),
                                           codes.stride(0), _stream()))
    return codes


class DualArModel:
    """Device weights of a Dual-AR model and the C structs that describe them.

    slow / fast: lists of dicts with QWeight 'qkv', 'o', 'gate', 'up', 'down'
    and bf16 tensors 'norm_attn', 'norm_mlp'; embed: list of bf16 [V, H];
    heads: list of QWeight [V, H]."""

    def __init__(self, slow, fast, slow_norm, fast_norm, embed, heads, n_heads, n_kv_heads, head_dim,
                 inter, rms_eps=1e-6):
        import ctypes
        self.slow, self.fast, self.embed, self.heads = slow, fast, embed, heads
        self.slow_norm, self.fast_norm = slow_norm, fast_norm
        V, H = embed[0].shape

        def block(d):
            return _lib.BlockWeightsC(d["qkv"].as_c(), d["o"].as_c(), d["gate"].as_c(), d["up"].as_c(),
                                      d["down"].as_c(), d["norm_attn"].data_ptr(), d["norm_mlp"].data_ptr())
        self._slow_c = (_lib.BlockWeightsC * max(len(slow), 1))(*[block(d) for d in slow])
        self._fast_c = (_lib.BlockWeightsC * max(len(fast), 1))(*[block(d) for d in fast])
        self._embed_c = (ctypes.c_void_p * len(embed))(*[t.data_ptr() for t in embed])
        self._heads_c = (_lib.QWeightC * len(heads))(*[h.as_c() for h in heads])
        self.c = _lib.DualArModelC(H, inter, V, n_heads, n_kv_heads, head_dim, len(embed), len(slow), len(fast),
                                   float(rms_eps), self._slow_c, self._fast_c, slow_norm.data_ptr(),
                                   fast_norm.data_ptr(), self._embed_c, self._heads_c)

    def workspace_bytes(self, B, max_kv_len_hint):
        import ctypes
        return int(_lib.load().dual_ar_decode_step_workspace_size(ctypes.byref(self.c), B, max_kv_len_hint))

    def new_workspace(self, B, max_kv_len_hint, device="cuda"):
        n = self.workspace_bytes(B, max_kv_len_hint)
        if n == 0:
            raise ValueError("unsupported Dual-AR configuration")
        return torch.zeros(n, dtype=torch.uint8, device=device)


KV_BF16, KV_MXFP8 = 0, 1


class KvState:
    """Per-slow-layer K/V caches and kv_len: bf16 tensors [B, Hkv, cap, D],
    or MxKvCache objects (MXFP8), all with shared shapes and strides."""

    def __init__(self, k_caches, v_caches, kv_len, max_kv_len_hint, live_rows=None):
        """live_rows: optional device int32 [1]; rows b >= live_rows[0] of a
        step are padding and append no K/V (see fp8s_kv_state)."""
        import ctypes
        mx = isinstance(k_caches[0], MxKvCache)
        if any(isinstance(t, MxKvCache) != mx for t in list(k_caches) + list(v_caches)):
            raise TypeError("the caches must be all bf16 tensors or all MxKvCache")
        k0 = k_caches[0].q if mx else k_caches[0]
        e0 = k_caches[0].e if mx else None
        for t in list(k_caches) + list(v_caches):
            tq = t.q if mx else t
            if tq.stride() != k0.stride() or tq.shape != k0.shape or tq.stride(3) != 1:
                raise ValueError("all caches must share shape and strides, D contiguous")
            if mx and (t.e.stride() != e0.stride() or t.e.stride(3) != 1):
                raise ValueError("all exponent caches must share strides, D/32 contiguous")
        if kv_len.dtype != torch.int32:
            raise TypeError("kv_len must be int32")
        if live_rows is not None and (live_rows.dtype != torch.int32 or not live_rows.is_cuda):
            raise TypeError("live_rows must be an int32 device tensor")
        self.k_caches, self.v_caches, self.kv_len, self.live_rows = k_caches, v_caches, kv_len, live_rows
        self.max_kv_len_hint = int(max_kv_len_hint)
        self.mx = mx
        ptrs = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
        if mx:
            self._kq, self._ke = ptrs([t.q for t in k_caches]), ptrs([t.e for t in k_caches])
            self._vq, self._ve = ptrs([t.q for t in v_caches]), ptrs([t.e for t in v_caches])
            self.c = _lib.KvStateC(None, None, k0.stride(0), k0.stride(1), k0.stride(2), k0.shape[2],
                                   kv_len.data_ptr(), int(max_kv_len_hint),
                                   live_rows.data_ptr() if live_rows is not None else None, KV_MXFP8,
                                   self._kq, self._ke, self._vq, self._ve, e0.stride(0), e0.stride(1), e0.stride(2))
        else:
            self._k, self._v = ptrs(k_caches), ptrs(v_caches)
            self.c = _lib.KvStateC(self._k, self._v, k0.stride(0), k0.stride(1), k0.stride(2), k0.shape[2],
                                   kv_len.data_ptr(), int(max_kv_len_hint),
                                   live_rows.data_ptr() if live_rows is not None else None, KV_BF16)

    def with_live_rows(self, live_rows):
        """The same caches and kv_len with a padding-row count (device int32 [1])."""
        return KvState(self.k_caches, self.v_caches, self.kv_len, self.max_kv_len_hint, live_rows)


def dual_ar_decode_step(model, kv, prev_codes, codes=None, slow_taps=None, fast_taps=None, logits_tap=None,
                        workspace=None, err=None):
    """One batched Dual-AR decode step; returns the frame's codes int32 [B, C]."""
    import ctypes
    _require_cuda(prev_codes, slow_taps, fast_taps, logits_tap)
    B, C = prev_codes.shape
    if codes is None:
        codes = torch.empty((B, C), dtype=torch.int32, device=prev_codes.device)
    if workspace is None:
        workspace = model.new_workspace(B, kv.c.max_kv_len_hint, prev_codes.device)
    _lib.check(_lib.load().dual_ar_decode_step(
        ctypes.byref(model.c), B, prev_codes.data_ptr(), ctypes.byref(kv.c), codes.data_ptr(),
        _opt_ptr(slow_taps), _opt_ptr(fast_taps), _opt_ptr(logits_tap), workspace.data_ptr(), workspace.numel(),
        _opt_ptr(err), _stream()))
    return codes


def profile_start(max_records=200000):
    """Start recording per-kernel HIP events inside the library."""
    _lib.check(_lib.load().fp8s_profile_start(int(max_records)))


def profile_stop():
    """Stop recording; returns [(kernel name, milliseconds), ...] in launch order."""
    import ctypes
    lib = _lib.load()
    n = lib.fp8s_profile_stop()
    if n < 0:
        _lib.check(n)
    out = []
    buf = ctypes.create_string_buffer(64)
    ms = ctypes.c_float()
    for i in range(n):
        _lib.check(lib.fp8s_profile_record(i, buf, 64, ctypes.byref(ms)))
        out.append((buf.value.decode(), float(ms.value)))
    return out


def set_debug_tap(kind, buf):
    """Point debug tap `kind` (TAP_MLP_X, TAP_STEP_SLOW, TAP_MLP_H) at a uint8 device
    tensor, or switch it off with None (see fp8s_set_debug_tap)."""
    if buf is None:
        _lib.check(_lib.load().fp8s_set_debug_tap(int(kind), None, 0))
    else:
        _require_cuda(buf)
        _lib.check(_lib.load().fp8s_set_debug_tap(int(kind), buf.data_ptr(), buf.numel() * buf.element_size()))
