#!/usr/bin/env python3
"""Decode-step hot-path benchmark on one MI355X (gfx950).

One step = one full batched Dual-AR decode step (dual_ar_decode_step): the
slow AR's 36 Qwen3-4B-sized layers (RMSNorm, FP8 QKV projection with the K/V
append, GQA decode attention over the active prefix, FP8 output projection,
FP8 SwiGLU MLP) for a batch of 64 sequences with kv_len ~ U{234..4096} in
caches of 32768 slots, then the 4-layer fast AR over the remaining 9
codebooks of 4096 entries and the 10 greedy codebook heads.  tokens/s =
64 / step time (each step decodes one frame per sequence).  Every input is
resident in HBM before timing starts; the 36 layers' 3.6 GB of FP8 weights
are all distinct and the KV prefixes (about 568 MB per layer) rotate over 4
physical cache sets, so the 256 MB Infinity Cache cannot serve repeats.

Prints ONE JSON line.  Extra keys: the per-kernel table of the step (time,
algorithmic bytes, HBM rate), the M sweep of the MLP alone (bsgemm and
MXFP8, M = 1..128) and the batch / context sweep of attention alone, and the
CPU oracle timed on the host cores on a bounded sample of the step.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-step tokens/s + achieved HBM GB/s (% of peak) for MLP & attn, M=1..128"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
ROTATE_BYTES = 512 << 20         # sweeps rotate at least this many touched bytes (> the 256 MB last-level cache)
H, I = 2560, 9728                # Qwen3-4B MLP
HQ, HKV, D, CAP = 32, 8, 128, 32768


def _wscale_bytes(n, k, mode):
    return (n // 128) * (k // 128) * 4 if mode == 0 else n * k // 32


def _ascale_bytes(m, k, mode):
    return m * (k // 128) * 4 if mode == 0 else m * k // 32


def mlp_bytes(M, mode):
    """Algorithmic bytes of one MLP call: FP8 weights + scales, x in, y out."""
    return 3 * H * I + 3 * _wscale_bytes(I, H, mode) + 2 * M * H * 2


def kernel_bytes(name, M, mode, kv_len=None, B=None):
    """Algorithmic bytes per launch of each library kernel (what the step it
    implements must read and write; workspace traffic that a fused design
    would avoid, such as split partials, is not counted)."""
    w_gu = 2 * I * H + 2 * _wscale_bytes(I, H, mode)
    w_dn = H * I + _wscale_bytes(H, I, mode)
    if name == "mlp_gu_small":
        return w_gu + M * H * 2 + 2 * M * I * 4
    if name == "mlp_gu":
        return w_gu + M * H + _ascale_bytes(M, H, mode) + 2 * M * I * 4
    if name == "mlp_down_small_fused":
        return w_dn + 2 * M * I * 4 + M * H * 2
    if name in ("mlp_down_small", "mlp_down"):
        return w_dn + M * I + _ascale_bytes(M, I, mode) + M * H * 2
    if name == "mlp_xq":
        return M * H * 2 + M * H + _ascale_bytes(M, H, mode)
    if name == "mlp_hq":
        return 2 * M * I * 4 + M * I + _ascale_bytes(M, I, mode)
    if name in ("attn_split", "attn_split_paged"):      # paged: the block table (4 B per page) is not counted
        return int(np.sum(kv_len.astype(np.int64))) * HKV * D * 2 * 2 + B * HQ * D * 2 + 4 * B
    if name in ("attn_split_mx", "attn_split_mx_paged"):
        return int(np.sum(kv_len.astype(np.int64))) * HKV * (D + D // 32) * 2 + B * HQ * D * 2 + 4 * B
    if name == "attn_merge":
        return B * HQ * D * 2 + 4 * B
    return 0


def attn_bytes(kv_len, B, mx=False):
    row = D + D // 32 if mx else 2 * D         # bytes per cached row: e4m3 + UE8M0, or bf16
    return int(np.sum(kv_len.astype(np.int64))) * HKV * row * 2 + 2 * B * HQ * D * 2 + 4 * B


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Workload:
    """Rotating sets of GPU-resident weights, activations and KV caches."""

    def __init__(self, torch, ops, B, M, mode, n_sets, kv_len, with_attn=True, with_mlp=True, mx_kv=False,
                 page=0, packed=False, cap=CAP):
        self.torch, self.ops = torch, ops
        self.mx_kv = mx_kv
        self.page = page
        self.B, self.M, self.mode = B, M, mode
        self.sets = []
        g = torch.Generator(device="cuda")
        for s in range(n_sets):
            g.manual_seed(1000 * (2 if mode else 1) + 17 * s + M)
            st = {}
            if with_mlp:
                ws = []
                for shape in ((I, H), (I, H), (H, I)):
                    wb = (torch.randn(shape, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
                    qw = ops.quantize_weight(wb, mode)
                    ws.append(ops.pack_weight(qw) if packed else qw)
                    del wb, qw
                st["w"] = ws
                x = torch.randn((M, H), generator=g, device="cuda")
                if mode == ops.MLP_MXFP8:
                    mask = torch.rand((M, H), generator=g, device="cuda") < 0.01
                    x = torch.where(mask, x * 50.0, x)
                st["x"] = x.to(torch.bfloat16)
                st["y"] = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
                st["ws"] = ops.new_mlp_workspace(M, H, I, mode)
            if with_attn:
                Lmax = int(kv_len.max())
                kc = torch.empty((B, HKV, cap, D), dtype=torch.bfloat16, device="cuda")
                vc = torch.empty((B, HKV, cap, D), dtype=torch.bfloat16, device="cuda")
                kc[:, :, :Lmax] = torch.randn((B, HKV, Lmax, D), generator=g, device="cuda").to(torch.bfloat16)
                vc[:, :, :Lmax] = torch.randn((B, HKV, Lmax, D), generator=g, device="cuda").to(torch.bfloat16)
                if page:                                # the prefixes on shuffled pages of a pool
                    mp = (Lmax + page - 1) // page
                    from fp8_transformer_step_amd import inputs
                    table = inputs.page_table(inputs.W_ATTN, B, mp, B * mp, extra=s)
                    idx = torch.from_numpy(table.reshape(-1).astype(np.int64)).cuda()
                    pools = []
                    for c in (kc, vc):
                        pool = torch.empty((B * mp, HKV, page, D), dtype=torch.bfloat16, device="cuda")
                        pool[idx] = c[:, :, :mp * page].reshape(B, HKV, mp, page, D).transpose(1, 2).reshape(
                            B * mp, HKV, page, D)
                        pools.append(pool)
                    del kc, vc
                    kc, vc = pools
                    st["bt"] = torch.from_numpy(table).cuda()
                if mx_kv:                               # MXFP8 caches, quantised from the bf16 ones
                    kc, vc = ops.quantize_kv_mx(kc), ops.quantize_kv_mx(vc)
                st["k"], st["v"] = kc, vc
                st["q"] = torch.randn((B, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
                st["o"] = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")
                st["kv"] = torch.from_numpy(kv_len).cuda()
                st["aws"] = ops.new_attn_workspace(B, HQ, D, Lmax)
                st["hint"] = Lmax
            self.sets.append(st)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def mlp(self, s):
        st = self.sets[s]
        self.ops.swiglu_mlp_fp8(st["x"], *st["w"], self.mode, y=st["y"], workspace=st["ws"], err=self.err)

    def attn(self, s):
        st = self.sets[s]
        if self.page:
            fn = self.ops.gqa_decode_attn_paged_mxkv if self.mx_kv else self.ops.gqa_decode_attn_paged
            fn(st["q"], st["k"], st["v"], st["bt"], st["kv"], st["hint"], out=st["o"], workspace=st["aws"],
               err=self.err)
            return
        fn = self.ops.gqa_decode_attn_mxkv if self.mx_kv else self.ops.gqa_decode_attn
        fn(st["q"], st["k"], st["v"], st["kv"], st["hint"], out=st["o"], workspace=st["aws"], err=self.err)


def time_parts(torch, ops, wl, parts, steps, warmup, graph=False):
    """Two timed regions of `steps` steps each (every step calls every part
    once on a rotating set), bracketed by synchronisation and HIP events:
      1. clean: gives ms per step (the headline);
      2. per kernel: the library records a HIP event pair around every kernel
         it launches, on the launch stream (the events add small gaps between
         launches, so this pass is not used for the headline).
    graph: a third region replays the `steps` steps captured once into a HIP
    graph (the same kernels on the same sets, without the host's launch gaps:
    a call of a few tens of microseconds can otherwise wait for the host to
    enqueue it).
    Returns (ms per step, wall ms per step, {kernel: [ms, ...]}[, graph ms
    per step])."""
    n = len(wl.sets)
    for i in range(warmup):
        for p in parts:
            p(i % n)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        for p in parts:
            p(i % n)
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    ms_step = t0.elapsed_time(t1) / steps
    ops.profile_start(steps * len(parts) * 8 + 64)
    for i in range(steps):
        for p in parts:
            p(i % n)
    torch.cuda.synchronize()
    recs = ops.profile_stop()
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    if not graph:
        return ms_step, wall, per
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for p in parts:
            p(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            for p in parts:
                p(i % n)
    g.replay()
    torch.cuda.synchronize()
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / steps
    del g
    return ms_step, wall, per, ms_graph


def pmc_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed profiler summary
    (FETCH_SIZE and WRITE_SIZE runs of this bench, scaled by a copy of known
    size), or None when there is none or any kernel source changed since it
    was taken."""
    from fp8_transformer_step_amd import profiling
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    rec = d.get("kernels", {}).get(kernel)
    if not rec or d.get("sources_sha256") != profiling.sources_sha256():
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def kernel_table(per, steps, M, mode, kv_len=None, B=None):
    """{kernel: {launches per step, mean us, GB/s, frac of peak}}."""
    out = {}
    for name, v in per.items():
        us = float(np.mean(v)) * 1e3
        nb = kernel_bytes(name, M, mode, kv_len, B)
        gbs = nb / (us * 1e-6) / 1e9 if us > 0 else 0.0
        out[name] = {"per_step": len(v) / steps, "us": us, "bytes": nb, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS}
    return out


def step_launch_plan(cfg, kv_len, mx=False):
    """(library kernel name, algorithmic bytes) of every launch of one
    dual_ar_decode_step, in launch order.  Algorithmic bytes are what the
    operation must move: weights and their scales, the activations it reads
    and writes, the K/V prefix; workspace traffic of split partials and the
    L2-resident re-reads of a row for its RMS are not counted.
    mx: the slow layers' caches are MXFP8 (D e4m3 bytes and D/32 exponents
    per position and KV head, read by attn_split_mx and appended as such)."""
    c = cfg
    B, H, I, V, C = c.batch, c.hidden, c.inter, c.codebook_size, c.n_codebooks
    A, NQKV, KVD = c.n_heads * c.head_dim, (c.n_heads + 2 * c.n_kv_heads) * c.head_dim, c.n_kv_heads * c.head_dim

    def ws(n, k):
        return (n // 128) * (k // 128) * 4

    def asc(k):
        return B * (k // 128) * 4

    def act_quant(name, K, norm):
        return (name, B * K * 2 + (K * 2 if norm else 0) + B * K + asc(K))

    # the MLP: M <= 16 forms h in the down GEMM's prologue from g and u,
    # M > 16 quantises it in a launch of its own
    mlp_tail = ([("mlp_down_small_fused", H * I + ws(H, I) + 2 * B * I * 4)] if B <= 16 else
                [("mlp_hq", 2 * B * I * 4 + B * I + asc(I)), ("mlp_down", H * I + ws(H, I) + B * I + asc(I))])

    # the attention quantises its output into the output projection's operand
    # itself when each KV head's query group spans whole 128-column groups
    fused = (c.n_heads // c.n_kv_heads) * c.head_dim % 128 == 0
    oq = B * A + asc(A) if fused else 0

    # the row finisher: residual (+ deferred partials) -> residual stream out,
    # RMSNorm, 1x128 quantisation of the next projection's operand
    def finish(with_residual):
        return ("row_finish", B * H * 2 + (B * H * 2 if with_residual else 0) + H * 2 + B * H + asc(H))

    # bytes a K/V row of one KV head takes in a cache: bf16, or e4m3 + UE8M0
    row_mx = c.head_dim + c.head_dim // 32

    def block(kv_bytes, single, mx_kv=False):
        attn = ([("attn_single", kv_bytes + 2 * B * A * 2 + 4 * B + oq)] if single else
                [("attn_split_mx" if mx_kv else "attn_split", kv_bytes + B * A * 2 + 4 * B),
                 ("attn_merge", B * A * 2 + 4 * B + oq)])
        qkv_out = B * A * 2 + (B * 2 * c.n_kv_heads * row_mx if mx_kv else B * 2 * KVD * 2)
        return [("qlinear", NQKV * H + ws(NQKV, H) + B * H + asc(H) + qkv_out)] + attn + (
                [] if fused else [act_quant("ql_act_quant", A, False)]) + [
                ("qlinear", H * A + ws(H, A) + B * A + asc(A)),
                finish(True),
                ("mlp_gu", 2 * I * H + 2 * ws(I, H) + B * H + asc(H) + 2 * B * I * 4)] + mlp_tail + [
                finish(True)]

    def head():
        return [("qlinear", V * H + ws(V, H) + B * H + asc(H) + B * V * 4)]

    # embedding rows straight into the finisher: rows gathered (+ the added
    # row), x written, norm weight, operand; the slow input reads the codes
    # and fills the fast AR's kv_len table, a fast micro-step takes its code
    # as the argmax of the previous head's logits
    operand = B * H * 2 + H * 2 + B * H + asc(H)
    out = [("embed_finish", B * C * H * 2 + 4 * B * C + (C - 1) * B * 4 + operand)]
    slow_kv = int(np.sum(kv_len, dtype=np.int64)) * (c.n_kv_heads * row_mx * 2 if mx else KVD * 2 * 2)
    # the slow AR's prefixes are split over chunks and merged; the fast AR's
    # few-slot caches (bf16 either way) are one chunk, written by the split
    # kernel itself
    for _ in range(c.n_slow_layers):
        out += block(slow_kv, False, mx)
    out += head()
    for p in range(C - 1):
        out.append(("embed_finish", B * V * 4 + 4 * B + B * H * 2 * (2 if p == 0 else 1) + operand))
        for _ in range(c.n_fast_layers):
            out += block((p + 1) * B * KVD * 2 * 2, True)
        out += head()
    out.append(("argmax", B * V * 4 + 4 * B))
    return out


def time_step(torch, ops, dm, kv, prev, steps, warmup, workspace, err):
    """ms per step over `steps` back-to-back steps (HIP events on the stream,
    bracketed by synchronisation), the wall clock per step, the library's
    per-launch records of a second pass of `steps` steps, and the ms of each
    step of a third pass with an event between steps."""
    codes = torch.empty(prev.shape, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        ops.dual_ar_decode_step(dm, kv, prev, codes=codes, workspace=workspace, err=err)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        ops.dual_ar_decode_step(dm, kv, prev, codes=codes, workspace=workspace, err=err)
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    ms = t0.elapsed_time(t1) / steps
    ops.profile_start(steps * 4096 + 64)
    for _ in range(steps):
        ops.dual_ar_decode_step(dm, kv, prev, codes=codes, workspace=workspace, err=err)
    torch.cuda.synchronize()
    recs = ops.profile_stop()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        ops.dual_ar_decode_step(dm, kv, prev, codes=codes, workspace=workspace, err=err)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ms, wall, recs, per_step


def bucket_curve(torch, dm, kv, max_b):
    """The step replayed from one captured graph per batch bucket (the same
    model and caches, the first B rows): ms per step and tokens/s per
    bucket, 10 replays each after 2."""
    from fp8_transformer_step_amd import graphs
    sg = graphs.StepGraphs(dm, kv, buckets=[b for b in (1, 8, 16, 24, 32, 48, 64) if b <= max_b])
    out = {}
    for B in sg.buckets:
        for _ in range(2):
            sg.replay(B)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            sg.replay(B)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / 10
        out[f"B={B}"] = {"ms_per_step": ms, "tokens/s": B / (ms * 1e-3)}
        log(f"graph bucket B={B}: {ms:.3f} ms/step, {B / (ms * 1e-3):.0f} tokens/s")
    if int(sg.err.item()) != 0:
        raise SystemExit(f"device error flag {int(sg.err.item())} in the bucket graphs")
    del sg
    return out


PEAK_FP8_TFLOPS = 5000.0                # dense FP8 MFMA peak of the chip


def prefill_gemm_sweep(torch, ops):
    """fp8_gemm_mx_packed (and the row-major fp8_gemm_mx, and the bsgemm
    fp8_gemm_bs_packed) on the pages' square shapes and on the MLP's prefill
    shapes at M = 4096, operands
    quantised from seeded bf16 and packed outside the timed loop (packing
    the activation is timed on its own): TFLOP/s and fraction of the dense
    FP8 peak."""
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    out = {}
    for M, N, K in ((1024, 1024, 1024), (4096, 4096, 4096), (8192, 8192, 8192), (16384, 16384, 16384),
                    (4096, 19456, 2560), (4096, 2560, 9728)):
        a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
        b = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        qa, ea = ops.qlinear_quantize(a, ops.Q_MX_1x32)
        qb, eb = ops.qlinear_quantize(b, ops.Q_MX_1x32)
        qa_bs, sa_bs = ops.qlinear_quantize(a, ops.Q_ACT_1x128)
        qb_bs, sb_bs = ops.qlinear_quantize(b, ops.Q_WGT_128x128)
        del a, b
        pa, pb = ops.fp8_pack_mx(qa, ea), ops.fp8_pack_mx(qb, eb)
        pa_bs, pb_bs = ops.fp8_pack_bs(qa_bs, sa_bs, 1), ops.fp8_pack_bs(qb_bs, sb_bs, 128)
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        n = max(3, min(30, int(2e12 / (2 * M * N * K))))
        res = {}
        for name, fn in (("packed", lambda: ops.fp8_gemm_mx_packed(pa, pb, c)),
                         ("row_major", lambda: ops.fp8_gemm_mx(qa, ea, qb, eb, c)),
                         ("bsgemm_packed", lambda: ops.fp8_gemm_bs_packed(pa_bs, pb_bs, c)),
                         ("pack_activation", lambda: ops.fp8_pack_mx(qa, ea))):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(n):
                fn()
            t1.record()
            torch.cuda.synchronize()
            us = t0.elapsed_time(t1) / n * 1e3
            res[name] = {"us": us}
            if name != "pack_activation":
                tf = 2 * M * N * K / (us * 1e-6) / 1e12
                res[name].update({"TFLOP/s": tf, "frac": tf / PEAK_FP8_TFLOPS})
        out[f"{M}x{N}x{K}"] = res
        log(f"gemm mx {M}x{N}x{K}: packed {res['packed']['us']:.1f} us {res['packed']['TFLOP/s']:.0f} TFLOP/s, "
            f"row-major {res['row_major']['TFLOP/s']:.0f}, bsgemm packed {res['bsgemm_packed']['TFLOP/s']:.0f}, "
            f"pack A {res['pack_activation']['us']:.1f} us")
        del qa, ea, qb, eb, pa, pb, qa_bs, sa_bs, qb_bs, sb_bs, pa_bs, pb_bs, c
        torch.cuda.empty_cache()
    return out


def mlp_large_sweep(torch, ops):
    """swiglu_mlp_fp8_large at the Qwen3-4B MLP shape (hidden 2560, inter
    9728) for M from 128 to 4096, bsgemm and MXFP8, weights packed outside
    the timed loop: whole-call time (four kernels: quantise x, gate/up GEMM,
    SwiGLU + quantise h, down GEMM), TFLOP/s over 6 M hidden inter flop, and
    the decode kernel swiglu_mlp_fp8 at M = 128 beside it."""
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    H, I = 2560, 9728
    out = {}
    for mode, name in ((ops.MLP_BSGEMM, "bsgemm"), (ops.MLP_MXFP8, "mxfp8")):
        ws = [(torch.randn(shape, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
              for shape in ((I, H), (I, H), (H, I))]
        qw = [ops.quantize_weight(w, mode) for w in ws]
        qgu, sgu = torch.cat([qw[0].w, qw[1].w]), torch.cat([qw[0].scale, qw[1].scale])
        if mode == ops.MLP_BSGEMM:
            pgu, pd = ops.fp8_pack_bs(qgu, sgu, 128), ops.fp8_pack_bs(qw[2].w, qw[2].scale, 128)
        else:
            pgu, pd = ops.fp8_pack_mx(qgu, sgu), ops.fp8_pack_mx(qw[2].w, qw[2].scale)
        del ws, qgu, sgu
        res = {}
        for M in (128, 512, 1024, 2048, 4096):
            x = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)
            y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
            wsp = torch.empty(int(ops._lib.load().swiglu_mlp_fp8_large_workspace_size(M, H, I, mode)),
                              dtype=torch.uint8, device="cuda")
            fns = [("large", lambda: ops.swiglu_mlp_fp8_large(x, pgu, pd, mode, y=y, workspace=wsp))]
            if M == 128:
                dws = torch.zeros(int(ops._lib.load().swiglu_mlp_fp8_workspace_size(M, H, I, mode)),
                                  dtype=torch.uint8, device="cuda")
                fns.append(("decode_kernel", lambda: ops.swiglu_mlp_fp8(x, *qw, mode, y=y, workspace=dws)))
            for kind, fn in fns:
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                n = 20
                t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t0.record()
                for _ in range(n):
                    fn()
                t1.record()
                torch.cuda.synchronize()
                us = t0.elapsed_time(t1) / n * 1e3
                tf = 6 * M * H * I / (us * 1e-6) / 1e12
                res[f"M={M}" + ("" if kind == "large" else ",decode_kernel")] = {
                    "us": us, "TFLOP/s": tf, "frac": tf / PEAK_FP8_TFLOPS}
                log(f"mlp large {name} M={M} {kind}: {us:.1f} us {tf:.0f} TFLOP/s")
            del x, y, wsp
        out[name] = res
        del qw, pgu, pd
        torch.cuda.empty_cache()
    return out


def extend_attn_sweep(torch, ops):
    """extend_attn (prefill / extend) at 32/8/128: a 4096-token prefill, 16
    sequences extending by 256 tokens after 1792 cached, 64 sequences by 16
    after 4080.  TFLOP/s counts 4 Hq D flop per (new token, attended
    position) against the bf16 MFMA peak; GB/s counts the K/V prefix once."""
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    Hq, Hkv, D = 32, 8, 128
    out = {}
    for B, T, L in ((1, 4096, 4096), (16, 256, 2048), (64, 16, 4096)):
        k = torch.randn((B, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((B, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
        q = torch.randn((B * T, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
        qs = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
        kv = torch.full((B,), L, dtype=torch.int32, device="cuda")
        o = torch.empty_like(q)
        for _ in range(3):
            ops.extend_attn(q, qs, k, v, kv, T, out=o)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            ops.extend_attn(q, qs, k, v, kv, T, out=o)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / 10 * 1e3
        pos = B * (T * (L - T) + T * (T + 1) // 2)
        tf = 4 * Hq * D * pos / (us * 1e-6) / 1e12
        gbs = B * L * Hkv * D * 2 * 2 / (us * 1e-6) / 1e9
        out[f"B={B},new={T},kv_len={L}"] = {"us": us, "TFLOP/s": tf, "frac_bf16_mfma": tf / 2500.0, "GB/s": gbs}
        log(f"extend B={B} new={T} kv_len={L}: {us:.1f} us {tf:.0f} TFLOP/s {gbs:.0f} GB/s")
        del k, v, q, o
        torch.cuda.empty_cache()
    return out


def token_selection_timing(torch, ops):
    """sample_top_k_top_p on the heads' logits (B = 64, V = 4096, the pages'
    temperature 0.8 / top_p 0.8 / top_k 30, and top_k off) and the window
    shift (64 x 16 frames x 10 codebooks): us per call over 50 calls."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    logits = torch.randn((64, 4096), generator=g, device="cuda") * 3.0
    u = torch.rand(64, generator=g, device="cuda")
    codes = torch.empty(64, dtype=torch.int32, device="cuda")
    prev = torch.zeros((64, 16, 10), dtype=torch.int32, device="cuda")
    nxt = torch.ones((64, 10), dtype=torch.int32, device="cuda")
    out = {}
    cases = {"sample B=64,V=4096,T=0.8,top_k=30,top_p=0.8":
             lambda: ops.sample_top_k_top_p(logits, u, 0.8, 30, 0.8, codes=codes),
             "sample B=64,V=4096,T=1.0,top_k=0,top_p=0.95":
             lambda: ops.sample_top_k_top_p(logits, u, 1.0, 0, 0.95, codes=codes),
             "window_shift bs=64,W=16,cw=10": lambda: ops.prev_tokens_shift_inplace(prev, nxt)}
    for name, fn in cases.items():
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(50):
            fn()
        t1.record()
        torch.cuda.synchronize()
        out[name] = {"us": t0.elapsed_time(t1) / 50 * 1e3}
        log(f"{name}: {out[name]['us']:.1f} us")
    return out


def percentiles(v):
    """p10, median and p90 of a list of per-step times."""
    a = np.asarray(v, np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.median(a)), "p90": float(np.percentile(a, 90))}


def mlp_sweep(torch, ops, inputs, n_sets):
    """The MLP alone at M in {1, 8, 32, 64, 128}, bsgemm and MXFP8, with
    row-major and fragment-packed weights, on rotating weight sets."""
    kv_len = inputs.kv_lengths(inputs.W_ATTN, 64, 234, 400)
    sweep = {}
    for mode, key, packed in ((ops.MLP_BSGEMM, "mlp_bsgemm", False), (ops.MLP_MXFP8, "mlp_mxfp8", False),
                              (ops.MLP_BSGEMM, "mlp_bsgemm_packed", True), (ops.MLP_MXFP8, "mlp_mxfp8_packed", True)):
        sweep[key] = {}
        # the bsgemm workload's M list, and the MXFP8 workload's "1..128"
        for M in ((1, 8, 32, 64, 128) if mode == ops.MLP_BSGEMM else (1, 2, 4, 8, 16, 32, 64, 96, 128)):
            w = Workload(torch, ops, 1, M, mode, n_sets, kv_len, with_attn=False, packed=packed)
            te, _, per, t = time_parts(torch, ops, w, [w.mlp], 20, 5, graph=True)
            gb = mlp_bytes(M, mode) / (t * 1e-3) / 1e9
            sweep[key][M] = {"us": t * 1e3, "us_eager": te * 1e3, "tokens/s": M / (t * 1e-3), "GB/s": gb,
                             "frac": gb / PEAK_HBM_GBS,
                             "rotated_bytes": n_sets * mlp_bytes(M, mode), "kernels": kernel_table(per, 20, M, mode)}
            log(f"{key} M={M}: {t * 1e3:.1f} us {gb:.0f} GB/s  " +
                " ".join(f"{k}={v['us']:.1f}" for k, v in sweep[key][M]["kernels"].items()))
            del w
            torch.cuda.empty_cache()
    return sweep


def time_step_graph(torch, ops, dm, kv, prev, steps, warmup, workspace, err):
    """ms per step when the step is captured once into a HIP graph and
    replayed (every kernel of every step still runs; the host launches one
    graph per step instead of each kernel)."""
    codes = torch.empty(prev.shape, dtype=torch.int32, device="cuda")

    def step():
        ops.dual_ar_decode_step(dm, kv, prev, codes=codes, workspace=workspace, err=err)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    del graph
    return t0.elapsed_time(t1) / steps


def step_kernel_table(recs, plan, steps):
    """{kernel: launches per step, us per step, us per launch, algorithmic
    bytes per step and per launch, GB/s, fraction of peak}; checks that the
    recorded launch sequence is the planned one."""
    n = len(plan)
    if len(recs) != n * steps:
        raise SystemExit(f"recorded {len(recs)} launches, expected {n} x {steps}")
    tab = {}
    for i, (name, ms) in enumerate(recs):
        pname, nbytes = plan[i % n]
        if name != pname:
            raise SystemExit(f"launch {i % n} of the step is {name}, expected {pname}")
        t = tab.setdefault(name, {"launches": 0, "us": 0.0, "bytes": 0})
        t["launches"] += 1
        t["us"] += ms * 1e3
        t["bytes"] += nbytes
    out = {}
    for name, t in tab.items():
        us, nb, k = t["us"] / steps, t["bytes"] / steps, t["launches"] / steps
        gbs = nb / (us * 1e-6) / 1e9 if us > 0 else 0.0
        out[name] = {"per_step": k, "us_per_step": us, "us_per_launch": us / k, "bytes_per_step": int(nb),
                     "bytes_per_launch": nb / k, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS}
    return out


def mxfp8_kv_step(torch, model, host, dm, prev, workspace, args):
    """The same step with the slow layers' caches in MXFP8 (the pages'
    MXFP8 decode attention; the K/V append quantises the new rows): ms per
    step, tokens/s and the per-kernel table.  A second configuration, not
    the headline: the caches hold the same prefixes quantised in 1x32 groups."""
    from fp8_transformer_step_amd import ops
    cfg = host.cfg
    log("bench: the step over MXFP8 KV caches")
    kv, _, _ = model.device_kv(host, mx=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms, wall, recs, per_step = time_step(torch, ops, dm, kv, prev, args.steps, args.warmup, workspace, err)
    if int(err.item()) != 0:
        raise SystemExit(f"device error flag {int(err.item())} (MXFP8 KV step)")
    plan = step_launch_plan(cfg, host.kv_len, mx=True)
    ktab = step_kernel_table(recs, plan, args.steps)
    step_bytes = int(sum(v["bytes_per_step"] for v in ktab.values()))
    log(f"step (MXFP8 KV) {ms:.3f} ms ({cfg.batch / (ms * 1e-3):.0f} tokens/s); attn_split_mx "
        f"{ktab['attn_split_mx']['us_per_launch']:.1f} us per layer")
    del kv
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "tokens/s": cfg.batch / (ms * 1e-3), "wall_ms_per_step": wall,
            "ms_per_step_dist": percentiles(per_step), "launches_per_step": len(plan),
            "step_hbm": {"bytes_per_step": step_bytes, "GB/s": step_bytes / (ms * 1e-3) / 1e9,
                         "frac": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "kernels": ktab}


def stream_ceiling(torch, ops):
    """What one launch can stream: fp8s_stream_read over the byte counts of
    the MLP (all weights, gate/up, down), the QKV projection and one attention
    call at B = 64, kv U[234, 4096], each on buffers rotating >= 512 MB."""
    lib = ops._lib.load()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    H, I = 2560, 9728
    sizes = {"mlp_weights": 3 * H * I, "mlp_gate_up": 2 * H * I, "mlp_down": H * I, "qkv_proj": 6144 * H,
             "attn_b64_kv4096": 533291008}
    out = {}
    for name, nb in sizes.items():
        nb = nb // 2048 * 2048
        n_bufs = max(2, -(-ROTATE_BYTES // nb))
        bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(n_bufs)]
        st = torch.cuda.current_stream().cuda_stream

        def run(i):
            ops._lib.check(lib.fp8s_stream_read(bufs[i % n_bufs].data_ptr(), nb, sink.data_ptr(), st))
        for i in range(2 * n_bufs):
            run(i)
        torch.cuda.synchronize()
        n = max(40, 2 * n_bufs)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(n):
            run(i)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / n * 1e3
        gbs = nb / (us * 1e-6) / 1e9
        out[name] = {"bytes": nb, "us": us, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS, "rotated_bytes": n_bufs * nb}
        log(f"stream_read {name}: {nb / 1e6:.1f} MB in {us:.2f} us = {gbs:.0f} GB/s "
            f"({100 * gbs / PEAK_HBM_GBS:.1f}% of peak)")
        del bufs
        torch.cuda.empty_cache()
    return out


def _blas_threads():
    try:
        import threadpoolctl
        return max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        return 1


def cpu_baseline(host):
    """The oracle as it stands, on the host cores, on a bounded sample of the
    step: one slow layer (full batch, the first cache set's prefixes), one
    fast-AR layer at its first micro-step and one codebook head, with their
    weights dequantised outside the timing, scaled to a full step (36 slow
    + 9 x 4 fast layer evaluations + 10 heads); the median of 3 samples."""
    import oracle
    f32 = __import__("fp8_transformer_step_amd.inputs", fromlist=["x"]).bf16_bits_to_f32
    blas = _blas_threads()
    c = host.cfg

    def block(d):
        p = {k: oracle.dequant_weight(f32(d[k]))[2] for k in ("qkv", "o", "gate", "up", "down")}
        p["norm_attn"], p["norm_mlp"] = f32(d["norm_attn"]), f32(d["norm_mlp"])
        return p
    ps, pf = block(host.slow[0]), block(host.fast[0])
    head = oracle.dequant_weight(f32(host.heads[1]))[2]
    Lmax = int(host.kv_len.max())
    k = np.zeros((c.batch, c.n_kv_heads, Lmax, c.head_dim), np.float32)
    v = np.zeros_like(k)
    for b in range(c.batch):
        kp, vp = host.kv_prefix(0, b)
        k[b, :, :kp.shape[1]], v[b, :, :vp.shape[1]] = f32(kp), f32(vp)
    L, F, C = c.n_slow_layers, c.n_fast_layers, c.n_codebooks
    samples = []
    for _ in range(3):
        fk = np.zeros((c.batch, c.n_kv_heads, c.n_codebooks - 1, c.head_dim))
        fv = np.zeros_like(fk)
        t0 = time.perf_counter()
        x = oracle.embed_sum([f32(t) for t in host.embed], host.prev_codes)
        t1 = time.perf_counter()
        x1, _ = oracle.decoder_layer(x, ps, k.copy(), v.copy(), host.kv_len, c.n_heads, c.n_kv_heads, c.head_dim,
                                     c.rms_eps)
        t2 = time.perf_counter()
        z, _ = oracle.decoder_layer(x1, pf, fk, fv, np.ones(c.batch, np.int32), c.n_heads, c.n_kv_heads,
                                    c.head_dim, c.rms_eps)
        t3 = time.perf_counter()
        oracle.greedy_code(oracle.rmsnorm(z, f32(host.fast_norm)), head)
        t4 = time.perf_counter()
        est = (t1 - t0) + L * (t2 - t1) + (C - 1) * F * (t3 - t2) + C * (t4 - t3)
        samples.append((est, t2 - t1, t3 - t2, t4 - t3))
    est, ts, tf, th = sorted(samples)[1]
    return {"value": c.batch / est, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"median of 3: one slow layer ({ts:.2f} s), one fast layer ({tf:.2f} s) and one head "
                      f"({th:.2f} s) at batch {c.batch}, float64 NumPy, weights dequantised outside the "
                      f"timing, scaled to a full step of {L} + {(C - 1) * F} layer evaluations and {C} heads "
                      f"= {est:.1f} s (samples {', '.join(f'{s[0]:.1f}' for s in samples)} s); host affinity "
                      f"{len(os.sched_getaffinity(0))} cores, {blas} BLAS threads"}


def config_cpu_baselines():
    """The oracle on the other headline configurations, median of 3 timed
    calls each (inputs and dequantised weights prepared outside the timing):
    the Qwen3-4B-shaped MLP at M = 64 on the bsgemm and MXFP8 paths, and
    decode attention at B = 64, kv U[234, 400] and U[234, 4096]."""
    import oracle
    from oracle import attention as oattn, fp8 as ofp8, mlp as omlp
    from fp8_transformer_step_amd import inputs
    f32 = inputs.bf16_bits_to_f32
    blas, cores = _blas_threads(), len(os.sched_getaffinity(0))
    out = {}

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1], ts

    H, I, M = 2560, 9728, 64
    for wl, mode, key in ((inputs.W_BSGEMM, omlp.MODE_BSGEMM, "C2_mlp_bsgemm_M64"),
                          (inputs.W_MXFP8, omlp.MODE_MXFP8, "C3_mlp_mxfp8_M64")):
        deq = []
        for wb in inputs.mlp_weights(wl, H, I):
            w32 = f32(wb)
            if mode == omlp.MODE_BSGEMM:
                q, s = ofp8.quant_weight_128x128(w32)
                deq.append(ofp8.dequant_block_fp32(q, s, 128, 128))
            else:
                q, s = ofp8.quant_mx_1x32(w32)
                deq.append(ofp8.dequant_mx_1x32(q, s))
        x = f32(inputs.mlp_activations(wl, M, H))
        t, ts = med3(lambda: omlp.swiglu_mlp(x, *deq, mode))
        out[key] = {"value": M / t, "unit": "tokens/s", "us_per_call": t * 1e6, "cores": cores,
                    "blas_threads": int(blas), "kind": "oracle", "samples_s": ts}
        del deq
    for hi in (400, 4096):
        B = 64
        kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, hi, extra=B + hi)
        qb, kb, vb = inputs.attention_prefix(inputs.W_ATTN, B, HQ, HKV, D, int(kv.max()), extra=B + hi)
        q, k, v = f32(qb), f32(kb), f32(vb)
        t, ts = med3(lambda: oattn.gqa_decode_attention(q, k, v, kv))
        out[f"C4_attn_B64_kv_U[234,{hi}]"] = {"value": B / t, "unit": "tokens/s", "us_per_call": t * 1e6,
                                              "cores": cores, "blas_threads": int(blas), "kind": "oracle",
                                              "samples_s": ts}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sets", type=int, default=8,
                    help="rotating weight sets of the MLP sweep (8 x 74.7 MB); the attention sweeps rotate "
                         "at least 512 MB of touched cache bytes on their own")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--mlp-only", action="store_true",
                    help="only the MLP at M in {1, 8, 32, 64, 128} (both paths), for counter runs; prints that "
                         "sweep as JSON")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only time fp8s_stream_read over the byte counts of the decode kernels (>= 512 MB "
                         "rotation); prints that table as JSON")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (3x) so that profiler byte counters can be "
                         "scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is single-GPU; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_transformer_step_amd import inputs, model, ops

    torch.cuda.set_device(0)
    if args.stream_ceiling:
        print(json.dumps({"stream_ceiling": stream_ceiling(torch, ops)}), flush=True)
        return
    if args.mlp_only:
        print(json.dumps({"mlp_sweep": mlp_sweep(torch, ops, inputs, args.sets)}), flush=True)
        return
    cfg = model.FULL
    log("bench: generating the seeded model and caches")
    host = model.HostModel(cfg)
    dm = model.device_model(host)
    kv, _, _ = model.device_kv(host)
    prev = torch.from_numpy(host.prev_codes).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    workspace = dm.new_workspace(cfg.batch, kv.c.max_kv_len_hint)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps after {args.warmup} warm-up steps")
    ms_step, wall, recs, per_step = time_step(torch, ops, dm, kv, prev, args.steps, args.warmup, workspace, err)
    ms_graph = time_step_graph(torch, ops, dm, kv, prev, args.steps, args.warmup, workspace, err)
    log(f"step as a replayed HIP graph: {ms_graph:.3f} ms (eager {ms_step:.3f} ms)")
    if int(err.item()) != 0:
        raise SystemExit(f"device error flag {int(err.item())}")
    plan = step_launch_plan(cfg, host.kv_len)
    ktab = step_kernel_table(recs, plan, args.steps)
    B = cfg.batch
    log(f"step {ms_step:.3f} ms ({B / (ms_step * 1e-3):.0f} tokens/s), {len(plan)} launches")
    for k, v in sorted(ktab.items(), key=lambda kv_: -kv_[1]["us_per_step"]):
        log(f"  {k:16s} {v['per_step']:5.0f} x {v['us_per_launch']:7.1f} us = {v['us_per_step']:8.1f} us/step "
            f"{v['GB/s']:6.0f} GB/s ({100 * v['frac']:.1f}% of HBM peak)")
    dom_name, dom = max(ktab.items(), key=lambda kv_: kv_[1]["us_per_step"])
    groups = {"attention": ("attn_",), "mlp": ("mlp_",), "projections": ("ql_act_quant", "qlinear")}
    parts = {}
    for gname, prefixes in groups.items():
        us = sum(v["us_per_step"] for k, v in ktab.items() if k.startswith(prefixes))
        nb = sum(v["bytes_per_step"] for k, v in ktab.items() if k.startswith(prefixes))
        gbs = nb / (us * 1e-6) / 1e9
        parts[gname] = {"us_per_step": us, "bytes_per_step": nb, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS}
    traffic = pmc_traffic(dom_name)
    step_bytes = int(sum(v["bytes_per_step"] for v in ktab.values()))
    log(f"step algorithmic bytes {step_bytes / 1e9:.2f} GB: {step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s "
        f"({100 * step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS:.1f}% of HBM peak over the whole step)")
    result = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 GEMMs (128x128 block / 1x128 group fp32 scales), bf16 activations and attention, "
                 "fp32 accumulate",
        "data": "synthetic: seeded random-init weights N(0,0.02) (windows of one seeded pool), K/V prefixes "
                "N(0,1), random previous codes; no trained weights or datasets",
        "config": {"workload": "full batched Dual-AR decode step: 36 slow layers (hidden 2560, intermediate "
                               "9728, 32/8 heads of dim 128) + 4-layer fast AR over 10 codebooks of 4096, "
                               "batch 64, kv_len U[234,4096] in 32768-slot caches (4 physical K/V sets)",
                   "batch": B, "hidden": cfg.hidden, "intermediate": cfg.inter,
                   "heads": [cfg.n_heads, cfg.n_kv_heads, cfg.head_dim], "cache": cfg.cap,
                   "slow_layers": cfg.n_slow_layers, "fast_layers": cfg.n_fast_layers,
                   "codebooks": [cfg.n_codebooks, cfg.codebook_size], "kv_len": [cfg.kv_lo, cfg.kv_hi]},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": dom["GB/s"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": dom["frac"], "traffic": traffic,
                     "algorithmic_bytes": dom["bytes_per_launch"], "launch_us": dom["us_per_launch"],
                     "launches_per_step": dom["per_step"]},
        "parts": parts,
        "launches_per_step": len(plan),
        "step_hbm": {"bytes_per_step": step_bytes, "GB/s": step_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "kernels": ktab,
        "wall_ms_per_step": wall,
        "ms_per_step_eager": ms_step,
        "ms_per_step_graph": ms_graph,
        "ms_per_step_dist": percentiles(per_step),
    }
    if not args.no_sweep:
        result["step_buckets"] = bucket_curve(torch, dm, kv, B)
    del kv
    torch.cuda.empty_cache()
    result["step_mxfp8_kv"] = mxfp8_kv_step(torch, model, host, dm, prev, workspace, args)
    del dm, workspace, prev
    torch.cuda.empty_cache()

    if not args.no_sweep:
        sweep = mlp_sweep(torch, ops, inputs, args.sets) | {"attn": {}, "attn_mxkv": {}, "attn_paged": {}}
        for Bs, lo, hi, mx, page in ((1, 234, 400, False, 0), (16, 234, 400, False, 0), (64, 234, 400, False, 0),
                                     (64, 234, 4096, False, 0), (64, 234, 8192, False, 0),
                                     (64, 1024, 1024, False, 0), (64, 2048, 2048, False, 0),
                                     (64, 4096, 4096, False, 0), (64, 8192, 8192, False, 0),
                                     (64, 234, 4096, True, 0), (64, 234, 8192, True, 0),
                                     (64, 234, 4096, False, 16), (64, 234, 4096, True, 16)):
            kv = inputs.kv_lengths(inputs.W_ATTN, Bs, lo, hi, extra=Bs + hi)
            # rotate >= 512 MB of the bytes a call touches (more than the 256 MB
            # last-level cache); short prefixes get 512-slot caches so that
            # many sets fit
            n_sets = max(2, min(1024, -(-ROTATE_BYTES // attn_bytes(kv, Bs, mx))))
            w = Workload(torch, ops, Bs, 1, 0, n_sets, kv, with_mlp=False, mx_kv=mx, page=page,
                         cap=CAP if hi > 400 else 512)
            te, _, per, t = time_parts(torch, ops, w, [w.attn], 20, 5, graph=True)
            gb = attn_bytes(kv, Bs, mx) / (t * 1e-3) / 1e9
            key = f"B={Bs},kv=" + (f"{lo}" if lo == hi else f"U[{lo},{hi}]") + (
                f",page={page},{'mxfp8' if mx else 'bf16'}" if page else "")
            sweep["attn_paged" if page else "attn_mxkv" if mx else "attn"][key] = {
                "us": t * 1e3, "us_eager": te * 1e3, "tokens/s": Bs / (t * 1e-3), "GB/s": gb,
                "frac": gb / PEAK_HBM_GBS, "rotated_bytes": n_sets * attn_bytes(kv, Bs, mx),
                "kernels": kernel_table(per, 20, 1, 0, kv, Bs)}
            log(f"attn{' mxkv' if mx else ''}{f' paged {page}' if page else ''} B={Bs} kv {lo}..{hi}: "
                f"{t * 1e3:.1f} us {gb:.0f} GB/s")
            del w
            torch.cuda.empty_cache()
        sweep["sampling"] = token_selection_timing(torch, ops)
        sweep["gemm_mx_prefill"] = prefill_gemm_sweep(torch, ops)
        sweep["extend_attn"] = extend_attn_sweep(torch, ops)
        sweep["mlp_large"] = mlp_large_sweep(torch, ops)
        result["sweep"] = sweep

    if args.copy_calibration:
        # a plain elementwise copy kernel: reads 512 MiB, writes 512 MiB
        src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": 512 << 20, "write": 512 << 20}
        del src, dst

    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(host)
        if not args.no_sweep:
            result["cpu_baselines_other_configs"] = config_cpu_baselines()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
