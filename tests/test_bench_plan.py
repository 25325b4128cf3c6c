"""The benchmark's host-side launch plan of one decode step (CPU only): the
(kernel, algorithmic bytes) list that the roofline figures are computed from.
It must follow the step's launch chain at each batch size (the MLP forms h in
the down GEMM's prologue up to 16 rows and in a launch of its own above), and
its byte counts must be the closed forms of what each launch moves."""

import numpy as np

import bench
from fp8_transformer_step_amd import model, profiling


def _plan(B, mx=False, kv=2165):
    cfg = model.scaled(model.FULL, batch=B)
    return cfg, bench.step_launch_plan(cfg, np.full(B, kv, np.int32), mx=mx)


def _count(plan, name):
    return sum(1 for n, _ in plan if n == name)


def test_b64_chain_and_launch_count():
    cfg, plan = _plan(64)
    L, F, C = cfg.n_slow_layers, cfg.n_fast_layers, cfg.n_codebooks
    evals = L + (C - 1) * F                    # layer evaluations per step
    assert _count(plan, "mlp_gu") == evals
    assert _count(plan, "mlp_hq") == evals
    assert _count(plan, "mlp_down") == evals
    assert _count(plan, "mlp_down_small_fused") == 0
    assert _count(plan, "attn_split") == L and _count(plan, "attn_merge") == L
    assert _count(plan, "attn_single") == (C - 1) * F
    assert _count(plan, "qlinear") == 2 * evals + C   # QKV and O per layer, one head per codebook
    assert _count(plan, "row_finish") == 2 * evals
    assert _count(plan, "embed_finish") == C and _count(plan, "argmax") == 1
    assert len(plan) == 633


def test_small_batch_forms_h_in_the_down_prologue():
    for B in (1, 8, 16):
        cfg, plan = _plan(B)
        evals = cfg.n_slow_layers + (cfg.n_codebooks - 1) * cfg.n_fast_layers
        assert _count(plan, "mlp_hq") == 0 and _count(plan, "mlp_down") == 0
        assert _count(plan, "mlp_down_small_fused") == evals
        assert len(plan) == 633 - evals
    _, plan = _plan(17)
    assert _count(plan, "mlp_hq") > 0


def test_byte_counts_are_the_closed_forms():
    B, kv = 64, 2165
    cfg, plan = _plan(B, kv=kv)
    H, I, D, Hq, Hkv = cfg.hidden, cfg.inter, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    nb = dict(plan)                            # the last launch of each name
    # attention over the slow prefix: K and V rows of every position and KV head, q, kv_len
    assert nb["attn_split"] == B * kv * Hkv * D * 2 * 2 + B * Hq * D * 2 + 4 * B
    # down GEMM of the MLP at B > 16: weights, 128x128 scales, the operand of h and its scales
    assert nb["mlp_down"] == H * I + (H // 128) * (I // 128) * 4 + B * I + B * (I // 128) * 4
    # the SwiGLU-quantise launch reads g and u in fp32 and writes the operand
    assert nb["mlp_hq"] == 2 * B * I * 4 + B * I + B * (I // 128) * 4
    # MXFP8 caches: e4m3 bytes and one exponent per 32 d, K and V
    _, pmx = _plan(B, mx=True, kv=kv)
    assert dict(pmx)["attn_split_mx"] == B * kv * Hkv * (D + D // 32) * 2 + B * Hq * D * 2 + 4 * B
    total = sum(b for _, b in plan)
    # every prefix at 2165 positions (the mean of U[234, 4096]): 36 x 567.6 MB
    # of K/V, 72 layer evaluations of 100.9 MB of weights, 10 heads of 10.5
    # MB, and the activations and intermediates each launch reads and writes
    kv_bytes = 36 * B * kv * Hkv * D * 2 * 2
    w_bytes = 72 * (6144 * H + H * 4096 + 3 * H * I) + 10 * 4096 * H
    assert kv_bytes + w_bytes < total < kv_bytes + w_bytes + 1.5e9


def test_profiler_name_map_knows_every_planned_kernel():
    known = {lib for _, lib in profiling.KERNELS}
    for B in (8, 64):
        for mx in (False, True):
            _, plan = _plan(B, mx=mx)
            for name, _ in plan:
                assert name in known, name
