#!/usr/bin/env python3
"""Decode-step hot-path benchmark on one MI355X (gfx950).

One step = the two parts of a decode step's hot path for a batch of B = 64
sequences, as a Qwen3-4B-sized layer computes them:
  * the FP8 SwiGLU MLP at M = 64 (hidden 2560, intermediate 9728, bsgemm
    128x128 weight scales, activations quantised in-kernel), one launch;
  * GQA decode attention (32 query / 8 KV heads, dim 128) over bf16 caches of
    32768 slots per sequence with ragged kv_len ~ U{234..400}.
tokens/s = B / step time.  Inputs are resident in HBM before timing starts.
Four independent weight/cache sets are rotated (reuse distance > 600 MB) so
the 256 MB Infinity Cache cannot serve repeats.

Prints ONE JSON line.  Extra keys: per-kernel HBM rates, the M sweep of the
MLP (bsgemm and MXFP8) and the B sweep of attention, and the CPU oracle timed
on the host cores as a reported baseline.
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
H, I = 2560, 9728                # Qwen3-4B MLP
HQ, HKV, D, CAP = 32, 8, 128, 32768


def mlp_bytes(M, mode):
    w = 3 * H * I
    s = 3 * (H // 128) * (I // 128) * 4 if mode == 0 else 3 * H * I // 32
    return w + s + 2 * M * H * 2


def attn_bytes(kv_len, B):
    return int(np.sum(kv_len.astype(np.int64))) * HKV * D * 2 * 2 + 2 * B * HQ * D * 2 + 4 * B


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Workload:
    """Rotating sets of GPU-resident weights, activations and KV caches."""

    def __init__(self, torch, ops, B, M, mode, n_sets, kv_len, with_attn=True, with_mlp=True):
        self.torch, self.ops = torch, ops
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
                    ws.append(ops.quantize_weight(wb, mode))
                    del wb
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
                kc = torch.empty((B, HKV, CAP, D), dtype=torch.bfloat16, device="cuda")
                vc = torch.empty((B, HKV, CAP, D), dtype=torch.bfloat16, device="cuda")
                kc[:, :, :Lmax] = torch.randn((B, HKV, Lmax, D), generator=g, device="cuda").to(torch.bfloat16)
                vc[:, :, :Lmax] = torch.randn((B, HKV, Lmax, D), generator=g, device="cuda").to(torch.bfloat16)
                st["k"], st["v"] = kc, vc
                st["q"] = torch.randn((B, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
                st["o"] = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")
                st["kv"] = torch.from_numpy(kv_len).cuda()
                st["aws"] = torch.empty(ops.attn_workspace_bytes(B, HQ, D, Lmax), dtype=torch.uint8,
                                        device="cuda")
                st["hint"] = Lmax
            self.sets.append(st)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def mlp(self, s):
        st = self.sets[s]
        self.ops.swiglu_mlp_fp8(st["x"], *st["w"], self.mode, y=st["y"], workspace=st["ws"], err=self.err)

    def attn(self, s):
        st = self.sets[s]
        self.ops.gqa_decode_attn(st["q"], st["k"], st["v"], st["kv"], st["hint"], out=st["o"],
                                 workspace=st["aws"], err=self.err)


def time_parts(torch, wl, parts, steps, warmup):
    """Run `steps` steps (each calls every part once on a rotating set);
    returns per-part mean launch durations (ms, HIP events on the launch
    stream) and the total ms per step."""
    n = len(wl.sets)
    for i in range(warmup):
        for p in parts:
            p(i % n)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in parts]
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        for j, p in enumerate(parts):
            ev[i][j][0].record()
            p(i % n)
            ev[i][j][1].record()
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    per = [float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)])) for j in range(len(parts))]
    return per, t0.elapsed_time(t1) / steps, wall


def cpu_baseline(B, kv_len):
    """The oracle as it stands, on the host cores: one step at B = 64 (MLP at
    M = 64 plus attention), weights dequantised once outside the timing,
    median of 3."""
    from oracle import attention as oattn
    from oracle import fp8, mlp as omlp
    from fp8_transformer_step_amd import inputs
    try:
        import threadpoolctl
        blas = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        blas = 1
    f32 = inputs.bf16_bits_to_f32
    wbits = inputs.mlp_weights(inputs.W_BSGEMM, H, I)
    deq = [fp8.dequant_block_fp32(*fp8.quant_weight_128x128(f32(b)), 128, 128) for b in wbits]
    xb = f32(inputs.mlp_activations(inputs.W_BSGEMM, B, H))
    Lmax = int(kv_len.max())
    qb, kb, vb = inputs.attention_prefix(inputs.W_ATTN, B, HQ, HKV, D, Lmax)
    q, k, v = f32(qb), f32(kb), f32(vb)
    times = []
    for _ in range(3):
        t = time.perf_counter()
        omlp.swiglu_mlp(xb, *deq, omlp.MODE_BSGEMM)
        oattn.gqa_decode_attention(q, k, v, kv_len)
        times.append(time.perf_counter() - t)
    t = float(np.median(times))
    return {"value": B / t, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"one full step at B={B} (MLP M={B} + attention), median of 3 runs, "
                      f"float64 NumPy, weights dequantised once outside the timing; "
                      f"{t:.3f} s per step; host affinity {len(os.sched_getaffinity(0))} cores"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is single-GPU; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_transformer_step_amd import inputs, ops

    torch.cuda.set_device(0)
    B = args.batch
    kv_len = inputs.kv_lengths(inputs.W_ATTN, B, 234, 400)
    log(f"bench: building {args.sets} rotating sets (B={B})")
    wl = Workload(torch, ops, B, B, ops.MLP_BSGEMM, args.sets, kv_len)
    (t_mlp, t_attn), ms_step, wall = time_parts(torch, wl, [wl.mlp, wl.attn], args.steps, args.warmup)
    torch.cuda.synchronize()
    if int(wl.err.item()) != 0:
        raise SystemExit(f"device error flag {int(wl.err.item())}")
    b_mlp, b_attn = mlp_bytes(B, 0), attn_bytes(kv_len, B)
    gbs_mlp = b_mlp / (t_mlp * 1e-3) / 1e9
    gbs_attn = b_attn / (t_attn * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us: mlp {t_mlp * 1e3:.1f} us {gbs_mlp:.0f} GB/s, "
        f"attn {t_attn * 1e3:.1f} us {gbs_attn:.0f} GB/s")
    dom = ("swiglu_mlp_fp8", b_mlp, t_mlp) if t_mlp >= t_attn else ("gqa_decode_attn", b_attn, t_attn)
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
        "dtype": "fp8e4m3 MLP, bf16 attention (fp32 accumulate)",
        "data": "synthetic (seeded, random-init weights N(0,0.02), q/K/V N(0,1))",
        "config": {"workload": "decode-step hot path, one Qwen3-4B-shaped layer at batch 64: "
                               "bsgemm FP8 SwiGLU MLP (2560/9728, M=64) + GQA decode attention "
                               "(32/8 heads, dim 128, cache 32768, kv_len U[234,400])",
                   "batch": B, "hidden": H, "intermediate": I, "heads": [HQ, HKV, D], "cache": CAP},
        "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": dom[1] / (dom[2] * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": dom[1] / (dom[2] * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes": dom[1], "launch_us": dom[2] * 1e3},
        "parts": {"mlp": {"us": t_mlp * 1e3, "bytes": b_mlp, "GB/s": gbs_mlp, "frac": gbs_mlp / PEAK_HBM_GBS},
                  "attn": {"us": t_attn * 1e3, "bytes": b_attn, "GB/s": gbs_attn,
                           "frac": gbs_attn / PEAK_HBM_GBS}},
        "wall_ms_per_step": wall,
    }
    del wl
    torch.cuda.empty_cache()

    if not args.no_sweep:
        sweep = {"mlp_bsgemm": {}, "mlp_mxfp8": {}, "attn": {}}
        for mode, key in ((ops.MLP_BSGEMM, "mlp_bsgemm"), (ops.MLP_MXFP8, "mlp_mxfp8")):
            for M in (1, 8, 32, 64, 128):
                w = Workload(torch, ops, 1, M, mode, args.sets, kv_len, with_attn=False)
                (t,), _, _ = time_parts(torch, w, [w.mlp], 20, 5)
                gb = mlp_bytes(M, mode) / (t * 1e-3) / 1e9
                sweep[key][M] = {"us": t * 1e3, "tokens/s": M / (t * 1e-3), "GB/s": gb, "frac": gb / PEAK_HBM_GBS}
                log(f"{key} M={M}: {t * 1e3:.1f} us {gb:.0f} GB/s")
                del w
                torch.cuda.empty_cache()
        for Bs, lo, hi in ((1, 234, 400), (16, 234, 400), (64, 234, 400), (64, 234, 8192)):
            kv = inputs.kv_lengths(inputs.W_ATTN, Bs, lo, hi, extra=Bs + hi)
            w = Workload(torch, ops, Bs, 1, 0, 2 if hi > 400 else args.sets, kv, with_mlp=False)
            (t,), _, _ = time_parts(torch, w, [w.attn], 20, 5)
            gb = attn_bytes(kv, Bs) / (t * 1e-3) / 1e9
            sweep["attn"][f"B={Bs},kv=U[{lo},{hi}]"] = {"us": t * 1e3, "tokens/s": Bs / (t * 1e-3), "GB/s": gb,
                                                        "frac": gb / PEAK_HBM_GBS}
            log(f"attn B={Bs} kv {lo}..{hi}: {t * 1e3:.1f} us {gb:.0f} GB/s")
            del w
            torch.cuda.empty_cache()
        result["sweep"] = sweep

    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(B, kv_len)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
