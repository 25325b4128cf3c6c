#!/usr/bin/env python3
"""Decode-step hot-path benchmark on one MI355X (gfx950).

One step = the two parts of a decode step's hot path for a batch of B = 64
sequences, as a Qwen3-4B-sized layer computes them:
  * the FP8 SwiGLU MLP at M = 64 (hidden 2560, intermediate 9728, bsgemm
    128x128 weight scales, activations quantised on the GPU);
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
    if name == "attn_split":
        return int(np.sum(kv_len.astype(np.int64))) * HKV * D * 2 * 2 + B * HQ * D * 2 + 4 * B
    if name == "attn_merge":
        return B * HQ * D * 2 + 4 * B
    return 0


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
                st["aws"] = ops.new_attn_workspace(B, HQ, D, Lmax)
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


def time_parts(torch, ops, wl, parts, steps, warmup):
    """Two timed regions of `steps` steps each (every step calls every part
    once on a rotating set), bracketed by synchronisation and HIP events:
      1. clean: gives ms per step (the headline);
      2. per kernel: the library records a HIP event pair around every kernel
         it launches, on the launch stream (the events add small gaps between
         launches, so this pass is not used for the headline).
    Returns (ms per step, wall ms per step, {kernel: [ms, ...]})."""
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
    return ms_step, wall, per


def pmc_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed profiler summary
    (FETCH_SIZE and WRITE_SIZE runs scaled by a copy of known size), or None
    when there is none or the kernel's source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (3x) so that profiler byte counters can be "
                         "scaled against a kernel of known traffic")
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
    ms_step, wall, per = time_parts(torch, ops, wl, [wl.mlp, wl.attn], args.steps, args.warmup)
    torch.cuda.synchronize()
    if int(wl.err.item()) != 0:
        raise SystemExit(f"device error flag {int(wl.err.item())}")
    ktab = kernel_table(per, args.steps, B, ops.MLP_BSGEMM, kv_len, B)
    t_mlp = sum(v["us"] * v["per_step"] for k, v in ktab.items() if k.startswith("mlp"))
    t_attn = sum(v["us"] * v["per_step"] for k, v in ktab.items() if k.startswith("attn"))
    b_mlp, b_attn = mlp_bytes(B, 0), attn_bytes(kv_len, B)
    gbs_mlp = b_mlp / (t_mlp * 1e-6) / 1e9
    gbs_attn = b_attn / (t_attn * 1e-6) / 1e9
    log(f"step {ms_step * 1e3:.1f} us: mlp kernels {t_mlp:.1f} us {gbs_mlp:.0f} GB/s, "
        f"attn kernels {t_attn:.1f} us {gbs_attn:.0f} GB/s")
    for k, v in sorted(ktab.items(), key=lambda kv: -kv[1]["us"] * kv[1]["per_step"]):
        log(f"  {k:22s} {v['us']:7.1f} us  {v['GB/s']:6.0f} GB/s  ({100 * v['frac']:.1f}% of HBM peak)")
    dom_name, dom = max(ktab.items(), key=lambda kv: kv[1]["us"] * kv[1]["per_step"])
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
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": dom["GB/s"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": dom["frac"], "traffic": pmc_traffic(dom_name),
                     "algorithmic_bytes": dom["bytes"], "launch_us": dom["us"]},
        "parts": {"mlp": {"us": t_mlp, "bytes": b_mlp, "GB/s": gbs_mlp, "frac": gbs_mlp / PEAK_HBM_GBS},
                  "attn": {"us": t_attn, "bytes": b_attn, "GB/s": gbs_attn, "frac": gbs_attn / PEAK_HBM_GBS}},
        "kernels": ktab,
        "wall_ms_per_step": wall,
    }
    del wl
    torch.cuda.empty_cache()

    if not args.no_sweep:
        sweep = {"mlp_bsgemm": {}, "mlp_mxfp8": {}, "attn": {}}
        for mode, key in ((ops.MLP_BSGEMM, "mlp_bsgemm"), (ops.MLP_MXFP8, "mlp_mxfp8")):
            for M in (1, 8, 32, 64, 128):
                w = Workload(torch, ops, 1, M, mode, args.sets, kv_len, with_attn=False)
                t, _, per = time_parts(torch, ops, w, [w.mlp], 20, 5)
                gb = mlp_bytes(M, mode) / (t * 1e-3) / 1e9
                sweep[key][M] = {"us": t * 1e3, "tokens/s": M / (t * 1e-3), "GB/s": gb, "frac": gb / PEAK_HBM_GBS,
                                 "kernels": kernel_table(per, 20, M, mode)}
                log(f"{key} M={M}: {t * 1e3:.1f} us {gb:.0f} GB/s  " +
                    " ".join(f"{k}={v['us']:.1f}" for k, v in sweep[key][M]["kernels"].items()))
                del w
                torch.cuda.empty_cache()
        for Bs, lo, hi in ((1, 234, 400), (16, 234, 400), (64, 234, 400), (64, 234, 8192)):
            kv = inputs.kv_lengths(inputs.W_ATTN, Bs, lo, hi, extra=Bs + hi)
            w = Workload(torch, ops, Bs, 1, 0, 2 if hi > 400 else args.sets, kv, with_mlp=False)
            t, _, per = time_parts(torch, ops, w, [w.attn], 20, 5)
            gb = attn_bytes(kv, Bs) / (t * 1e-3) / 1e9
            sweep["attn"][f"B={Bs},kv=U[{lo},{hi}]"] = {"us": t * 1e3, "tokens/s": Bs / (t * 1e-3), "GB/s": gb,
                                                        "frac": gb / PEAK_HBM_GBS,
                                                        "kernels": kernel_table(per, 20, 1, 0, kv, Bs)}
            log(f"attn B={Bs} kv {lo}..{hi}: {t * 1e3:.1f} us {gb:.0f} GB/s")
            del w
            torch.cuda.empty_cache()
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
        result["cpu_baseline"] = cpu_baseline(B, kv_len)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
