"""Throughput of one GPT training step (fwd + bwd + Muon) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d24] [--no-cpu-baseline]

Prints ONE JSON line: tokens/s over K timed steps (gpt_step + muon_update on
synthetic Zipf(1.1) token batches already resident in HBM), MFU against the bf16
dense peak, the roofline of the dominant kernel (measured with HIP events around
its launches inside the timed steps) and the fp64 CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "training tokens/sec + MFU on 1 MI355X, d12 and d24 GPT at seq 2048"
PEAK_BF16 = 2.5166e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP8 = 5.0332e15       # MI355X dense fp8 MFMA, FLOP/s
PEAK_HBM = 8.0e12          # bytes/s
LR = 0.02
# rocprofv3 traffic summaries (FETCH_SIZE + WRITE_SIZE, copy-calibrated) per dominant kernel
TRAFFIC = {"gemm_bf16_dma_kernel<256,256,NT>": "gemm_bf16_dma_kernel_NT__d24_step_traffic.md",
           "gemm_fp8_dma_kernel<256,256,NT>": "gemm_fp8_dma_kernel_NT__d24_fp8_step_traffic.md"}


def cpu_baseline(cfg: dict) -> dict:
    """The fp64 oracle on a bounded sample of the step: fwd+bwd of one sequence of
    `t` tokens at the full width/depth/vocabulary, plus the Newton-Schulz work of one
    layer's six matrices; scaled to the full step (B*T tokens, all L layers)."""
    import numpy as np
    from gpt_pretraining_step_train_amd import inputs
    from oracle import gpt_oracle, polar_express

    t = 256
    c1 = dict(cfg, batch=1, seq_len=t)
    params = inputs.init_weights(c1, seed=0)
    tok, tgt = inputs.token_batch(1, t, cfg["vocab"], dist="zipf", seed=0)
    t0 = time.perf_counter()
    gpt_oracle.loss_and_grads(params, tok, tgt, c1)
    t_fb = time.perf_counter() - t0
    table, _ = polar_express.coefficients()
    t0 = time.perf_counter()
    for i in range(1, 7):  # one layer's six matrices
        g = np.asarray(params[i], dtype=np.float64)
        gpt_oracle.muon_matrix(g, np.zeros_like(g), table)
    t_ns = time.perf_counter() - t0
    n_tok = cfg["batch"] * cfg["seq_len"]
    # attention cost grows with T; scale the sampled fwd+bwd by the FLOP ratio
    from gpt_pretraining_step_train_amd import configs
    f_full = configs.step_flops(cfg)
    f_samp = configs.step_flops(c1)
    fb_full = f_full["linear"] + f_full["head"] + f_full["attn"]
    fb_samp = f_samp["linear"] + f_samp["head"] + f_samp["attn"]
    t_step = t_fb * fb_full / fb_samp + t_ns * cfg["depth"]
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info())
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {
        "value": n_tok / t_step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"fp64 numpy oracle: fwd+bwd of 1 x {t} tokens at full width/depth/vocab "
                   f"({t_fb:.1f} s) scaled by FLOPs to {cfg['batch']}x{cfg['seq_len']} tokens, plus "
                   f"Newton-Schulz of one layer's 6 matrices ({t_ns:.1f} s) x {cfg['depth']} layers; "
                   f"estimated step {t_step:.0f} s"),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d24")
    ap.add_argument("--accum", type=int, default=1, metavar="K",
                    help="K micro-batches accumulated per optimizer update (gpt_step_accumulate, grad scale 1/K): "
                         "one timed step is K forward/backward passes and one Muon update")
    ap.add_argument("--adamw", action="store_true",
                    help="also run AdamW on E and U in every step (lr 1e-3, betas 0.8/0.95, eps 1e-10: the "
                         "pages print none; the values do not change the cost)")
    ap.add_argument("--fp8", action="store_true",
                    help="e4m3 operands on every Linear GEMM (the configs' fp8 recipe); default bf16")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="sliding-window attention: query i sees keys i-W < j <= i (0: full causal)")
    ap.add_argument("--kv-heads", type=int, default=0, metavar="H",
                    help="grouped-query attention with H key/value heads (0: one per query head)")
    ap.add_argument("--extras", type=int, default=0, metavar="MASK",
                    help="1 per-layer residual scaling, 2 smear, 4 backout, 8 value embeddings, 16 NorMuon (parameters at their start values, "
                         "which do not change the cost; AdamW updates them when --adamw is given)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dominant", default=None,
                    help="kernel timed for the roofline (default: the NT GEMM of the step's precision)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run three plain device copies of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        torch.cuda.set_device(0)
        x = torch.ones(args.copy_probe * 2 ** 20 // 4, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)  # one elementwise kernel: reads and writes the bytes once
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": x.numel() * 4, "copies": 3}), flush=True)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the step has no multi-GPU path in this build "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from gpt_pretraining_step_train_amd import binding, configs, inputs

    cfg = configs.get(args.config, attn_window=args.window, n_kv_head=args.kv_heads, extras=args.extras)
    if args.dominant is None:
        args.dominant = "gemm_fp8_dma_kernel<256,256,NT>" if args.fp8 else "gemm_bf16_dma_kernel<256,256,NT>"
    cfg["precision"] = "fp8" if args.fp8 else "bf16"
    torch.cuda.set_device(0)
    model = binding.Model(cfg, seed=0)
    B, T, V = cfg["batch"], cfg["seq_len"], cfg["vocab"]
    batches = []
    for s in range(8):
        tok, tgt = inputs.token_batch(B, T, V, dist="zipf", seed=s)
        batches.append((torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()))
    stream = torch.cuda.current_stream()

    K = max(1, args.accum)

    def one(i):
        for k in range(K):
            tok, tgt = batches[(i * K + k) % len(batches)]
            loss = model.step(tok, tgt, accumulate=k > 0, grad_scale=1.0 / K) if K > 1 else model.step(tok, tgt)
        model.muon_update(LR)
        if args.adamw:
            model.adamw_update(1e-3, 0.8, 0.95, 1e-10, 0.0)
        return loss

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    model.prof_enable(args.dominant)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    losses = [one(args.warmup + i) for i in range(args.steps)]
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    n_launch, k_ms, k_flops = model.prof_read()
    model.prof_enable(None)
    ms_step = gpu_ms / args.steps
    n_tok = B * T * K
    tps = n_tok / (ms_step / 1e3)
    fl = configs.step_flops(cfg)
    if K > 1:  # K forward/backward passes per Muon update
        fl = {k: (v if k == "muon" else K * v) for k, v in fl.items()}
        fl["total"] = fl["linear"] + fl["head"] + fl["attn"] + fl["muon"]
    mfu = fl["total"] / (ms_step / 1e3) / PEAK_BF16
    # fp8: the Linear GEMM flops run at the fp8 peak, the rest (attention, NS) at bf16
    mfu_fp8 = None
    if args.fp8:
        t_ideal = (fl["linear"] + fl["head"]) / PEAK_FP8 + (fl["attn"] + fl["muon"]) / PEAK_BF16
        mfu_fp8 = t_ideal / (ms_step / 1e3)
    achieved = k_flops / (k_ms / 1e3) if k_ms > 0 else None
    from gpt_pretraining_step_train_amd import profiling
    rec = None
    if args.dominant in TRAFFIC and args.config == "d24" and not args.kv_heads:  # same GEMM launches
        rec = profiling.read_traffic(os.path.join(ROOT, "profiles", TRAFFIC[args.dominant]))
    peak = PEAK_FP8 if "fp8" in args.dominant else PEAK_BF16  # a contraction takes its own dtype's peak
    roof = {
        "kernel": args.dominant, "bound": "mfma", "achieved": achieved / 1e12 if achieved else None,
        "peak": peak / 1e12, "unit": "TFLOP/s",
        "frac": (achieved / peak) if achieved else None,
        "traffic": rec["bytes_per_launch"] if rec else None,
        "traffic_detail": ({"fetch_bytes": rec["fetch_bytes_per_launch"], "write_bytes": rec["write_bytes_per_launch"],
                            "source": "profiles/" + TRAFFIC[args.dominant]} if rec else None),
        "launches": n_launch, "avg_launch_us": 1e3 * k_ms / n_launch if n_launch else None,
        "share_of_step_time": (k_ms / gpu_ms) if gpu_ms > 0 else None,
    }
    out = {
        "metric": METRIC, "value": tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3 linears, bf16 attention/NS" if args.fp8 else "bf16", "data": "synthetic (seeded Zipf(1.1) token ids, 8 batches cycled)",
        "config": {"workload": f"{args.config} GPT training step{' (fp8 linears)' if args.fp8 else ''}: "
                               + (f"{K} accumulated fwd+bwd micro-batches of B={B} x T={T}, then Muon(5 NS)"
                                f"{'+AdamW(E,U)' if args.adamw else ''}" if K > 1 else
                                f"fwd+bwd+Muon(5 NS){'+AdamW(E,U)' if args.adamw else ''} on B={B} x T={T}")
                               + (f", sliding-window attention W={args.window}" if args.window else "")
                               + (f", grouped-query attention with {args.kv_heads} key/value heads"
                                  if args.kv_heads else "")
                               + (f", extras mask {args.extras} (1 residual scaling, 2 smear, 4 backout, 8 value embeddings, 16 NorMuon)"
                                  if args.extras else ""),
                   "depth": cfg["depth"], "d_model": cfg["d_model"], "n_head": cfg["n_head"],
                   "n_kv_head": configs.kv_heads(cfg), "attn_window": args.window, "extras": args.extras,
                   "vocab": V, "global_batch": B * K, "micro_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "mfu": mfu, "mfu_at_fp8_peak_for_linears": mfu_fp8, "flops_per_step": fl["total"], "wall_s": wall,
        "loss_first_last": [losses[0], losses[-1]],
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
