"""Throughput of one GPT training step (fwd + bwd + Muon) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d24] [--no-cpu-baseline]

Prints ONE JSON line: tokens/s over K timed steps (gpt_step + muon_update on
synthetic Zipf(1.1) token batches already resident in HBM), MFU against the bf16
dense peak, the roofline of the dominant kernel (measured with HIP events around
its launches inside the timed steps) and the fp64 CPU oracle timed on this host's
cores.  The default run (d24, bf16) also times the other configurations, each on
its own model (`other_configs`: d12, d26 and d24 with e4m3 Linear GEMMs, laptop,
tiny).
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


def _cores() -> dict:
    """Host threads available to this process and the BLAS pool numpy uses."""
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info())
    except Exception:
        blas = None
    return {"cores": cores, "blas_threads": blas}


def cpu_baseline(cfg: dict) -> dict:
    """The fp64 oracle timed on this host.

    Measured: one whole d12 step at batch 1 (one 2048-token sequence at full width,
    depth and vocabulary): forward, backward and Muon (momentum + 5 Newton-Schulz
    iterations) on all 72 block matrices; tokens/s = 2048 / that time.  The headline
    workload (`cfg`, d24 at B = 16) does not fit the bench's time budget in fp64, so an
    estimate for it is given separately and labelled as one: fwd+bwd of one 256-token
    sequence at full width/depth/vocabulary and Newton-Schulz of one layer's six
    matrices, both timed, scaled by FLOPs to the whole step."""
    import numpy as np
    from gpt_pretraining_step_train_amd import configs, inputs
    from oracle import gpt_oracle, polar_express

    table, _ = polar_express.coefficients()
    # measured: the d12 step at B = 1
    c12 = configs.get("d12", batch=1)
    params = inputs.init_weights(c12, seed=0)
    tok, tgt = inputs.token_batch(1, c12["seq_len"], c12["vocab"], dist="zipf", seed=0)
    t0 = time.perf_counter()
    _, grads, _, _ = gpt_oracle.loss_and_grads(params, tok, tgt, c12)
    moms = [np.zeros_like(g) for g in grads]
    gpt_oracle.muon_update(params, grads, moms, c12, LR, table)
    t12 = time.perf_counter() - t0
    del params, grads, moms
    # estimated: the headline workload, from a bounded sample
    t = 256
    c1 = dict(cfg, batch=1, seq_len=t)
    params = inputs.init_weights(c1, seed=0)
    tok, tgt = inputs.token_batch(1, t, cfg["vocab"], dist="zipf", seed=0)
    t0 = time.perf_counter()
    gpt_oracle.loss_and_grads(params, tok, tgt, c1)
    t_fb = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(1, 7):  # one layer's six matrices
        g = np.asarray(params[i], dtype=np.float64)
        gpt_oracle.muon_matrix(g, np.zeros_like(g), table)
    t_ns = time.perf_counter() - t0
    f_full, f_samp = configs.step_flops(cfg), configs.step_flops(c1)
    fb = lambda f: f["linear"] + f["head"] + f["attn"]  # noqa: E731
    t_est = t_fb * fb(f_full) / fb(f_samp) + t_ns * cfg["depth"]
    return {
        "value": c12["seq_len"] / t12, "unit": "tokens/s", **_cores(), "kind": "oracle",
        "workload": "d12 GPT training step at B=1 x T=2048 (fwd+bwd+Muon on all 72 block matrices)",
        "sample": f"one whole d12 step at batch 1, timed in full: {t12:.1f} s for 2048 tokens (fp64 numpy)",
        "headline_estimate": {
            "estimated": True, "value": cfg["batch"] * cfg["seq_len"] / t_est, "unit": "tokens/s",
            "workload": f"{cfg['name']} B={cfg['batch']} x T={cfg['seq_len']}",
            "sample": (f"fwd+bwd of 1 x {t} tokens at full width/depth/vocab ({t_fb:.1f} s) scaled by FLOPs, plus "
                       f"Newton-Schulz of one layer's 6 matrices ({t_ns:.1f} s) x {cfg['depth']} layers; "
                       f"estimated step {t_est:.0f} s")},
    }


def time_steps(model, cfg, batches, steps, warmup, accum=1, adamw=False):
    """Mean ms per step (accum x gpt_step + muon_update [+ adamw_update]) over `steps`
    steps after `warmup`, HIP events on the current stream; returns (ms, losses)."""
    import torch
    stream = torch.cuda.current_stream()
    K = max(1, accum)

    def one(i):
        for k in range(K):
            tok, tgt = batches[(i * K + k) % len(batches)]
            loss = model.step(tok, tgt, accumulate=k > 0, grad_scale=1.0 / K) if K > 1 else model.step(tok, tgt)
        model.muon_update(LR)
        if adamw:
            model.adamw_update(1e-3, 0.8, 0.95, 1e-10, 0.0)
        return loss

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    if steps == 0:
        return 0.0, []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    losses = [one(warmup + i) for i in range(steps)]
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, losses


def make_batches(cfg, n=8):
    import torch
    from gpt_pretraining_step_train_amd import inputs
    out = []
    for s in range(n):
        tok, tgt = inputs.token_batch(cfg["batch"], cfg["seq_len"], cfg["vocab"], dist=cfg["tokens"], seed=s)
        out.append((torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()))
    return out


def mfu_fields(cfg, ms, fp8):
    """MFU of one step: algorithmic FLOPs (Muon included) against the bf16 peak; the
    forward+backward FLOPs alone (model FLOPs, no Newton-Schulz); for e4m3 steps also
    against the fp8 peak and blended (Linear GEMM FLOPs at the fp8 peak, the rest at bf16)."""
    from gpt_pretraining_step_train_amd import configs
    fl = configs.step_flops(cfg)
    t = ms / 1e3
    out = {"mfu": fl["total"] / t / PEAK_BF16,
           "mfu_model_flops": (fl["total"] - fl["muon"]) / t / PEAK_BF16,
           "flops_per_step": fl["total"]}
    if fp8:
        out["mfu_fp8_peak"] = fl["total"] / t / PEAK_FP8
        out["mfu_blended"] = ((fl["linear"] + fl["head"]) / PEAK_FP8 + (fl["attn"] + fl["muon"]) / PEAK_BF16) / t
    return out


def other_configs(steps, warmup) -> dict:
    """The other configurations, each timed on its own model: d12 (bf16, the metric's
    second model), d26 with e4m3 Linear GEMMs (the fp8 config), d24 with e4m3 Linear
    GEMMs (the d24 record command's --fp8), and the two small ones (launch-bound)."""
    import torch
    from gpt_pretraining_step_train_amd import binding, configs
    out = {}
    plan = [("d12", {}, steps), ("d26", {"precision": "fp8"}, steps), ("d24", {"precision": "fp8"}, steps),
            ("laptop", {}, 5 * steps), ("tiny", {}, 5 * steps)]
    for name, over, k in plan:
        cfg = configs.get(name, **over)
        model = binding.Model(cfg, seed=0)
        batches = make_batches(cfg)
        ms, losses = time_steps(model, cfg, batches, k, warmup)
        n_tok = cfg["batch"] * cfg["seq_len"]
        key = name + ("_fp8" if cfg["precision"] == "fp8" else "")
        out[key] = {"value": n_tok / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms, "steps": k,
                    "dtype": cfg["precision"], "global_batch": cfg["batch"], "seq_len": cfg["seq_len"],
                    "depth": cfg["depth"], "d_model": cfg["d_model"],
                    **mfu_fields(cfg, ms, cfg["precision"] == "fp8"), "loss_first_last": [losses[0], losses[-1]]}
        if name in ("tiny", "laptop"):  # launch-bound: the same step replayed from a HIP graph
            gms = time_graph_steps(model, batches[0], k, warmup)
            out[key]["hip_graph"] = {"value": n_tok / (gms / 1e3), "unit": "tokens/s", "ms_per_step": gms,
                                     "what": "gpt_step_async + muon_update captured once, replayed on one resident batch"}
        del model
        torch.cuda.empty_cache()
    return out


def time_graph_steps(model, batch, steps, warmup):
    """Mean ms per replay of one captured step (gpt_step_async + muon_update)."""
    import torch
    tok, tgt = batch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        model.step_async(tok, tgt)
        model.muon_update(LR)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    model.step_result()  # the last replay's loss and error flags
    return ev0.elapsed_time(ev1) / steps


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
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing d12, d26-fp8, d24-fp8, laptop and tiny after the headline d24 line")
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
    # e4m3 Linears only with --fp8; otherwise the configuration's own precision (fp32 for
    # tiny), with d26's e4m3 default taken as bf16
    cfg["precision"] = "fp8" if args.fp8 else ("bf16" if cfg["precision"] == "fp8" else cfg["precision"])
    torch.cuda.set_device(0)
    model = binding.Model(cfg, seed=0)
    B, T, V = cfg["batch"], cfg["seq_len"], cfg["vocab"]
    batches = make_batches(cfg)
    K = max(1, args.accum)
    time_steps(model, cfg, batches, 0, args.warmup, K, args.adamw)
    model.prof_enable(args.dominant)
    w0 = time.perf_counter()
    ms_step, losses = time_steps(model, cfg, batches, args.steps, 0, K, args.adamw)
    wall = time.perf_counter() - w0
    gpu_ms = ms_step * args.steps
    n_launch, k_ms, k_flops = model.prof_read()
    model.prof_enable(None)
    del model
    torch.cuda.empty_cache()
    n_tok = B * T * K
    tps = n_tok / (ms_step / 1e3)
    fl = configs.step_flops(cfg)
    if K > 1:  # K forward/backward passes per Muon update
        fl = {k: (v if k == "muon" else K * v) for k, v in fl.items()}
        fl["total"] = fl["linear"] + fl["head"] + fl["attn"] + fl["muon"]
    t_s = ms_step / 1e3
    mfu = fl["total"] / t_s / PEAK_BF16
    mfu_extra = {"mfu_model_flops": (fl["total"] - fl["muon"]) / t_s / PEAK_BF16}
    if args.fp8:  # against the fp8 peak, and blended: Linear GEMM flops at the fp8 peak, the rest at bf16
        mfu_extra["mfu_fp8_peak"] = fl["total"] / t_s / PEAK_FP8
        mfu_extra["mfu_blended"] = ((fl["linear"] + fl["head"]) / PEAK_FP8 + (fl["attn"] + fl["muon"]) / PEAK_BF16) / t_s
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
        "vs_baseline": None, "dtype": "fp8-e4m3 linears, bf16 attention/NS" if args.fp8 else cfg["precision"], "data": "synthetic (seeded Zipf(1.1) token ids, 8 batches cycled)",
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
        "mfu": mfu, **mfu_extra, "flops_per_step": fl["total"], "wall_s": wall,
        "loss_first_last": [losses[0], losses[-1]],
        "roofline": roof,
    }
    default_run = (args.config == "d24" and not args.fp8 and K == 1 and not args.adamw and not args.window
                   and not args.kv_heads and not args.extras)
    if default_run and not args.no_other_configs:
        out["other_configs"] = other_configs(min(args.steps, 10), max(2, min(args.warmup, 3)))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
