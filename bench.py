#!/usr/bin/env python3
"""Benchmark of the causal GQA flash-attention hot path on one MI355X.

One step = one pass of the whole hot path on seeded synthetic inputs already
resident in device memory:
  * attn_fwd, then the backward's three stages (preprocess, dK/dV, dQ) on the
    training workload (default: bf16, B=4, 12 query / 4 key-value heads,
    N=1024, d=64);
  * attn_decode + attn_lse_merge on the decode workload (bf16, 32/8 heads,
    d=128, a 4096-key cache in 16 splits), rotating over enough distinct caches
    that every step reads its keys and values from HBM, not from cache.
Each launch is bracketed by HIP events on the stream it runs on.

Prints ONE JSON line.  `value` is the training workload's algorithmic
fwd+bwd TFLOP/s (4*d flop per unmasked (query, key) pair forward, 10*d
backward) over the time of its four launches; the decode workload's GB/s is
reported beside it.  `roofline` describes the kernel with the largest share of
the step's time; `cpu_baseline` times the CPU f64 oracle on a bounded sample
of the same training workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 bf16 flop/clk/CU (dense)
PEAK_HBM_GBS = 8000.0          # 8 TB/s HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa12x4_b4_n1024_d64",
                    help="training workload name (see workloads.TRAIN_CONFIGS)")
    ap.add_argument("--decode-caches", type=int, default=24,
                    help="distinct KV caches the decode leg rotates over (cold-cache reads)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this build runs on one GPU only; "
                                   "multi-GPU runs are not supported"}))
        sys.exit(2)

    import torch
    import attention_causal_gqa_flash_amd as attn
    from attention_causal_gqa_flash_amd import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    attn.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    cfg = W.TRAIN_CONFIGS[args.workload]
    dcfg = W.C5
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    x = W.train_inputs(cfg)
    g = {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in x.items()}
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    o = torch.empty((B, Hq, N, d), device=dev)
    lse = torch.empty((B, Hq, N), device=dev)
    delta = torch.empty((B, Hq, N), device=dev)
    dq = torch.empty((B, Hq, N, d), device=dev)
    dk = torch.empty((B, Hkv, N, d), device=dev)
    dv = torch.empty((B, Hkv, N, d), device=dev)

    xd = W.decode_inputs(dcfg)
    ddt = torch.bfloat16 if dcfg.dtype == "bf16" else torch.float32
    dq_in = torch.from_numpy(xd["q"]).to(dev).to(ddt)
    kc0 = torch.from_numpy(xd["k_cache"]).to(dev).to(ddt)
    vc0 = torch.from_numpy(xd["v_cache"]).to(dev).to(ddt)
    ncache = max(1, args.decode_caches)
    # distinct cache pairs (same values, different memory) so each step misses in cache
    caches = [(kc0.clone(), vc0.clone()) for _ in range(ncache)]
    S = dcfg.n_splits
    part_o = torch.empty((dcfg.B, dcfg.Hq, S, dcfg.d), device=dev)
    part_lse = torch.empty((dcfg.B, dcfg.Hq, S), device=dev)
    dec_o = torch.empty((dcfg.B, dcfg.Hq, dcfg.d), device=dev)
    dec_lse = torch.empty((dcfg.B, dcfg.Hq), device=dev)

    names = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "decode_split", "lse_merge"]

    def launches(step):
        kc, vc = caches[step % ncache]
        return [
            lambda: attn.attn_fwd(g["q"], g["k"], g["v"], True, cfg.scale, o=o, lse=lse),
            lambda: attn.attn_bwd_preprocess(o, g["dout"], delta=delta),
            lambda: attn.attn_bwd_dkdv(g["q"], g["k"], g["v"], lse, g["dout"], delta, True,
                                       cfg.scale, dk=dk, dv=dv),
            lambda: attn.attn_bwd_dq(g["q"], g["k"], g["v"], lse, g["dout"], delta, True,
                                     cfg.scale, dq=dq),
            lambda: attn.attn_decode(dq_in, kc, vc, S, dcfg.scale, part_o=part_o,
                                     part_lse=part_lse),
            lambda: attn.attn_lse_merge(part_o, part_lse, o=dec_o, lse=dec_lse),
        ]

    for s in range(args.warmup):
        for fn in launches(s):
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in names] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        for (e0, e1), fn in zip(ev[s], launches(args.warmup + s)):
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {n: np.array([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(K)])
          for i, n in enumerate(names)}
    mean_us = {n: float(ms[n].mean() * 1e3) for n in names}

    # algorithmic work
    pairs = cfg.pairs
    flop = {"fwd": 4 * d * pairs,
            "bwd_dkdv": 8 * d * pairs,      # S recompute, dP, dV, dK
            "bwd_dq": 2 * d * pairs}        # dQ (its S/dP recompute is not credited)
    train_us = sum(mean_us[n] for n in ("fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"))
    train_flop = cfg.fwd_flop + cfg.bwd_flop
    value = train_flop / (train_us * 1e-6) / 1e12

    dec_bytes = dcfg.algorithmic_bytes()
    dec_us = mean_us["decode_split"] + mean_us["lse_merge"]
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9

    # dominant kernel of the step and its roofline
    dom = max(names, key=lambda n: mean_us[n])
    if dom in flop:
        achieved = flop[dom] / (mean_us[dom] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(mean_us[dom], 3)}
    elif dom == "bwd_preprocess":
        nbytes = B * Hq * N * d * (2 if cfg.dtype == "bf16" else 4) + B * Hq * N * d * 4 + B * Hq * N * 4
        achieved = nbytes / (mean_us[dom] * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "avg_launch_us": round(mean_us[dom], 3)}
    else:
        achieved = dec_bytes / (mean_us["decode_split"] * 1e-6) / 1e9
        roof = {"kernel": "decode_split", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None, "avg_launch_us": round(mean_us["decode_split"], 3)}

    kernels = {n: {"avg_us": round(mean_us[n], 3)} for n in names}
    for n, f in flop.items():
        kernels[n]["TFLOP_s"] = round(f / (mean_us[n] * 1e-6) / 1e12, 2)
        kernels[n]["frac_bf16_peak"] = round(f / (mean_us[n] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    result = {
        "metric": "attn fwd+bwd TFLOP/s & % bf16 MFMA peak; decode GB/s & % HBM peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "Hq": Hq, "Hkv": Hkv, "seq_len": N, "head_dim": d,
                   "causal": True, "decode_workload": dcfg.name},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_bwd_us": round(train_us, 3),
        "decode": {"GB_per_s": round(dec_gbs, 1), "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "us_per_call": round(dec_us, 3), "bytes": dec_bytes,
                   "distinct_caches": ncache},
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg, x, budget_s: float) -> dict:
    """The f64 oracle on (batch, key/value-group) slices of the same workload,
    fwd + bwd, until the time budget is used; reported in the metric's unit."""
    import oracle
    G = cfg.Hq // cfg.Hkv
    groups = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    done, flop = 0, 0
    t0 = time.perf_counter()
    while done < len(groups) and time.perf_counter() - t0 < budget_s:
        b, g = groups[done]
        hs = slice(g * G, (g + 1) * G)
        q, k, v, do = (x["q"][b:b + 1, hs], x["k"][b:b + 1, g:g + 1], x["v"][b:b + 1, g:g + 1],
                       x["dout"][b:b + 1, hs])
        oracle.attn_fwd(q, k, v, True, cfg.scale)
        oracle.attn_bwd(q, k, v, do, True, cfg.scale)
        done += 1
        flop += G * cfg.N * (cfg.N + 1) // 2 * 14 * cfg.d
    el = time.perf_counter() - t0
    return {"value": round(flop / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, kv-group) slices of {cfg.name}, "
                      f"fwd+bwd in f64, {el:.1f} s"}


if __name__ == "__main__":
    main()
