#!/usr/bin/env python3
"""Benchmark of the causal GQA flash-attention hot path on one MI355X.

One step = one pass of the whole hot path on seeded synthetic inputs already
resident in device memory:
  * the training op: attn_fwd, then attn_bwd (at d=64 the preprocess, then
    one kernel holding both the dK/dV and the dQ work; at d=128 the dQ kernel,
    which also computes the preprocess's row terms, then the dK/dV kernel) on
    the training workload
    (default: bf16, B=4, 12 query / 4 key-value heads, N=1024, d=64);
  * the decode op: split-KV decode + LSE merge (attn_decode_merged: the decode
    kernel then the merge kernel) on the decode workload (bf16, 32/8 heads, d=128, a 4096-key cache in 16
    splits), rotating over enough distinct caches (default 24 x 16 MiB) that
    every step reads its keys and values from HBM rather than from cache.

The K timed steps are captured into two HIP graphs (K training ops, K decode
ops) and replayed once each between HIP events; the launches are the same
C-ABI calls an eager caller makes, without the host-side launch overhead that
would otherwise dominate the short decode op.  Each kernel's average duration
is measured the same way (a graph of K launches of that kernel alone; the
gradient stage `bwd_grads` is timed per attn_bwd_grads call, which includes a
zero-fill launch of dk/dv when they are accumulated with atomics).

Outside the step, `fwd_chunk` times attn_fwd_kv on a 512-token prefill chunk
against a 4096-key context (workload chunk_gqa32x8_nq512_nk4096_d128, 4·d flop
per visible pair), and `decode_append` times one decode step with cache append over
8 sequences of their own lengths (attn_decode_append, workload
decode_append_gqa32x8_b8_lc4096_d128_s16), rotating over 4 distinct cache pairs.

Prints ONE JSON line.  `value` is the training workload's algorithmic fwd+bwd
TFLOP/s (4*d flop per unmasked (query, key) pair forward, 10*d backward);
`decode` gives the decode workload's GB/s of algorithmic bytes (K and V caches
+ q read once, o and lse written once).  `roofline` describes the kernel with
the largest share of the step's time; `cpu_baseline` times the CPU f64 oracle
on a bounded sample of the same training workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 bf16 flop/clk/CU (dense)
PEAK_HBM_GBS = 8000.0          # 8 TB/s HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa12x4_b4_n1024_d64",
                    help="training workload name (see workloads.TRAIN_CONFIGS)")
    ap.add_argument("--decode-caches", type=int, default=24,
                    help="distinct KV caches the decode op rotates over (cold-cache reads)")
    ap.add_argument("--append-caches", type=int, default=4,
                    help="distinct cache pairs the decode-append measurement rotates over")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--no-kernel-breakdown", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch eagerly instead of replaying graphs (for counter collection; "
                         "short ops are then bound by host launch overhead)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="only run a plain device-to-device copy of known size (the reference "
                         "dispatch that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--traffic-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="summarise four rocprofv3 counter_collection.csv files (the bench's and "
                         "the calibration copy's FETCH_SIZE and WRITE_SIZE runs) as markdown")
    return ap.parse_args()


# Size of the calibration copy: far beyond L2 and the last-level cache.
CALIB_BYTES = 1 << 30

# Kernel symbol fragment -> kernel name used in the bench output.
KERNEL_NAMES = (("fwd_mfma_kernel", "fwd"), ("bwd_pre_kernel", "bwd_preprocess"),
                ("bwd_fused_kernel", "bwd_grads"),
                ("bwd_dkdv_kernel", "bwd_dkdv"), ("bwd_dq_kernel", "bwd_dq"),
                ("decode_mfma_kernel<128, false>", "decode_merged"),
                ("lse_merge", "lse_merge"))

TRAFFIC_TAG = "traffic-json: "


def kernel_source_sha() -> str:
    """sha256 over the library's kernel sources: a counter summary taken from
    other sources no longer describes these kernels."""
    import hashlib
    d = os.path.join(ROOT, "attention_causal_gqa_flash_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.md")


def load_traffic(workload: str):
    """Per-kernel HBM bytes per launch from the committed counter summary of this
    workload, or None when there is none or the kernel sources changed since."""
    try:
        with open(traffic_file(workload)) as f:
            for line in f:
                if line.startswith(TRAFFIC_TAG):
                    t = json.loads(line[len(TRAFFIC_TAG):])
                    return t["kernels"] if t.get("source_sha") == kernel_source_sha() else None
    except OSError:
        pass
    return None


def read_counter_csv(path: str, counter: str) -> dict:
    """{kernel symbol: [per-dispatch values]} of one counter in a rocprofv3
    counter_collection.csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload) -> str:
    """Markdown summary of FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel,
    scaled to bytes by the calibration copy (which reads and writes CALIB_BYTES)."""
    fetch, write = read_counter_csv(fetch_csv, "FETCH_SIZE"), read_counter_csv(write_csv, "WRITE_SIZE")
    cf = [v for vals in read_counter_csv(copy_fetch_csv, "FETCH_SIZE").values() for v in vals]
    cw = [v for vals in read_counter_csv(copy_write_csv, "WRITE_SIZE").values() for v in vals]
    if not cf or not cw:
        raise SystemExit("no calibration dispatches in the copy runs")
    # median over the copy dispatches: KiB the counter reports for CALIB_BYTES moved
    kf, kw = sorted(cf)[len(cf) // 2], sorted(cw)[len(cw) // 2]
    sf, sw = CALIB_BYTES / (kf * 1024), CALIB_BYTES / (kw * 1024)
    lines = [f"calibration copy of {CALIB_BYTES} B: FETCH_SIZE {kf:.0f} KiB (scale {sf:.4f}), "
             f"WRITE_SIZE {kw:.0f} KiB (scale {sw:.4f})", "",
             "| kernel | dispatches | FETCH_SIZE KiB (mean) | WRITE_SIZE KiB (mean) | "
             "HBM read B (scaled) | HBM write B (scaled) |", "|---|---|---|---|---|---|"]
    kernels = {}
    for frag, name in KERNEL_NAMES:
        fv = [v for k, vals in fetch.items() if frag in k for v in vals]
        wv = [v for k, vals in write.items() if frag in k for v in vals]
        if not fv or not wv:
            continue
        mf, mw = sum(fv) / len(fv), sum(wv) / len(wv)
        rb, wb = mf * 1024 * sf, mw * 1024 * sw
        kernels[name] = {"read_bytes": round(rb), "write_bytes": round(wb), "bytes": round(rb + wb)}
        lines.append(f"| {name} | {len(fv)} | {mf:.1f} | {mw:.1f} | {rb:.0f} | {wb:.0f} |")
    lines += ["", TRAFFIC_TAG + json.dumps({"workload": workload, "source_sha": kernel_source_sha(),
                                            "kernels": kernels})]
    return "\n".join(lines)


def calibration_copy():
    import torch
    n = CALIB_BYTES // 4
    src = torch.empty(n, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": CALIB_BYTES, "dispatches": 5}), flush=True)


def eager_time_us(torch, fns, reps: int) -> float:
    """Run `fns` eagerly between HIP events; microseconds divided by `reps`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for fn in fns:
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


WARM_S = 0.05


def graph_time_us(torch, fns, reps: int) -> float:
    """Capture `fns` (a list of zero-argument launch callables) in a graph and
    return the replay time in microseconds divided by `reps`."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn in fns[: min(len(fns), 3)]:
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    # untimed replays for at least WARM_S seconds: the GPU's clocks ramp up over
    # the first tens of milliseconds of work (a single replay of a 40-step graph
    # of the B=4 workload measured 77.5 us per step, the third one 72.5)
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARM_S:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def main():
    args = parse()
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary, workload=args.workload))
        return
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on one GPU only; "
                                   "multi-GPU runs are not supported"}))
        sys.exit(2)

    import torch
    import attention_causal_gqa_flash_amd as attn
    from attention_causal_gqa_flash_amd import bounds as BD
    from attention_causal_gqa_flash_amd import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.calibration_copy:
        calibration_copy()
        return
    attn.lib()
    dev = torch.device("cuda:0")

    cfg = W.TRAIN_CONFIGS[args.workload]
    dcfg = W.C5
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    f32 = dict(device=dev, dtype=torch.float32)

    x = W.train_inputs(cfg)
    g = {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in x.items()}
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    o, lse, delta = torch.empty((B, Hq, N, d), **f32), torch.empty((B, Hq, N), **f32), \
        torch.empty((B, Hq, N), **f32)
    dq = torch.empty((B, Hq, N, d), **f32)
    dk, dv = torch.empty((B, Hkv, N, d), **f32), torch.empty((B, Hkv, N, d), **f32)

    xd = W.decode_inputs(dcfg)
    ddt = torch.bfloat16 if dcfg.dtype == "bf16" else torch.float32
    qd = torch.from_numpy(xd["q"]).to(dev).to(ddt)
    kc0 = torch.from_numpy(xd["k_cache"]).to(dev).to(ddt)
    vc0 = torch.from_numpy(xd["v_cache"]).to(dev).to(ddt)
    ncache = max(1, args.decode_caches)
    caches = [(kc0.clone(), vc0.clone()) for _ in range(ncache)]
    S = dcfg.n_splits
    part_o, part_lse = torch.empty((dcfg.B, dcfg.Hq, S, dcfg.d), **f32), \
        torch.empty((dcfg.B, dcfg.Hq, S), **f32)
    dec_o, dec_lse = torch.empty((dcfg.B, dcfg.Hq, dcfg.d), **f32), torch.empty((dcfg.B, dcfg.Hq), **f32)

    def fwd():
        attn.attn_fwd(g["q"], g["k"], g["v"], True, cfg.scale, o=o, lse=lse)

    def pre():
        attn.attn_bwd_preprocess(o, g["dout"], delta=delta)

    def dkdv():
        attn.attn_bwd_dkdv(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, cfg.scale,
                           dk=dk, dv=dv)

    def dqk():
        attn.attn_bwd_dq(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, cfg.scale, dq=dq)

    def grads():
        attn.attn_bwd_grads(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, cfg.scale, dq=dq,
                            dk=dk, dv=dv)

    dt_code = 1 if cfg.dtype == "bf16" else 0
    grads_one_kernel = attn.attn_bwd_grads_single_launch(dt_code, N, d, cfg.scale)

    bwd_ws = torch.empty(max(256, attn.attn_bwd_workspace_bytes(1 if cfg.dtype == "bf16" else 0,
                                                                B, Hq, Hkv, N, d)),
                         device=dev, dtype=torch.uint8)

    def bwd():
        # the whole backward as a caller runs it (dK/dV and dQ side by side)
        attn.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["dout"], True, cfg.scale, dq=dq, dk=dk,
                      dv=dv, workspace=bwd_ws)

    def decode(i):
        kc, vc = caches[i % ncache]
        return lambda: attn.attn_decode_merged(qd, kc, vc, S, dcfg.scale, part_o=part_o,
                                               part_lse=part_lse, o=dec_o, lse=dec_lse)

    # decode step with cache append (per-sequence lengths), outside the step:
    # rotates over distinct cache pairs so that its reads come from HBM
    acfg = W.C6
    xa = W.decode_append_inputs(acfg)
    ga = {n: torch.from_numpy(xa[n]).to(dev).to(ddt) for n in ("q", "k_new", "v_new")}
    a_lens = torch.from_numpy(xa["seq_lens"]).to(dev)
    ka0 = torch.from_numpy(xa["k_cache"]).to(dev).to(ddt)
    va0 = torch.from_numpy(xa["v_cache"]).to(dev).to(ddt)
    a_ncache = max(1, args.append_caches)
    a_caches = [(ka0.clone(), va0.clone()) for _ in range(a_ncache)]
    del ka0, va0
    a_po = torch.empty((acfg.B, acfg.Hq, acfg.n_splits, acfg.d), **f32)
    a_pl = torch.empty((acfg.B, acfg.Hq, acfg.n_splits), **f32)
    a_o, a_lse = torch.empty((acfg.B, acfg.Hq, acfg.d), **f32), torch.empty((acfg.B, acfg.Hq), **f32)

    # forward of a prefill chunk against a cache (attn_fwd_kv), outside the step
    ccfg = W.C7
    xc = W.chunk_inputs(ccfg)
    gc = {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in xc.items()}
    c_o = torch.empty((ccfg.B, ccfg.Hq, ccfg.Nq, ccfg.d), **f32)
    c_lse = torch.empty((ccfg.B, ccfg.Hq, ccfg.Nq), **f32)

    # the training step over rotated q and k (attn_fwd_rope / attn_bwd_rope), outside the step
    q_rot, k_rot = torch.empty_like(g["q"]), torch.empty_like(g["k"])

    def fwd_rope():
        attn.attn_fwd_rope(g["q"], g["k"], g["v"], True, cfg.scale, 10000.0, q_rot=q_rot, k_rot=k_rot,
                           o=o, lse=lse)

    def bwd_rope():
        attn.attn_bwd_rope(q_rot, k_rot, g["v"], o, lse, g["dout"], True, cfg.scale, 10000.0, dq=dq,
                           dk=dk, dv=dv, workspace=bwd_ws)

    def fwd_chunk():
        attn.attn_fwd_kv(gc["q"], gc["k"], gc["v"], True, ccfg.scale, o=c_o, lse=c_lse)

    def decode_append(i):
        kc, vc = a_caches[i % a_ncache]
        return lambda: attn.attn_decode_append(ga["q"], ga["k_new"], ga["v_new"], kc, vc, a_lens,
                                               acfg.n_splits, acfg.scale, part_o=a_po,
                                               part_lse=a_pl, o=a_o, lse=a_lse)

    train_op = [fwd, bwd]
    for s in range(args.warmup):
        for fn in train_op:
            fn()
        decode(s)()
        if not args.eager:
            decode_append(s)()
            fwd_chunk()
    torch.cuda.synchronize()

    K = args.steps
    timer = eager_time_us if args.eager else graph_time_us
    train_fns = [fn for _ in range(K) for fn in train_op]
    dec_fns = [decode(s) for s in range(K)]
    # the timed region: K steps = K training ops and K decode ops
    train_us = timer(torch, train_fns, K)
    dec_us = timer(torch, dec_fns, K)
    step_us = train_us + dec_us
    # the measurements beside the step (skipped in the eager counter-collection
    # runs, whose per-kernel counters must describe the step's kernels alone)
    extras = {"decode_append": None, "fwd_chunk": None, "fwd_bwd_rope": None}
    if not args.eager:
        app_us = timer(torch, [decode_append(s) for s in range(K)], K)
        app_bytes = acfg.algorithmic_bytes()
        app_gbs = app_bytes / (app_us * 1e-6) / 1e9
        extras["decode_append"] = {"workload": acfg.name, "GB_per_s": round(app_gbs, 1),
                                   "frac_hbm_peak": round(app_gbs / PEAK_HBM_GBS, 4),
                                   "us_per_call": round(app_us, 3), "bytes": app_bytes,
                                   "distinct_caches": a_ncache, "launches_per_call": 2,
                                   "seq_lens": list(acfg.seq_lens),
                                   # the caches rotate through HBM: compulsory bytes at its peak
                                   "floor_us": round(app_bytes / (BD.PEAK_HBM / 1e6), 3),
                                   "of_floor": round(app_bytes / (BD.PEAK_HBM / 1e6) / app_us, 4)}
        rope_us = timer(torch, [f for _ in range(K) for f in (fwd_rope, bwd_rope)], K)
        extras["fwd_bwd_rope"] = {"us_per_step": round(rope_us, 3),
                                  "TFLOP_s": round((cfg.fwd_flop + cfg.bwd_flop) / (rope_us * 1e-6) / 1e12, 2),
                                  "rotary_cost_us": round(rope_us - train_us, 3)}
        chunk_us = timer(torch, [fwd_chunk] * K, K)
        chunk_tflops = ccfg.fwd_flop / (chunk_us * 1e-6) / 1e12
        cf = BD.fwd(ccfg.B, ccfg.Hq, ccfg.Hkv, ccfg.Nq, ccfg.Nk, ccfg.d, True,
                    **BD.fwd_tile(ccfg.B, ccfg.Hq, ccfg.Nq, ccfg.d))
        extras["fwd_chunk"] = {"workload": ccfg.name, "TFLOP_s": round(chunk_tflops, 2),
                               "frac_bf16_peak": round(chunk_tflops / PEAK_BF16_TFLOPS, 4),
                               "us_per_call": round(chunk_us, 3), "flop": ccfg.fwd_flop,
                               "floor_us": cf["floor_us"], "of_floor": round(cf["floor_us"] / chunk_us, 4)}

    pairs = cfg.pairs
    train_flop = cfg.fwd_flop + cfg.bwd_flop
    value = train_flop / (train_us * 1e-6) / 1e12
    dec_bytes = dcfg.algorithmic_bytes()
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9

    flop = {"fwd": 4 * d * pairs,
            "bwd_grads": 10 * d * pairs,    # the whole gradient stage
            "bwd_dkdv": 8 * d * pairs,      # recomputed S, dP, dV, dK
            "bwd_dq": 2 * d * pairs}        # dQ (its S and dP recompute is not credited)
    kernels = {}
    if not args.no_kernel_breakdown:
        for name, fn in (("fwd", fwd), ("bwd_preprocess", pre), ("bwd_grads", grads),
                         ("bwd_dkdv", dkdv), ("bwd_dq", dqk)):
            kernels[name] = {"avg_us": round(timer(torch, [fn] * K, K), 3)}
        kernels["bwd_grads"]["one_kernel"] = grads_one_kernel
        kernels["decode_merged"] = {"avg_us": round(dec_us, 3)}
        for n, f in flop.items():
            t = kernels[n]["avg_us"] * 1e-6
            kernels[n]["TFLOP_s"] = round(f / t / 1e12, 2)
            kernels[n]["frac_bf16_peak"] = round(f / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        pre_bytes = B * Hq * N * d * (2 if cfg.dtype == "bf16" else 4) + B * Hq * N * d * 4 + B * Hq * N * 4
        kernels["bwd_preprocess"]["GB_s"] = round(pre_bytes / (kernels["bwd_preprocess"]["avg_us"] * 1e-6) / 1e9, 1)
        kernels["decode_merged"]["GB_s"] = round(dec_gbs, 1)

    # time floors from the tile sizes (bounds.py), next to each measured time
    if kernels and cfg.dtype == "bf16":
        ft = BD.fwd_tile(B, Hq, N, d)
        hs = BD.head_split(B, Hq, Hkv, N)
        kv = dict(BKV=64, SR=128, hs=hs)
        floors = {
            "fwd": (BD.fwd(B, Hq, Hkv, N, N, d, True, **ft), BD.best_fwd(B, Hq, Hkv, N, N, d)),
            "bwd_preprocess": (BD.preprocess(B, Hq, Hkv, N, d, hs > 1), None),
            "bwd_grads": (BD.bwd_grads(B, Hq, Hkv, N, N, d, True, BQ=128, BN=64, **kv),
                          BD.best_bwd_grads(B, Hq, Hkv, N, N, d)),
            "bwd_dkdv": (BD.bwd_dkdv(B, Hq, Hkv, N, N, d, True, **kv), BD.best_bwd_dkdv(B, Hq, Hkv, N, N, d)),
            "bwd_dq": (BD.bwd_dq(B, Hq, Hkv, N, N, d, True, 128, 64), BD.best_bwd_dq(B, Hq, Hkv, N, N, d)),
            "decode_merged": (BD.decode(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.L, dcfg.d, dcfg.n_splits, resident=False),
                              BD.best_decode(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.L, dcfg.d, resident=False)),
        }
        for n, (fl, best) in floors.items():
            k = kernels[n]
            k["floor_us"] = fl["floor_us"]
            k["floor_bound"] = max(fl["terms_us"], key=fl["terms_us"].get)
            k["of_floor"] = round(fl["floor_us"] / k["avg_us"], 4)
            k["tile"] = fl["tile"]
            if best is not None:
                k["best_tile"], k["best_floor_us"] = best["tile"], best["floor_us"]

    traffic = load_traffic(cfg.name)
    if traffic:
        for n, t in traffic.items():
            if n in kernels:
                kernels[n]["hbm_bytes_measured"] = t["bytes"]

    roof = None
    if kernels:
        # the kernels the training step launches: the gradient stage is one
        # kernel (bwd_grads) or the dK/dV and dQ kernels
        in_step = ["fwd", "bwd_preprocess", "decode_merged"] + (
            ["bwd_grads"] if grads_one_kernel else ["bwd_dkdv", "bwd_dq"])
        dom = max(in_step, key=lambda n: kernels[n]["avg_us"])
        t = kernels[dom]["avg_us"]
        if dom in flop:
            ach = flop[dom] / (t * 1e-6) / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic[dom]["bytes"] if traffic and dom in traffic else None,
                    "avg_launch_us": t}
            for key in ("floor_us", "floor_bound", "of_floor", "tile", "best_tile", "best_floor_us"):
                if key in kernels[dom]:
                    roof[key] = kernels[dom][key]
        else:
            ach = kernels[dom]["GB_s"]
            roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                    "traffic": traffic[dom]["bytes"] if traffic and dom in traffic else None,
                    "avg_launch_us": t}

    result = {
        "metric": "attn fwd+bwd TFLOP/s & % bf16 MFMA peak; decode GB/s & % HBM peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "Hq": Hq, "Hkv": Hkv, "seq_len": N, "head_dim": d,
                   "causal": True, "decode_workload": dcfg.name},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_bwd_us": round(train_us, 3),
        # the step's kernels run one after another: their floors add (the two
        # gradient kernels, side by side at d = 128, share the CUs: one floor)
        "fwd_bwd_floor_us": (round(sum(kernels[n]["floor_us"] for n in ("fwd", "bwd_preprocess", "bwd_grads")), 3)
                             if "floor_us" in kernels.get("fwd", {}) else None),
        "decode": {"GB_per_s": round(dec_gbs, 1), "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "us_per_call": round(dec_us, 3), "bytes": dec_bytes, "distinct_caches": ncache,
                   "launches_per_call": 2},
        "decode_append": extras["decode_append"],
        "fwd_chunk": extras["fwd_chunk"],
        "fwd_bwd_rope": extras["fwd_bwd_rope"],
        "kernels": kernels,
        "roofline": roof,
        "timing": ("eager launches between HIP events" if args.eager else
                   "HIP graph replay of K back-to-back ops between HIP events"),
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
    while time.perf_counter() - t0 < budget_s and done < 64 * len(groups):
        b, g = groups[done % len(groups)]
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
            "sample": f"{done} (batch, kv-group) slices of {cfg.name} ({len(groups)} per pass), "
                      f"fwd+bwd in f64, {el:.1f} s"}


if __name__ == "__main__":
    main()
