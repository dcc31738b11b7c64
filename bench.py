#!/usr/bin/env python3
"""Benchmark of the causal GQA flash-attention hot path on one MI355X.

One step = one pass of the whole hot path on seeded synthetic inputs already
resident in device memory:
  * the training op: attn_fwd, then attn_bwd on the headline training workload
    (default: the largest one, bf16, B=1, 32 query / 8 key-value heads,
    N=4096, d=128; at d=128 attn_bwd runs the dQ kernel, which also computes
    the preprocess's row terms, then the dK/dV kernel; at d=64 the preprocess
    then one kernel holding both the dK/dV and the dQ work), each step on the
    next of several distinct sets of inputs and outputs (more than 512 MB
    together, twice the last-level cache), so that every step reads its
    inputs from HBM; `train_input_sets` gives the count and the training
    op's time on one set, whose inputs stay cached from step to step;
  * the decode op: split-KV decode + LSE merge (attn_decode_merged: the decode
    kernel then the merge kernel) on the decode workload (bf16, 32/8 heads,
    d=128, a 4096-key cache in 16 splits), each step on the next of 24
    distinct caches (24 x 16 MiB, more than L2 and the 256 MB last-level
    cache), so that every step reads its keys and values from HBM.

Timing.  Launches are captured into HIP graphs (the same C-ABI calls an
eager caller makes, without host launch overhead).  The timed region: after W
untimed warm-up steps, K steps run as R replays of a graph of M = 10 steps,
queued back to back between two device synchronisations, each replay between
its own pair of HIP events; `ms_per_step` is the whole region divided by K,
`step_us_median` the median replay divided by M.  `value` is the headline
workload's algorithmic fwd+bwd TFLOP/s (4*d flop per unmasked (query, key)
pair forward, 10*d backward) at the MEDIAN time of the training op alone, and
`decode` the decode op's GB/s at its median (each over >= 100 replays of a
graph of ~2 ms of that op: a graph launch costs the GPU about 10 us of its
own, which that amortises).

Beside the step (reported, not timed into `ms_per_step`):
  * `configs`: every training config (C1 f32 tiny; C2 4x1024 d64; C3 N=128
    and 512 d128; C4 4096 d128) -- fwd alone, attn_bwd alone and fwd+bwd,
    each the median of >= 100 replays of ~2 ms graphs; decode cold (24-cache
    rotation), warm (one cache, labelled), the decode kernel alone and the
    read floor (attn_read_probe streaming the same 16 MiB per call over the
    same rotation);
  * `kernels`: each kernel of the headline step timed alone (median of
    iterations of a graph of launches of that kernel), with its algorithmic
    TFLOP/s, the time floor of its tiling (bounds.py) and, while the kernel
    sources are those the counters were taken from, its measured HBM bytes;
  * `roofline`: the kernel with the largest share of the step;
  * `fwd_chunk` (attn_fwd_kv, a 512-token prefill chunk against 4096 keys),
    `decode_append` (8 sequences of their own lengths, cache append) and
    `fwd_bwd_rope` (the headline step over rotated q and k);
  * `cpu_baseline`: the CPU f64 oracle on the headline workload, one key/value
    group at a time until the time budget is spent (all 8 groups of the 4096-
    token workload take about 25 s on 16 threads), with the core count and
    the CPU model; `configs[*].oracle_s` times the oracle per config (best of 3
    for C1-C3 and decode, the one run above for C4).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 bf16 flop/clk/CU (dense)
PEAK_HBM_GBS = 8000.0          # 8 TB/s HBM3E
HEADLINE = "gqa32x8_b1_n4096_d128"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE,
                    help="headline training workload (see workloads.TRAIN_CONFIGS)")
    ap.add_argument("--decode-caches", type=int, default=24,
                    help="distinct KV caches the decode op rotates over (cold-cache reads)")
    ap.add_argument("--append-caches", type=int, default=4,
                    help="distinct cache pairs the decode-append measurement rotates over")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="time budget of the oracle CPU baseline on the headline workload "
                         "(0 disables every oracle timing)")
    ap.add_argument("--min-iters", type=int, default=100,
                    help="iterations per median (each also spans >= 200 ms)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table")
    ap.add_argument("--no-kernel-breakdown", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip fwd_chunk, decode_append and fwd_bwd_rope")
    ap.add_argument("--eager", action="store_true",
                    help="launch eagerly instead of replaying graphs (for counter collection: "
                         "only the K timed steps run)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="only run a plain device-to-device copy of known size (the reference "
                         "dispatch that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--traffic-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="summarise four rocprofv3 counter_collection.csv files (the bench's and "
                         "the calibration copy's FETCH_SIZE and WRITE_SIZE runs) as markdown")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 counter_collection.csv files of SQ/GRBM counter "
                         "passes (MFMA busy, LDS, VALU, waits per kernel) as markdown")
    return ap.parse_args()


# The training op rotates over input sets of at least this many bytes together
# (twice the 256 MB last-level cache), at most TRAIN_MAX_SETS of them.
TRAIN_ROTATE_BYTES = 512 << 20
TRAIN_MAX_SETS = 32

# Size of the calibration copy: far beyond L2 and the last-level cache.
CALIB_BYTES = 1 << 30

# Kernel symbol fragment -> kernel name used in the bench output.
KERNEL_NAMES = (("fwd_mfma_kernel", "fwd"), ("bwd_pre_kernel", "bwd_preprocess"),
                ("bwd_fused_kernel", "bwd_grads"),
                ("bwd_dkdv", "bwd_dkdv"), ("bwd_dq_kernel", "bwd_dq"),
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


# gfx950 (MI355X): 8 XCDs x 32 CUs x 4 SIMDs
XCDS, CUS, SIMDS = 8, 256, 1024


def counter_summary(csvs) -> str:
    """Markdown summary of SQ/GRBM counter passes per kernel (means over dispatches).

    rocprofv3 reports each counter summed over its hardware instances:
    GRBM_GUI_ACTIVE over the 8 XCDs (so the cycles of one XCD, the dispatch's
    active clock count, are that / 8); SQ counters over every SE / SIMD.
      MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x 1024 SIMDs)
      bf16 flop  = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
      LDS busy   = SQ_LDS_IDX_ACTIVE / (GUI cycles x 256 CUs)
      conflicts  = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      clock      = GUI cycles / kernel duration
    """
    import csv
    import re
    agg, dur = {}, {}
    for path in csvs:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                k = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                if "attn::" not in k:
                    continue
                k = re.sub(r"^void attn::", "", k.split("(")[0]).strip()
                agg.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                dur.setdefault(k, {})[(path, r["Dispatch_Id"])] = \
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lines = ["| kernel | dispatches | duration us (median) | clock GHz | MFMA busy % | bf16 GFLOP "
             "executed | LDS busy % | LDS conflict cycles % | VALU insts / MFMA insts | "
             "LDS wait % of wave cycles | any-wait % of wave cycles |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(agg):
        m = {n: sum(v) / len(v) for n, v in agg[k].items()}
        ds = sorted(dur[k].values())
        t_us = ds[len(ds) // 2] / 1e3
        gui = m.get("GRBM_GUI_ACTIVE", 0.0) / XCDS

        def pct(num, den):
            return f"{100.0 * num / den:.1f}" if num is not None and den else "-"
        mfma = m.get("SQ_VALU_MFMA_BUSY_CYCLES")
        mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        lds = m.get("SQ_LDS_IDX_ACTIVE")
        conf = m.get("SQ_LDS_BANK_CONFLICT")
        valu, nm = m.get("SQ_INSTS_VALU"), m.get("SQ_INSTS_MFMA")
        wc = m.get("SQ_WAVE_CYCLES")
        wl, wa = m.get("SQ_WAIT_INST_LDS"), m.get("SQ_WAIT_INST_ANY")
        lines.append(
            f"| {k} | {len(ds)} | {t_us:.1f} | {gui / t_us / 1e3:.2f} | "
            f"{pct(mfma, gui * SIMDS)} | {(mops or 0) * 512 / 1e9:.1f} | {pct(lds, gui * CUS)} | "
            f"{pct(conf, lds)} | {(valu / nm if valu and nm else float('nan')):.2f} | "
            f"{pct(wl, wc)} | {pct(wa, wc)} |")
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


WARM_S = 0.05


class Timer:
    """Graph-replay timing with HIP events (torch.cuda.Event records on the
    current stream, which is the stream every captured launch runs on)."""

    def __init__(self, torch, min_iters: int, min_ms: float = 200.0):
        self.torch, self.min_iters, self.min_ms = torch, min_iters, min_ms

    def graph(self, fns):
        """Capture the zero-argument launch callables `fns` into one graph."""
        torch = self.torch
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
        torch.cuda.synchronize()
        return g

    def warm(self, g):
        # the GPU's clocks ramp up over the first tens of milliseconds of work
        t0 = time.perf_counter()
        while True:
            g.replay()
            self.torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_S:
                break

    def median_us(self, fns, per_replay: int = 1) -> dict:
        """Median over >= min_iters iterations (and >= min_ms) of one replay of a
        graph of `fns`, each bracketed by its own events; microseconds per op
        (`per_replay` ops per replay)."""
        torch = self.torch
        g = self.graph(fns)
        self.warm(g)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        one_ms = max(e0.elapsed_time(e1), 1e-3)
        iters = max(self.min_iters, math.ceil(self.min_ms / one_ms))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 / per_replay for a, b in ev)
        return {"median_us": round(statistics.median(ts), 3), "mean_us": round(sum(ts) / len(ts), 3),
                "min_us": round(ts[0], 3), "iters": iters}

    def ops_for(self, fn, target_us: float = 2000.0) -> int:
        """How many launches of `fn` make a replay of about target_us: a graph
        launch costs the GPU several microseconds of its own (about 10 us
        measured on MI355X between back-to-back one-op replays), which a
        replay of ~2 ms amortises to well under 1%."""
        t = self.median_once(fn)
        return max(1, min(512, math.ceil(target_us / max(t, 0.5))))

    def median_once(self, fn) -> float:
        torch = self.torch
        g = self.graph([fn])
        self.warm(g)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / 5

    def op(self, fn) -> dict:
        n = self.ops_for(fn)
        r = self.median_us([fn] * n, n)
        r["ops_per_replay"] = n
        return r


def main():
    args = parse()
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary, workload=args.workload))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
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
    T = Timer(torch, args.min_iters)
    f32 = dict(device=dev, dtype=torch.float32)

    def train_setup(cfg, like=None):
        """Device inputs and outputs of a training workload, and its launch callables
        (like: the device inputs of another set, copied instead of drawn again)."""
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        x = W.train_inputs(cfg) if like is None else None
        g = ({n: torch.from_numpy(a).to(dev).to(tdt) for n, a in x.items()} if like is None
             else {n: a.clone() for n, a in like.items()})
        B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
        t = {"o": torch.empty((B, Hq, N, d), **f32), "lse": torch.empty((B, Hq, N), **f32),
             "delta": torch.empty((B, Hq, N), **f32), "dq": torch.empty((B, Hq, N, d), **f32),
             "dk": torch.empty((B, Hkv, N, d), **f32), "dv": torch.empty((B, Hkv, N, d), **f32)}
        code = 1 if cfg.dtype == "bf16" else 0
        t["ws"] = torch.empty(max(256, attn.attn_bwd_workspace_bytes(code, B, Hq, Hkv, N, d)),
                              device=dev, dtype=torch.uint8)
        s = cfg.scale
        fn = {
            "fwd": lambda: attn.attn_fwd(g["q"], g["k"], g["v"], True, s, o=t["o"], lse=t["lse"]),
            "bwd": lambda: attn.attn_bwd(g["q"], g["k"], g["v"], t["o"], t["lse"], g["dout"], True, s,
                                         dq=t["dq"], dk=t["dk"], dv=t["dv"], workspace=t["ws"]),
            "bwd_preprocess": lambda: attn.attn_bwd_preprocess(t["o"], g["dout"], delta=t["delta"]),
            "bwd_dkdv": lambda: attn.attn_bwd_dkdv(g["q"], g["k"], g["v"], t["lse"], g["dout"],
                                                   t["delta"], True, s, dk=t["dk"], dv=t["dv"]),
            "bwd_dq": lambda: attn.attn_bwd_dq(g["q"], g["k"], g["v"], t["lse"], g["dout"], t["delta"],
                                               True, s, dq=t["dq"]),
            "bwd_grads": lambda: attn.attn_bwd_grads(g["q"], g["k"], g["v"], t["lse"], g["dout"],
                                                     t["delta"], True, s, dq=t["dq"], dk=t["dk"],
                                                     dv=t["dv"]),
        }
        return x, g, t, fn

    cfg = W.TRAIN_CONFIGS[args.workload]
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    x, g, tt, fns = train_setup(cfg)
    # The training op runs on distinct sets of inputs and outputs in turn, as
    # many as make more than TRAIN_ROTATE_BYTES together (twice the 256 MB
    # last-level cache), so that each step reads its inputs from HBM rather
    # than finding the previous step's copy cached.
    set_bytes = sum(a.numel() * a.element_size() for a in list(g.values()) + list(tt.values()))
    nsets = int(min(TRAIN_MAX_SETS, max(2, math.ceil(TRAIN_ROTATE_BYTES / set_bytes))))
    train_sets = [(g, tt, fns)] + [train_setup(cfg, like=g)[1:] for _ in range(nsets - 1)]
    fns["fwd"]()
    fns["bwd_preprocess"]()
    torch.cuda.synchronize()

    # decode workload: K and V of each cache pair in one allocation (the read
    # probe streams both in one launch)
    dcfg = W.C5
    ddt = torch.bfloat16 if dcfg.dtype == "bf16" else torch.float32
    xd = W.decode_inputs(dcfg)
    qd = torch.from_numpy(xd["q"]).to(dev).to(ddt)
    kv0 = torch.stack([torch.from_numpy(xd["k_cache"]), torch.from_numpy(xd["v_cache"])]).to(dev).to(ddt)
    ncache = max(1, args.decode_caches)
    caches = [kv0.clone() for _ in range(ncache)]
    del kv0
    S = dcfg.n_splits
    part_o, part_lse = torch.empty((dcfg.B, dcfg.Hq, S, dcfg.d), **f32), \
        torch.empty((dcfg.B, dcfg.Hq, S), **f32)
    dec_o, dec_lse = torch.empty((dcfg.B, dcfg.Hq, dcfg.d), **f32), torch.empty((dcfg.B, dcfg.Hq), **f32)
    probe_out = torch.zeros(1, device=dev, dtype=torch.int32)

    def decode(i):
        kv = caches[i % ncache]
        return lambda: attn.attn_decode_merged(qd, kv[0], kv[1], S, dcfg.scale, part_o=part_o,
                                               part_lse=part_lse, o=dec_o, lse=dec_lse)

    def decode_only(i):
        kv = caches[i % ncache]
        return lambda: attn.attn_decode(qd, kv[0], kv[1], S, dcfg.scale, part_o=part_o,
                                        part_lse=part_lse)

    def probe(i):
        kv = caches[i % ncache]
        return lambda: attn.attn_read_probe(kv, out=probe_out)

    def train_op(i):
        f = train_sets[i % nsets][2]
        return lambda: (f["fwd"](), f["bwd"]())

    # ---------------------------------------------------------------- the timed region
    # K steps = R replays of a graph of M steps (each step: the training op,
    # then the decode op on the next cache), every replay between its own pair
    # of HIP events, the replays queued back to back between two device
    # synchronisations
    Wm = args.warmup
    M = max(1, min(args.steps, 10))
    R = max(1, math.ceil(args.steps / M))
    K = R * M
    if args.eager:
        for s in range(Wm):
            train_op(s)()
            decode(s)()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(R)]
        torch.cuda.synchronize()
        for r in range(R):
            ev[r][0].record()
            for s in range(M):
                train_op(r * M + s)()
                decode(r * M + s)()
            ev[r][1].record()
        torch.cuda.synchronize()
    else:
        steps = [f for s in range(M) for f in (train_op(s), decode(s))]
        g_step = T.graph(steps)
        for _ in range(max(1, math.ceil(Wm / M))):
            g_step.replay()
        T.warm(g_step)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(R)]
        torch.cuda.synchronize()
        for r in range(R):
            ev[r][0].record()
            g_step.replay()
            ev[r][1].record()
        torch.cuda.synchronize()
    total_ms = ev[0][0].elapsed_time(ev[-1][1])
    step_ts = sorted(e[0].elapsed_time(e[1]) * 1e3 / M for e in ev)
    step_med_us = statistics.median(step_ts)
    train_flop = cfg.fwd_flop + cfg.bwd_flop
    dec_bytes = dcfg.algorithmic_bytes()
    if args.eager:
        train_us = dec_us = float("nan")
        value = float("nan")
    else:
        # the two ops of the step, each timed alone: medians over >= 100 replays
        # of graphs of ~2 ms of that op (the training op rotating over its input
        # sets; the decode op rotating over the caches); and the training op on
        # one set, whose inputs then stay cached between steps
        nt = max(nsets, T.ops_for(train_op(0)) // nsets * nsets)
        tr = T.median_us([train_op(i) for i in range(nt)], nt)
        tr_one = T.op(train_op(0))
        nd = max(ncache, T.ops_for(decode(0)) // ncache * ncache)
        dr = T.median_us([decode(i) for i in range(nd)], nd)
        train_us, dec_us = tr["median_us"], dr["median_us"]
        value = train_flop / (train_us * 1e-6) / 1e12
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9

    result = {
        "metric": "attn fwd+bwd TFLOP/s & % bf16 MFMA peak; decode GB/s & % HBM peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(total_ms / K, 5),
        "step_us_median": round(step_med_us, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "Hq": Hq, "Hkv": Hkv, "seq_len": N, "head_dim": d,
                   "causal": True, "decode_workload": dcfg.name},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_bwd_us": round(train_us, 3),
        "train_input_sets": {"sets": nsets, "bytes_per_set": set_bytes,
                             "fwd_bwd_us_one_set": None if args.eager else tr_one["median_us"]},
        "decode": {"GB_per_s": round(dec_gbs, 1), "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "us_per_call": round(dec_us, 3), "bytes": dec_bytes, "distinct_caches": ncache,
                   "launches_per_call": 2},
        "timing": ("eager launches" if args.eager else
                   f"K steps as {R} replays of a graph of {M} steps between HIP events "
                   f"(ms_per_step, step_us_median); value, fwd_bwd_us and decode: medians over "
                   f">= {args.min_iters} replays of graphs of ~2 ms of that op alone"),
    }
    if args.eager:
        print(json.dumps(result), flush=True)
        return

    # ---------------------------------------------------------------- per kernel
    pairs = cfg.pairs
    flop = {"fwd": 4 * d * pairs,
            "bwd_grads": 10 * d * pairs,    # the whole gradient stage
            "bwd_dkdv": 8 * d * pairs,      # recomputed S, dP, then dV, dK
            "bwd_dq": 2 * d * pairs}        # dQ (its S and dP recompute is not credited)
    dt_code = 1 if cfg.dtype == "bf16" else 0
    grads_one_kernel = attn.attn_bwd_grads_plan(dt_code, B, Hq, Hkv, N, N, d, True, cfg.scale)[0]
    kernels = {}
    if not args.no_kernel_breakdown:
        for name in ("fwd", "bwd_preprocess", "bwd_grads", "bwd_dkdv", "bwd_dq"):
            r = T.op(fns[name])
            kernels[name] = {"avg_us": r["median_us"], "iters": r["iters"],
                             "launches_per_replay": r["ops_per_replay"]}
        kernels["bwd_grads"]["one_kernel"] = grads_one_kernel
        for n, fl in flop.items():
            t = kernels[n]["avg_us"] * 1e-6
            kernels[n]["TFLOP_s"] = round(fl / t / 1e12, 2)
            kernels[n]["frac_bf16_peak"] = round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        esz = 2 if cfg.dtype == "bf16" else 4
        pre_bytes = B * Hq * N * d * esz + B * Hq * N * d * 4 + B * Hq * N * 4
        kernels["bwd_preprocess"]["GB_s"] = round(pre_bytes / (kernels["bwd_preprocess"]["avg_us"] * 1e-6) / 1e9, 1)
        kernels["decode_merged"] = {"avg_us": round(dec_us, 3), "GB_s": round(dec_gbs, 1)}
        if cfg.dtype == "bf16":
            ft = BD.fwd_tile(B, Hq, N, d)
            # the dK/dV kernel's tile: 128 keys x 64 query rows per step at
            # d = 128 when the 128-key tiles number at least a quarter of the
            # CUs, else 64 keys x 128 rows
            use128 = d == 128 and 4 * -(-N // 128) * B * Hkv >= BD.CUS
            bkv, sr = (128, 64) if use128 else (64, 128)
            hs = BD.head_split(B, Hq, Hkv, N, BKV=bkv)
            kv = dict(BKV=bkv, SR=sr, hs=hs)
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
    else:
        traffic = None
    result["kernels"] = kernels

    roof = None
    if kernels:
        # the kernels the training step launches: the gradient stage is one
        # kernel (bwd_grads) or the dQ and dK/dV kernels; the d = 128 step's dQ
        # kernel also computes the preprocess's row terms (timed as bwd_dq
        # without them)
        in_step = ["fwd", "decode_merged"] + (["bwd_preprocess", "bwd_grads"] if grads_one_kernel
                                              else ["bwd_dkdv", "bwd_dq"])
        dom = max(in_step, key=lambda n: kernels[n]["avg_us"])
        t = kernels[dom]["avg_us"]
        if dom in flop:
            ach = flop[dom] / (t * 1e-6) / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic[dom]["bytes"] if traffic and dom in traffic else None,
                    "avg_launch_us": t, "flop_per_launch": flop[dom]}
            for key in ("floor_us", "floor_bound", "of_floor", "tile", "best_tile", "best_floor_us"):
                if key in kernels[dom]:
                    roof[key] = kernels[dom][key]
        else:
            ach = kernels[dom]["GB_s"]
            roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                    "traffic": traffic[dom]["bytes"] if traffic and dom in traffic else None,
                    "avg_launch_us": t}
    result["roofline"] = roof

    # ---------------------------------------------------------------- every config
    configs = {}
    if not args.no_configs:
        for c in (W.C1, W.C2, W.C3_128, W.C3_512, W.C4):
            if c.name == cfg.name:
                cx, cf = x, fns
            else:
                cx, _, _, cf = train_setup(c)
            row = {"shape": f"B{c.B} Hq{c.Hq} Hkv{c.Hkv} N{c.N} d{c.d} {c.dtype}"}
            for name, ops, fl in (("fwd", [cf["fwd"]], c.fwd_flop), ("bwd", [cf["bwd"]], c.bwd_flop),
                                  ("fwd_bwd", [cf["fwd"], cf["bwd"]], c.fwd_flop + c.bwd_flop)):
                n = T.ops_for(lambda: [f() for f in ops])
                r = T.median_us(ops * n, n)
                row[f"{name}_us"] = r["median_us"]
                if c.dtype == "bf16":
                    tf = fl / (r["median_us"] * 1e-6) / 1e12
                    row[f"{name}_TFLOP_s"] = round(tf, 2)
                    row[f"{name}_frac_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
            row["iters_min"] = args.min_iters
            configs[c.name] = row
            if c.name != cfg.name:
                del cf
            torch.cuda.synchronize()
        cold = T.median_us([decode(i) for i in range(ncache)], ncache)
        warm = T.median_us([decode(0)] * ncache, ncache)
        kern = T.median_us([decode_only(i) for i in range(ncache)], ncache)
        floor = T.median_us([probe(i) for i in range(ncache)], ncache)
        merge_only = T.op(lambda: attn.attn_lse_merge(part_o, part_lse, o=dec_o, lse=dec_lse))
        rb = 2 * dcfg.B * dcfg.Hkv * dcfg.L * dcfg.d * 2
        configs[dcfg.name] = {
            "shape": f"q B{dcfg.B} Hq{dcfg.Hq} d{dcfg.d}; caches Hkv{dcfg.Hkv} L{dcfg.L} bf16; "
                     f"{S} splits",
            "decode_merged_us": cold["median_us"],
            "GB_per_s": round(dec_bytes / (cold["median_us"] * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(dec_bytes / (cold["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "decode_kernel_us": kern["median_us"],
            "lse_merge_us": merge_only["median_us"],
            "warm_cache_decode_merged_us (one cache, L2/LLC-resident)": warm["median_us"],
            "read_floor_us": floor["median_us"],
            "read_floor_GB_per_s": round(rb / (floor["median_us"] * 1e-6) / 1e9, 1),
            "of_read_floor": round(floor["median_us"] / cold["median_us"], 4),
            # the op is two launches (the partials must be complete before any
            # merge): its floor is one streaming read of the caches plus one
            # merge launch
            "two_launch_floor_us": round(floor["median_us"] + merge_only["median_us"], 3),
            "of_two_launch_floor": round((floor["median_us"] + merge_only["median_us"]) / cold["median_us"], 4),
            "distinct_caches": ncache,
        }
    result["configs"] = configs

    # ---------------------------------------------------------------- beside the step
    extras = {"fwd_chunk": None, "decode_append": None, "fwd_bwd_rope": None}
    if not args.no_extras:
        acfg = W.C6
        xa = W.decode_append_inputs(acfg)
        ga = {n: torch.from_numpy(xa[n]).to(dev).to(ddt) for n in ("q", "k_new", "v_new")}
        a_lens = torch.from_numpy(xa["seq_lens"]).to(dev)
        ka0 = torch.from_numpy(xa["k_cache"]).to(dev).to(ddt)
        va0 = torch.from_numpy(xa["v_cache"]).to(dev).to(ddt)
        a_n = max(1, args.append_caches)
        a_caches = [(ka0.clone(), va0.clone()) for _ in range(a_n)]
        del ka0, va0
        a_po = torch.empty((acfg.B, acfg.Hq, acfg.n_splits, acfg.d), **f32)
        a_pl = torch.empty((acfg.B, acfg.Hq, acfg.n_splits), **f32)
        a_o, a_lse = torch.empty((acfg.B, acfg.Hq, acfg.d), **f32), torch.empty((acfg.B, acfg.Hq), **f32)

        def decode_append(i):
            kc, vc = a_caches[i % a_n]
            return lambda: attn.attn_decode_append(ga["q"], ga["k_new"], ga["v_new"], kc, vc, a_lens,
                                                   acfg.n_splits, acfg.scale, part_o=a_po,
                                                   part_lse=a_pl, o=a_o, lse=a_lse)
        app_us = T.median_us([decode_append(i) for i in range(8 * a_n)], 8 * a_n)["median_us"]
        app_bytes = acfg.algorithmic_bytes()
        app_gbs = app_bytes / (app_us * 1e-6) / 1e9
        extras["decode_append"] = {"workload": acfg.name, "GB_per_s": round(app_gbs, 1),
                                   "frac_hbm_peak": round(app_gbs / PEAK_HBM_GBS, 4),
                                   "us_per_call": app_us, "bytes": app_bytes,
                                   "distinct_caches": a_n, "launches_per_call": 2,
                                   "seq_lens": list(acfg.seq_lens)}

        ccfg = W.C7
        xc = W.chunk_inputs(ccfg)
        tdt = torch.bfloat16 if ccfg.dtype == "bf16" else torch.float32
        gc = {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in xc.items()}
        c_o = torch.empty((ccfg.B, ccfg.Hq, ccfg.Nq, ccfg.d), **f32)
        c_lse = torch.empty((ccfg.B, ccfg.Hq, ccfg.Nq), **f32)
        chunk_us = T.op(lambda: attn.attn_fwd_kv(gc["q"], gc["k"], gc["v"], True, ccfg.scale, o=c_o,
                                                 lse=c_lse))["median_us"]
        chunk_tf = ccfg.fwd_flop / (chunk_us * 1e-6) / 1e12
        cfl = BD.fwd(ccfg.B, ccfg.Hq, ccfg.Hkv, ccfg.Nq, ccfg.Nk, ccfg.d, True,
                     **BD.fwd_tile(ccfg.B, ccfg.Hq, ccfg.Nq, ccfg.d))
        extras["fwd_chunk"] = {"workload": ccfg.name, "TFLOP_s": round(chunk_tf, 2),
                               "frac_bf16_peak": round(chunk_tf / PEAK_BF16_TFLOPS, 4),
                               "us_per_call": chunk_us, "flop": ccfg.fwd_flop,
                               "floor_us": cfl["floor_us"], "of_floor": round(cfl["floor_us"] / chunk_us, 4)}

        q_rot, k_rot = torch.empty_like(g["q"]), torch.empty_like(g["k"])

        def rope_step():
            attn.attn_fwd_rope(g["q"], g["k"], g["v"], True, cfg.scale, 10000.0, q_rot=q_rot,
                               k_rot=k_rot, o=tt["o"], lse=tt["lse"])
            attn.attn_bwd_rope(q_rot, k_rot, g["v"], tt["o"], tt["lse"], g["dout"], True, cfg.scale,
                               10000.0, dq=tt["dq"], dk=tt["dk"], dv=tt["dv"], workspace=tt["ws"])
        rope_us = T.op(rope_step)["median_us"]
        extras["fwd_bwd_rope"] = {"us_per_step": rope_us,
                                  "TFLOP_s": round(train_flop / (rope_us * 1e-6) / 1e12, 2),
                                  "rotary_cost_us": round(rope_us - train_us, 3)}
    result.update(extras)

    # ---------------------------------------------------------------- the oracle
    result["cpu_baseline"] = None
    if args.cpu_seconds > 0:
        base, c4_oracle = cpu_baseline(cfg, x, args.cpu_seconds)
        result["cpu_baseline"] = base
        if configs:
            oracle_per_config(configs, c4_oracle, cfg)
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg, x, budget_s: float):
    """The f64 oracle on the headline workload, fwd then bwd, one (batch,
    key/value group) slice at a time until the budget is spent (at least one
    slice); reported in the metric's unit."""
    import oracle
    G = cfg.Hq // cfg.Hkv
    groups = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    done, t_fwd, t_all = 0, 0.0, 0.0
    while done < len(groups) and (done == 0 or t_all < budget_s):
        b, g = groups[done]
        hs = slice(g * G, (g + 1) * G)
        q, k, v, do = (x["q"][b:b + 1, hs], x["k"][b:b + 1, g:g + 1], x["v"][b:b + 1, g:g + 1],
                       x["dout"][b:b + 1, hs])
        t0 = time.perf_counter()
        oracle.attn_fwd(q, k, v, True, cfg.scale)
        t1 = time.perf_counter()
        oracle.attn_bwd(q, k, v, do, True, cfg.scale)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_all += t2 - t0
        done += 1
    frac = done / len(groups)
    flop = (cfg.fwd_flop + cfg.bwd_flop) * frac
    base = {"value": round(flop / t_all / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, kv-group) slices of {cfg.name} (each a kv "
                      f"head and its {G} query heads), fwd then bwd in f64, {t_all:.1f} s"}
    full = {"fwd_s": round(t_fwd / frac, 3), "fwd_bwd_s": round(t_all / frac, 3),
            "measured_fraction": round(frac, 4)}
    return base, full


def oracle_per_config(configs, headline_oracle, hcfg):
    """Wall time of the oracle per config: best of 3 for the small ones (and the
    decode), the headline's one run (extrapolated from the slices it ran)."""
    import oracle
    from attention_causal_gqa_flash_amd import workloads as W
    for c in (W.C1, W.C2, W.C3_128, W.C3_512, W.C4):
        if c.name not in configs:
            continue
        if c.name == hcfg.name:
            configs[c.name]["oracle_s"] = dict(headline_oracle, runs=1)
            continue
        if c.name == W.C4.name:
            continue      # one run of the 4096-token workload only as the headline
        xx = W.train_inputs(c)
        bf, bb = float("inf"), float("inf")
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.attn_fwd(xx["q"], xx["k"], xx["v"], True, c.scale)
            t1 = time.perf_counter()
            oracle.attn_bwd(xx["q"], xx["k"], xx["v"], xx["dout"], True, c.scale)
            t2 = time.perf_counter()
            bf, bb = min(bf, t1 - t0), min(bb, t2 - t0)
        configs[c.name]["oracle_s"] = {"fwd_s": round(bf, 4), "fwd_bwd_s": round(bb, 4), "runs": 3}
        configs[c.name]["gpu_vs_oracle_fwd_bwd"] = round(bb / (configs[c.name]["fwd_bwd_us"] * 1e-6), 1)
    dc = W.C5
    if dc.name in configs:
        xd = W.decode_inputs(dc)
        best = float("inf")
        for _ in range(3):
            t0 = time.perf_counter()
            po, pl = oracle.attn_decode(xd["q"], xd["k_cache"], xd["v_cache"], dc.scale, dc.n_splits)
            oracle.lse_merge(po, pl)
            best = min(best, time.perf_counter() - t0)
        configs[dc.name]["oracle_s"] = {"decode_s": round(best, 4), "runs": 3}
    if hcfg.name in configs and "fwd_bwd_us" in configs[hcfg.name]:
        configs[hcfg.name]["gpu_vs_oracle_fwd_bwd"] = round(
            headline_oracle["fwd_bwd_s"] / (configs[hcfg.name]["fwd_bwd_us"] * 1e-6), 1)
    configs["oracle_cores"] = oracle.num_threads()
    configs["oracle_cpu_model"] = cpu_model()


if __name__ == "__main__":
    main()
