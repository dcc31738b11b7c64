"""GPU parity: the HIP path (through the C ABI) against the CPU f64 oracle.

Tolerances (max abs = max over every element of |gpu - oracle|; relative
Frobenius = ||gpu - oracle||_F / ||oracle||_F over the whole tensor):
  f32 inputs : every output (o, lse, dq, dk, dv) max abs <= 1e-5, on every
               shape;
  bf16 inputs: o max abs <= 1e-2, lse max abs <= 1e-3, dq/dk/dv relative
               Frobenius <= 2e-2.
Both sides see the same inputs: float32 draws rounded to bf16 where the
workload is bf16, widened exactly for the oracle.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import attention_causal_gqa_flash_amd as attn
from attention_causal_gqa_flash_amd import workloads as W

pytestmark = pytest.mark.gpu


def _to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def _gpu_fwd_bwd(x, dtype, causal, scale):
    g = {n: _to_dev(a, dtype) for n, a in x.items()}
    o, lse = attn.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=scale)
    dq, dk, dv = attn.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["dout"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]


def _relF(got, ref):
    n = np.linalg.norm(ref)
    d = np.linalg.norm(got - ref)
    return d / n if n > 0 else d


def _check(got, ref, dtype, label=""):
    o, lse, dq, dk, dv = got
    ro, rl, rdq, rdk, rdv = ref
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), label
    if dtype == "f32":
        for name, a, b in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk),
                           ("dv", dv, rdv)):
            tol = 1e-5
            err = float(np.abs(a - b).max())
            assert err <= tol, f"{label} {name}: max abs {err:.3e} > {tol:.1e}"
    else:
        eo = float(np.abs(o - ro).max())
        el = float(np.abs(lse - rl).max())
        assert eo <= 1e-2, f"{label} o: max abs {eo:.3e}"
        assert el <= 1e-3, f"{label} lse: max abs {el:.3e}"
        for name, a, b in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            e = _relF(a, b)
            assert e <= 2e-2 or np.linalg.norm(a - b) <= 1e-6, f"{label} {name}: relF {e:.3e}"


def _oracle_fwd_bwd(x, causal, scale):
    ro, rl = oracle.attn_fwd(x["q"], x["k"], x["v"], causal, scale)
    rdq, rdk, rdv = oracle.attn_bwd(x["q"], x["k"], x["v"], x["dout"], causal, scale)
    return ro, rl, rdq, rdk, rdv


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [W.C1, W.C2, W.C3_128, W.C3_512], ids=lambda c: c.name)
def test_workload_full(cfg):
    print(f"\n[case] {cfg.name} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} N={cfg.N} d={cfg.d}", flush=True)
    x = W.train_inputs(cfg)
    got = _gpu_fwd_bwd(x, cfg.dtype, True, cfg.scale)
    ref = _oracle_fwd_bwd(x, True, cfg.scale)
    _check(got, ref, cfg.dtype, label=cfg.name)


def test_long_context_all_groups():
    """N = 4096, d = 128, 32/8 heads: the whole problem on the GPU and in the oracle,
    compared element by element over every output of every grouped-query group (a
    key/value head and its 4 query heads; the oracle runs one group at a time)."""
    cfg = W.C4
    print(f"\n[case] {cfg.name} all {cfg.Hkv} groups", flush=True)
    x = W.train_inputs(cfg)
    o, lse, dq, dk, dv = _gpu_fwd_bwd(x, cfg.dtype, True, cfg.scale)
    G = cfg.Hq // cfg.Hkv
    parts = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    for g in range(cfg.Hkv):
        hs = slice(g * G, (g + 1) * G)
        xs = {"q": x["q"][:, hs], "k": x["k"][:, g:g + 1], "v": x["v"][:, g:g + 1],
              "dout": x["dout"][:, hs]}
        ref = _oracle_fwd_bwd(xs, True, cfg.scale)
        got = (o[:, hs], lse[:, hs], dq[:, hs], dk[:, g:g + 1], dv[:, g:g + 1])
        _check(got, ref, cfg.dtype, label=f"{cfg.name} group {g}")
        for n, a in zip(parts, ref):
            parts[n].append(a)
        print(f"  group {g} ok", flush=True)
    # and over the whole tensors at once (the per-group relative Frobenius errors
    # bound this one, but it is the tolerance's own definition)
    ref = [np.concatenate(parts[n], axis=1) for n in parts]
    _check((o, lse, dq, dk, dv), ref, cfg.dtype, label=f"{cfg.name} whole")


def test_decode_workload():
    cfg = W.C5
    print(f"\n[case] {cfg.name}", flush=True)
    x = W.decode_inputs(cfg)
    g = {n: _to_dev(a, cfg.dtype) for n, a in x.items()}
    po, pl = attn.attn_decode(g["q"], g["k_cache"], g["v_cache"], cfg.n_splits, scale=cfg.scale)
    o, lse = attn.attn_lse_merge(po, pl)
    torch.cuda.synchronize()
    rpo, rpl = oracle.attn_decode(x["q"], x["k_cache"], x["v_cache"], cfg.scale, cfg.n_splits)
    ro, rl = oracle.lse_merge(rpo, rpl)
    assert float(np.abs(po.cpu().numpy() - rpo).max()) <= 1e-2
    assert float(np.abs(pl.cpu().numpy() - rpl).max()) <= 1e-3
    assert float(np.abs(o.cpu().numpy() - ro).max()) <= 1e-2
    assert float(np.abs(lse.cpu().numpy() - rl).max()) <= 1e-3


# ---------------------------------------------------------------------------
# further shapes: ragged lengths, every head dim, group sizes, non-causal,
# other scales, both dtypes
# ---------------------------------------------------------------------------

EXTRA = [
    # B, Hq, Hkv, N, d, dtype, causal, scale (None = 1/sqrt(d))
    (1, 1, 1, 1, 64, "bf16", True, None),
    (1, 2, 1, 1, 128, "bf16", True, None),
    (2, 4, 2, 100, 64, "bf16", True, None),
    (1, 6, 2, 333, 128, "bf16", True, None),
    (1, 4, 4, 257, 128, "bf16", False, None),
    (1, 8, 2, 190, 64, "bf16", False, None),
    (3, 4, 1, 129, 128, "bf16", True, None),
    (1, 4, 2, 300, 64, "bf16", True, -0.1),
    (1, 2, 2, 150, 128, "bf16", True, 0.0),
    (1, 2, 1, 200, 64, "bf16", True, 0.3),
    (2, 2, 1, 77, 16, "bf16", True, None),
    (1, 3, 1, 65, 32, "bf16", True, None),
    (1, 2, 1, 130, 64, "f32", True, None),
    (1, 2, 2, 50, 128, "f32", False, None),
    (2, 4, 2, 33, 32, "f32", True, None),
    (4, 16, 4, 1024, 64, "bf16", True, None),   # d = 64 grid large enough for 128-row tiles
    (2, 128, 32, 300, 128, "bf16", True, None),  # d = 128 grid large enough for 256-row tiles
    (4, 128, 16, 256, 128, "bf16", False, None),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,causal,scale", EXTRA,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_N{c[3]}_d{c[4]}_{c[5]}_{'c' if c[6] else 'nc'}"
                              f"_s{c[7]}" for c in EXTRA])
def test_extra_shapes(B, Hq, Hkv, N, d, dtype, causal, scale):
    print(f"\n[case] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype} causal={causal} scale={scale}",
          flush=True)
    x = W.random_train(B, Hq, Hkv, N, d, dtype=dtype, seed=N * 7 + d)
    s = float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale))
    got = _gpu_fwd_bwd(x, dtype, causal, s)
    ref = _oracle_fwd_bwd(x, causal, s)
    _check(got, ref, dtype, label=f"N{N} d{d} {dtype}")


def test_repeat_consistency():
    """o, lse and dq are bitwise deterministic; dk and dv may sum a group's query
    heads with atomics (order-dependent in the last bits only)."""
    x = W.random_train(1, 8, 2, 300, 128, dtype="bf16", seed=5)
    a = _gpu_fwd_bwd(x, "bf16", True, 0.088)
    b = _gpu_fwd_bwd(x, "bf16", True, 0.088)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u, v)
    for u, v in zip(a[3:], b[3:]):
        assert np.abs(u - v).max() <= 1e-5 * max(1.0, np.abs(u).max())


DECODE = [
    # B, Hq, Hkv, L, d, n_splits, dtype
    (1, 32, 8, 4096, 128, 16, "bf16"),
    (2, 8, 2, 1000, 128, 7, "bf16"),
    (1, 4, 4, 5, 64, 8, "bf16"),        # more splits than keys: empty chunks
    (1, 16, 1, 1, 128, 1, "bf16"),      # a one-key cache, G = 16
    (1, 4, 2, 513, 64, 16, "f32"),
    (3, 6, 3, 77, 32, 3, "bf16"),
    (1, 2, 1, 300, 16, 5, "f32"),
    # group sizes that do not divide 16 (heads repeat unevenly over the 16
    # score columns) and chunks longer than one pass of the 8 waves (256 keys)
    (1, 12, 4, 2000, 64, 3, "bf16"),    # G = 3, 667-key chunks
    (2, 10, 2, 1500, 128, 2, "bf16"),   # G = 5, 750-key chunks
    (1, 14, 2, 700, 128, 4, "bf16"),    # G = 7
]


@pytest.mark.parametrize("B,Hq,Hkv,L,d,S,dtype", DECODE,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_L{c[3]}_d{c[4]}_S{c[5]}_{c[6]}" for c in DECODE])
def test_decode_shapes(B, Hq, Hkv, L, d, S, dtype):
    print(f"\n[case] decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} S={S} {dtype}", flush=True)
    cfg = W.DecodeConfig("adhoc", dtype, B, Hq, Hkv, L, d, S, seed=L + d)
    x = W.decode_inputs(cfg)
    g = {n: _to_dev(a, dtype) for n, a in x.items()}
    po, pl = attn.attn_decode(g["q"], g["k_cache"], g["v_cache"], S, scale=cfg.scale)
    o, lse = attn.attn_lse_merge(po, pl)
    torch.cuda.synchronize()
    rpo, rpl = oracle.attn_decode(x["q"], x["k_cache"], x["v_cache"], cfg.scale, S)
    ro, rl = oracle.lse_merge(rpo, rpl)
    tol_o, tol_l = (1e-5, 1e-5) if dtype == "f32" else (1e-2, 1e-3)
    gpl = pl.cpu().numpy()
    empty = np.isneginf(rpl)
    assert np.array_equal(np.isneginf(gpl), empty)
    assert float(np.abs(gpl[~empty] - rpl[~empty]).max()) <= tol_l
    assert float(np.abs(po.cpu().numpy() - rpo).max()) <= tol_o
    assert float(np.abs(o.cpu().numpy() - ro).max()) <= tol_o
    assert float(np.abs(lse.cpu().numpy() - rl).max()) <= tol_l
    # the decoded row equals the last row of a causal forward over the cache
    full_o, full_l = oracle.attn_fwd(x["q"][:, :, None], x["k_cache"], x["v_cache"], False, cfg.scale)
    assert float(np.abs(o.cpu().numpy() - full_o[:, :, 0]).max()) <= tol_o


# ---------------------------------------------------------------------------
# backward with an upstream gradient of lse
# ---------------------------------------------------------------------------

DLSE = [
    (4, 12, 4, 1024, 64, True, "bf16"),     # the one-launch gradient kernel, 3-way head split
    (1, 8, 2, 300, 128, True, "bf16"),      # d = 128: dQ computing the row terms, then dK/dV (head split)
    (2, 6, 3, 200, 64, False, "bf16"),
    (1, 2, 1, 64, 16, True, "f32"),         # generic kernels
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype", DLSE,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_N{c[3]}_d{c[4]}_{'c' if c[5] else 'nc'}_{c[6]}" for c in DLSE])
def test_bwd_dlse(B, Hq, Hkv, N, d, causal, dtype):
    print(f"\n[case] bwd_dlse B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} {dtype}", flush=True)
    x = W.random_train(B, Hq, Hkv, N, d, dtype=dtype, seed=N + d, dout_scale=0.1)
    dl = np.random.default_rng(N).standard_normal((B, Hq, N)).astype(np.float32) * 0.3
    g = {n: _to_dev(a, dtype) for n, a in x.items()}
    scale = d ** -0.5
    o, lse = attn.attn_fwd(g["q"], g["k"], g["v"], causal, scale)
    dq, dk, dv = attn.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["dout"], causal, scale,
                               dlse=torch.from_numpy(dl).cuda())
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]
    ro, rl = oracle.attn_fwd(x["q"], x["k"], x["v"], causal, scale)
    rdq, rdk, rdv = oracle.attn_bwd_dlse(x["q"], x["k"], x["v"], x["dout"], dl.astype(np.float64),
                                         causal, scale)
    _check(got, (ro, rl, rdq, rdk, rdv), dtype, label=f"dlse N{N} d{d}")


# ---------------------------------------------------------------------------
# Nq queries against Nk >= Nq keys (a prefill chunk against a cache)
# ---------------------------------------------------------------------------

FWD_KV = [
    (2, 8, 2, 100, 1000, 128, True, "bf16"),
    (1, 12, 4, 1, 777, 64, True, "bf16"),      # one decode row
    (2, 6, 3, 64, 101, 64, True, "bf16"),
    (1, 4, 2, 200, 300, 64, False, "bf16"),
    (1, 8, 2, 512, 4096, 128, True, "bf16"),   # a 512-token chunk at the end of a 4k context
    (1, 2, 1, 20, 50, 16, True, "f32"),        # generic kernels
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype", FWD_KV,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}_{c[7]}"
                              for c in FWD_KV])
def test_fwd_kv(B, Hq, Hkv, Nq, Nk, d, causal, dtype):
    print(f"\n[case] fwd_kv B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype}",
          flush=True)
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=Nq + Nk)
    q = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])      # the last Nq query rows
    scale = d ** -0.5
    o, lse = attn.attn_fwd_kv(_to_dev(q, dtype), _to_dev(x["k"], dtype), _to_dev(x["v"], dtype),
                              causal, scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(q, x["k"], x["v"], causal, scale)
    tol_o, tol_l = (1e-5, 1e-5) if dtype == "f32" else (1e-2, 1e-3)
    assert float(np.abs(o.cpu().numpy() - ro).max()) <= tol_o
    assert float(np.abs(lse.cpu().numpy() - rl).max()) <= tol_l


def test_fwd_kv_square_equals_fwd():
    x = W.random_train(2, 12, 4, 333, 64, seed=3)
    g = {n: _to_dev(a, "bf16") for n, a in x.items()}
    o1, l1 = attn.attn_fwd(g["q"], g["k"], g["v"], True, 0.125)
    o2, l2 = attn.attn_fwd_kv(g["q"], g["k"], g["v"], True, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


BWD_KV = [
    (4, 12, 4, 256, 1024, 64, True, "bf16", False),   # one-launch gradients, 3-way head split
    (1, 8, 2, 300, 700, 128, True, "bf16", True),     # d = 128, dQ with the row terms then dK/dV, with dlse
    (2, 6, 3, 64, 101, 64, True, "bf16", False),      # ragged tiles on both sides
    (1, 4, 2, 200, 300, 64, False, "bf16", False),
    (2, 6, 2, 1, 333, 64, True, "bf16", True),        # one row against a cache
    (1, 4, 1, 512, 4096, 128, True, "bf16", False),   # a 512-token chunk at the end of 4k keys
    (1, 2, 1, 20, 50, 16, True, "f32", True),         # generic kernels
    (1, 4, 2, 37, 130, 32, False, "f32", False),
    # 12 query heads on one kv head at 3008 queries against 3072 keys: the
    # one-launch plan's dK/dV side splits its level groups where the head
    # split changes, which once planned 49 groups for a 48-group argument
    (1, 12, 1, 3008, 3072, 64, True, "bf16", False),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype,with_dlse", BWD_KV,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}"
                              f"_{c[7]}{'_dlse' if c[8] else ''}" for c in BWD_KV])
def test_bwd_kv(B, Hq, Hkv, Nq, Nk, d, causal, dtype, with_dlse):
    print(f"\n[case] bwd_kv B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype} "
          f"dlse={with_dlse}", flush=True)
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=Nq + 3 * Nk, dout_scale=0.1)
    q = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])
    do = np.ascontiguousarray(x["dout"][:, :, Nk - Nq:])
    dl = (np.random.default_rng(Nq).standard_normal((B, Hq, Nq)).astype(np.float32) * 0.3
          if with_dlse else None)
    scale = d ** -0.5
    gq, gk, gv, gdo = (_to_dev(a, dtype) for a in (q, x["k"], x["v"], do))
    o, lse = attn.attn_fwd_kv(gq, gk, gv, causal, scale)
    dq, dk, dv = attn.attn_bwd_kv(gq, gk, gv, o, lse, gdo, causal, scale,
                                  dlse=None if dl is None else torch.from_numpy(dl).cuda())
    torch.cuda.synchronize()
    assert dq.shape == (B, Hq, Nq, d) and dk.shape == (B, Hkv, Nk, d)
    got = [t.cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]
    ro, rl = oracle.attn_fwd(q, x["k"], x["v"], causal, scale)
    if dl is None:
        rdq, rdk, rdv = oracle.attn_bwd(q, x["k"], x["v"], do, causal, scale)
    else:
        rdq, rdk, rdv = oracle.attn_bwd_dlse(q, x["k"], x["v"], do, dl.astype(np.float64), causal,
                                             scale)
    _check(got, (ro, rl, rdq, rdk, rdv), dtype, label=f"bwd_kv Nq{Nq} Nk{Nk} d{d}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_kv_square_equals_bwd(d):
    """Nq = Nk through attn_bwd_kv runs the same kernels as attn_bwd: the same bits (dq is
    deterministic; dk, dv too where the key tiles alone fill the GPU)."""
    x = W.random_train(1, 8, 2, 2048, d, seed=5, dout_scale=0.1)
    g = {n: _to_dev(a, "bf16") for n, a in x.items()}
    o, lse = attn.attn_fwd(g["q"], g["k"], g["v"], True, 0.1)
    r1 = attn.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["dout"], True, 0.1)
    r2 = attn.attn_bwd_kv(g["q"], g["k"], g["v"], o, lse, g["dout"], True, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0])
    rel = [float((a - b).norm() / b.norm()) for a, b in zip(r1[1:], r2[1:])]
    assert max(rel) <= 1e-6, rel


# ---------------------------------------------------------------------------
# a seeded sweep of random shapes: the host-side choices (key split of the
# forward, 64- or 128-key dK/dV kernel, head split, one-launch plan, generic
# kernels) change with the grid, and these shapes land on both sides of them
# ---------------------------------------------------------------------------

def _sweep_cases(n, seed, max_work=1.5e9):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([16, 32, 64, 128], p=[0.1, 0.1, 0.4, 0.4]))
        dtype = "f32" if (d <= 32 and rng.random() < 0.5) or rng.random() < 0.1 else "bf16"
        Hkv = int(rng.integers(1, 9))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        B = int(rng.integers(1, 5))
        Nk = int(rng.integers(1, 1500))
        Nq = Nk if rng.random() < 0.6 else int(rng.integers(1, Nk + 1))
        causal = bool(rng.random() < 0.75)
        dlse = bool(rng.random() < 0.25)                      # an upstream gradient of lse
        obf = dtype == "bf16" and bool(rng.random() < 0.25)   # O written in bf16
        gbf = bool(rng.random() < 0.2)                        # gradients written in bf16
        neg = bool(rng.random() < 0.1)                        # a negative scale
        if B * G * Hkv * Nq * Nk * d > max_work:   # keeps the oracle to about a second
            continue
        cases.append((B, G * Hkv, Hkv, Nq, Nk, d, dtype, causal, dlse, obf, gbf, neg))
    return cases


# ATTN_SWEEP_N / ATTN_SWEEP_SEED select a longer run (e.g. 1000 shapes)
SWEEP = _sweep_cases(int(os.environ.get("ATTN_SWEEP_N", "24")),
                     int(os.environ.get("ATTN_SWEEP_SEED", "20261203"))) + [
    # either side of the host's thresholds on a 256-CU part (short sequences, many heads):
    # d = 64 forward: 128 128-row work items take four key parts, 132 two
    (1, 128, 16, 128, 128, 64, "bf16", True, False, False, False, False),
    (1, 132, 12, 128, 128, 64, "bf16", True, False, False, False, False),
    # d = 64 forward: 512 128-row work items run unsplit, 510 split
    (4, 128, 16, 128, 128, 64, "bf16", True, False, False, False, False),
    (2, 255, 85, 128, 128, 64, "bf16", True, False, False, False, False),
    # d = 128 forward: 256 items unsplit, 255 split
    (2, 128, 32, 128, 128, 128, "bf16", True, False, False, False, False),
    (1, 255, 85, 128, 128, 128, "bf16", True, False, False, False, False),
    # d = 128 dK/dV: 4 x 2 key tiles x 32 kv heads reach 256 (128-key kernel), 31 do not
    (2, 32, 16, 256, 256, 128, "bf16", True, False, False, False, False),
    (1, 62, 31, 256, 256, 128, "bf16", True, False, False, False, False),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal,dlse,obf,gbf,neg", SWEEP,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{c[6]}_{'c' if c[7] else 'nc'}"
                              f"{'_dlse' if c[8] else ''}{'_obf' if c[9] else ''}{'_gbf' if c[10] else ''}"
                              f"{'_neg' if c[11] else ''}" for c in SWEEP])
def test_random_shape_sweep(B, Hq, Hkv, Nq, Nk, d, dtype, causal, dlse, obf, gbf, neg):
    print(f"\n[case] sweep B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
          f"dlse={dlse} o_bf16={obf} grads_bf16={gbf} neg_scale={neg}", flush=True)
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=Nq * 131 + Nk * 7 + d, dout_scale=0.1)
    q = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])
    do = np.ascontiguousarray(x["dout"][:, :, Nk - Nq:])
    dl = (np.random.default_rng(Nq + Nk).standard_normal((B, Hq, Nq)).astype(np.float32) * 0.3
          if dlse else None)
    scale = float(np.float32(d ** -0.5 * (-0.7 if neg else 1.0)))
    gq, gk, gv, gdo = (_to_dev(a, dtype) for a in (q, x["k"], x["v"], do))
    gdl = None if dl is None else torch.from_numpy(dl).cuda()
    o, lse = attn.attn_fwd_ex(gq, gk, gv, causal, scale, o_dtype=torch.bfloat16 if obf else torch.float32)
    bwd = attn.attn_bwd_bf16grad if gbf else attn.attn_bwd_ex
    dq, dk, dv = bwd(gq, gk, gv, o, lse, gdo, causal, scale, dlse=gdl)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]
    ro, rl = oracle.attn_fwd(q, x["k"], x["v"], causal, scale)
    if dl is None:
        rdq, rdk, rdv = oracle.attn_bwd(q, x["k"], x["v"], do, causal, scale)
    else:
        rdq, rdk, rdv = oracle.attn_bwd_dlse(q, x["k"], x["v"], do, dl.astype(np.float64), causal, scale)
    label = f"sweep Nq{Nq} Nk{Nk} d{d} {dtype}"
    if obf:   # o rounded to bf16: half a unit in its last place on top of the bound
        e16 = float(np.abs(got[0] - ro).max())
        assert e16 <= 1e-2 + 2.0 ** -9 * float(np.abs(ro).max()), f"{label} bf16 o: max abs {e16:.3e}"
        got[0] = ro
    # f32 inputs keep the f32 bound unless something was rounded to bf16 on the way
    _check(got, (ro, rl, rdq, rdk, rdv), "f32" if dtype == "f32" and not (obf or gbf) else "bf16", label)


# ---------------------------------------------------------------------------
# bf16 gradients (attn_bwd_bf16grad): the f32 gradients of attn_bwd_ex rounded
# to nearest even
# ---------------------------------------------------------------------------

BF16_GRAD = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal, with_dlse, o dtype
    (2, 12, 4, 300, 300, 64, "bf16", True, False, "f32"),
    (1, 8, 2, 200, 700, 128, "bf16", True, True, "bf16"),    # cross-length, dlse, bf16 o
    (4, 12, 4, 256, 1024, 64, "bf16", True, False, "f32"),   # dK/dV head subsets added by atomics
    (1, 4, 2, 100, 100, 32, "f32", False, False, "f32"),     # generic kernels
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal,with_dlse,o_dtype", BF16_GRAD,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{c[6]}_{'c' if c[7] else 'nc'}"
                              f"{'_dlse' if c[8] else ''}_o{c[9]}" for c in BF16_GRAD])
def test_bf16_gradients(B, Hq, Hkv, Nq, Nk, d, dtype, causal, with_dlse, o_dtype):
    print(f"\n[case] bf16grad B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
          f"dlse={with_dlse} o={o_dtype}", flush=True)
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=Nq * 5 + Nk + d, dout_scale=0.1)
    q = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])
    do = np.ascontiguousarray(x["dout"][:, :, Nk - Nq:])
    dl = (np.random.default_rng(Nk).standard_normal((B, Hq, Nq)).astype(np.float32) * 0.3
          if with_dlse else None)
    scale = float(np.float32(d ** -0.5))
    gq, gk, gv, gdo = (_to_dev(a, dtype) for a in (q, x["k"], x["v"], do))
    gdl = None if dl is None else torch.from_numpy(dl).cuda()
    o, lse = attn.attn_fwd_ex(gq, gk, gv, causal, scale,
                              o_dtype=torch.bfloat16 if o_dtype == "bf16" else torch.float32)
    g16 = attn.attn_bwd_bf16grad(gq, gk, gv, o, lse, gdo, causal, scale, dlse=gdl)
    g32 = attn.attn_bwd_ex(gq, gk, gv, o, lse, gdo, causal, scale, dlse=gdl)
    torch.cuda.synchronize()
    assert all(t.dtype == torch.bfloat16 for t in g16)
    assert g16[0].shape == (B, Hq, Nq, d) and g16[1].shape == (B, Hkv, Nk, d)
    # the same f32 values rounded once: dq is deterministic; dk, dv may carry atomics
    # (order-dependent last bits of the f32 value, so at most one bf16 step apart)
    assert torch.equal(g16[0], g32[0].to(torch.bfloat16))
    for a, b in zip(g16[1:], g32[1:]):
        r = b.to(torch.bfloat16).float()
        assert float((a.float() - r).abs().max()) <= float(r.abs().max()) * 2.0 ** -7
    # against the oracle at the bf16 gradient tolerance
    if dl is None:
        ref = oracle.attn_bwd(q, x["k"], x["v"], do, causal, scale)
    else:
        ref = oracle.attn_bwd_dlse(q, x["k"], x["v"], do, dl.astype(np.float64), causal, scale)
    for name, a, b in zip(("dq", "dk", "dv"), g16, ref):
        e = _relF(a.float().cpu().numpy().astype(np.float64), b)
        assert e <= 2e-2, f"bf16grad {name}: relF {e:.3e}"


# ---------------------------------------------------------------------------
# bf16 output (attn_fwd_ex / attn_bwd_ex)
# ---------------------------------------------------------------------------

EX = [
    (4, 12, 4, 1024, 1024, 64, True, "bf16"),    # key-split forward, one-launch gradients
    (2, 16, 4, 700, 700, 64, True, "bf16"),      # 128-row forward tiles
    (1, 8, 2, 300, 800, 128, True, "bf16"),
    (1, 4, 2, 100, 100, 32, False, "bf16"),      # generic kernels, bf16 inputs
    (1, 2, 1, 40, 70, 16, True, "f32"),          # generic kernels, f32 inputs
    (3, 12, 4, 8, 8, 64, True, "bf16"),          # short causal rows (row 0 is v_0), four key parts
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype", EX,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}_{c[7]}"
                              for c in EX])
def test_bf16_output(B, Hq, Hkv, Nq, Nk, d, causal, dtype):
    print(f"\n[case] bf16 output B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype}",
          flush=True)
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=Nq + 5 * Nk, dout_scale=0.1)
    q = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])
    do = np.ascontiguousarray(x["dout"][:, :, Nk - Nq:])
    scale = d ** -0.5
    gq, gk, gv, gdo = (_to_dev(a, dtype) for a in (q, x["k"], x["v"], do))
    o16, l16 = attn.attn_fwd_ex(gq, gk, gv, causal, scale, o_dtype=torch.bfloat16)
    o32, l32 = attn.attn_fwd_ex(gq, gk, gv, causal, scale)
    dq, dk, dv = attn.attn_bwd_ex(gq, gk, gv, o16, l16, gdo, causal, scale)
    torch.cuda.synchronize()
    # the same kernels: the bf16 output is the f32 output rounded to nearest even
    assert o16.dtype == torch.bfloat16 and torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)
    got = [t.float().cpu().numpy().astype(np.float64) for t in (o32, l16, dq, dk, dv)]
    ro, rl = oracle.attn_fwd(q, x["k"], x["v"], causal, scale)
    rdq, rdk, rdv = oracle.attn_bwd(q, x["k"], x["v"], do, causal, scale)
    # the f32 o at the input dtype's bound; o rounded to bf16 adds half a unit in its
    # last place (2^-9 relative), which alone exceeds 1e-2 wherever |o| >= 4 (a causal
    # row 0 is v_0 itself); the gradients, computed from the bf16 o, at the bf16 bounds
    e16 = float(np.abs(o16.float().cpu().numpy() - ro).max())
    assert e16 <= 1e-2 + 2.0 ** -9 * float(np.abs(ro).max()), f"bf16 o: max abs {e16:.3e}"
    _check(got, (ro, rl, rdq, rdk, rdv), "bf16", label=f"bf16 out Nq{Nq} Nk{Nk} d{d} (f32 o)")
    if dtype == "f32":
        for name, a, b in (("o", got[0], ro), ("lse", got[1], rl)):
            err = float(np.abs(a - b).max())
            assert err <= 1e-5, f"f32 {name}: max abs {err:.3e}"



# ---------------------------------------------------------------------------
# rotary positions
# ---------------------------------------------------------------------------

ROPE = [
    (2, 3, 37, 64, 0, 10000.0, "bf16"),
    (1, 4, 130, 128, 4000, 500000.0, "bf16"),
    (1, 2, 9, 16, 1_000_000, 10000.0, "f32"),     # positions of a million: angle reduction
    (2, 2, 33, 32, 7, 10.0, "f32"),
]


@pytest.mark.parametrize("B,H,N,d,pos0,base,dtype", ROPE,
                         ids=[f"B{c[0]}_H{c[1]}_N{c[2]}_d{c[3]}_p{c[4]}_{c[6]}" for c in ROPE])
def test_rope(B, H, N, d, pos0, base, dtype):
    print(f"\n[case] rope B={B} H={H} N={N} d={d} pos0={pos0} {dtype}", flush=True)
    x = W.random_train(B, H, H, N, d, dtype=dtype, seed=N + d)["q"]
    gx = _to_dev(x, dtype)
    for inverse in (False, True):
        y = attn.attn_rope(gx, pos0, base, inverse=inverse)
        z = gx.clone()
        attn.attn_rope(z, pos0, base, inverse=inverse, y=z)            # in place
        torch.cuda.synchronize()
        assert torch.equal(y, z)
        ref = oracle.rope(x, pos0, base, inverse=inverse)
        got = y.float().cpu().numpy().astype(np.float64)
        if dtype == "f32":
            assert float(np.abs(got - ref).max()) <= 1e-6 * max(1.0, float(np.abs(ref).max()))
        else:   # rounded to bf16: within one bf16 unit in the last place of the exact value
            assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-6 * float(np.abs(x).max()))


ATTN_ROPE = [
    (2, 8, 2, 300, 300, 128, True, "bf16", False),
    (2, 32, 8, 512, 512, 128, True, "bf16", False),   # 128-row forward tiles (no key split)
    (4, 16, 4, 1024, 1024, 64, True, "bf16", False),  # the same at d = 64
    (4, 12, 4, 256, 1024, 64, True, "bf16", True),    # chunk against a cache, with dlse
    (1, 4, 2, 100, 200, 64, False, "bf16", False),
    (1, 2, 1, 20, 50, 16, True, "f32", False),        # generic kernels
    (1, 4, 2, 64, 64, 32, True, "f32", True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype,with_dlse", ATTN_ROPE,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}"
                              f"_{c[7]}{'_dlse' if c[8] else ''}" for c in ATTN_ROPE])
def test_attn_rope(B, Hq, Hkv, Nq, Nk, d, causal, dtype, with_dlse):
    print(f"\n[case] attn_rope B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype} "
          f"dlse={with_dlse}", flush=True)
    base = 10000.0
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=7 * Nq + Nk, dout_scale=0.1)
    q = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])
    do = np.ascontiguousarray(x["dout"][:, :, Nk - Nq:])
    dl = (np.random.default_rng(Nk).standard_normal((B, Hq, Nq)).astype(np.float32) * 0.3
          if with_dlse else None)
    scale = d ** -0.5
    gq, gk, gv, gdo = (_to_dev(a, dtype) for a in (q, x["k"], x["v"], do))
    o, lse, q_rot, k_rot = attn.attn_fwd_rope(gq, gk, gv, causal, scale, base)
    dq, dk, dv = attn.attn_bwd_rope(q_rot, k_rot, gv, o, lse, gdo, causal, scale, base,
                                    dlse=None if dl is None else torch.from_numpy(dl).cuda())
    torch.cuda.synchronize()
    # the rotated inputs are attn_rope's: k bit for bit; q, which the bf16 forward rotates
    # in its prologue on the hardware sine and cosine (about 1e-6 of the pair's size, where
    # attn_rope's library sine and cosine are exact to f32), rounds to the same bf16 value
    # except near rounding midpoints (one unit in the last place) and near zero (the
    # sine and cosine error, at most 3e-5 for these N(0, 1) pairs)
    assert torch.equal(k_rot, attn.attn_rope(gk, 0, base))
    ref_q = attn.attn_rope(gq, Nk - Nq, base)
    if dtype == "f32":
        assert torch.equal(q_rot, ref_q)
    else:
        a, r = q_rot.float(), ref_q.float()
        _, ex = torch.frexp(r)                                 # |r| in [2^(ex-1), 2^ex)
        ulp = torch.ldexp(torch.ones_like(r), torch.clamp(ex - 8, min=-133))
        assert bool(((a - r).abs() <= ulp + 3e-5).all())
        assert float((a != r).float().mean()) < 0.01
    got = [t.cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]
    dl64 = None if dl is None else dl.astype(np.float64)
    if dtype == "f32":
        ro, rl = oracle.attn_fwd_rope(q, x["k"], x["v"], causal, scale, base)
        rdq, rdk, rdv = oracle.attn_bwd_rope(q, x["k"], x["v"], do, causal, scale, base, dl64)
    else:
        # the matrix cores take bf16 operands, so the path rounds the rotated q and k to bf16
        # (test_rope holds that rounding to one unit in the last place); the oracle takes the
        # same decision on its own exact rotation, then attends and rotates the gradients back
        qr = W.round_bf16(oracle.rope(q, Nk - Nq, base).astype(np.float32)).astype(np.float64)
        kr = W.round_bf16(oracle.rope(x["k"], 0, base).astype(np.float32)).astype(np.float64)
        ro, rl = oracle.attn_fwd(qr, kr, x["v"], causal, scale)
        if dl64 is None:
            gq_, gk_, rdv = oracle.attn_bwd(qr, kr, x["v"], do, causal, scale)
        else:
            gq_, gk_, rdv = oracle.attn_bwd_dlse(qr, kr, x["v"], do, dl64, causal, scale)
        rdq = oracle.rope(gq_, Nk - Nq, base, inverse=True)
        rdk = oracle.rope(gk_, 0, base, inverse=True)
    label = f"attn_rope Nq{Nq} Nk{Nk} d{d}"
    if dtype == "f32":
        _check(got, (ro, rl, rdq, rdk, rdv), dtype, label=label)
        return
    # bf16: where the path's rotation lands within its own error of a rounding midpoint it
    # may round to the other neighbour than the oracle did (one unit in the last place);
    # each such element moves the scores it enters, and so o and lse, by a bounded amount
    a = _rope_rounding_allowance(oracle.rope(q, Nk - Nq, base), oracle.rope(x["k"], 0, base),
                                 scale, causal, Hq // Hkv)
    el = np.abs(got[1] - rl)
    assert np.all(el <= 1e-3 + a), f"{label} lse: max excess {float((el - 1e-3 - a).max()):.3e}"
    eo = np.abs(got[0] - ro).max(axis=-1)
    vmax = float(np.abs(x["v"]).max())
    assert np.all(eo <= 1e-2 + np.expm1(2 * a) * vmax), f"{label} o: max abs {float(eo.max()):.3e}"
    for name, g_, r_ in (("dq", got[2], rdq), ("dk", got[3], rdk), ("dv", got[4], rdv)):
        e = _relF(g_, r_)
        assert e <= 2e-2, f"{label} {name}: relF {e:.3e}"


def _rope_rounding_allowance(qx, kx, scale, causal, G, eps_abs=6e-5, eps_rel=2.0 ** -20):
    """Per query row, a bound on how far the scores move where the path rounds a rotated
    element to the other bf16 neighbour than the oracle: only an element whose exact
    rotated value (qx [B,Hq,Nq,d], kx [B,Hkv,Nk,d], f64) lies within the path's rotation
    error (eps_abs + eps_rel |x|: the hardware sine and cosine of the fused forward, the
    library ones of the rotation pass) of a rounding midpoint can, and by one unit in the
    last place.  Returns [B,Hq,Nq]: scale * max over the visible keys j of
    sum_c (u_q[i,c] |k_jc| + |q_ic| u_k[j,c]), u = that unit where the element is such,
    else 0.  lse moves by at most that much, each probability by a factor within
    exp(+-2 that)."""
    def amb_ulp(x):
        ax = np.abs(x)
        e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
        ulp = np.exp2(e - 7)                                   # bf16: 8 significant bits
        mid = (np.floor(ax / ulp) + 0.5) * ulp
        return np.where(np.abs(ax - mid) <= eps_abs + eps_rel * ax, ulp, 0.0)
    uq, uk = amb_ulp(qx), amb_ulp(kx)
    B, Hq, Nq, _ = qx.shape
    Nk = kx.shape[2]
    vis = (np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)) if causal else None
    out = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            m = uq[b, h] @ np.abs(kx[b, g]).T + np.abs(qx[b, h]) @ uk[b, g].T   # [Nq, Nk]
            if vis is not None:
                m = np.where(vis, m, 0.0)
            out[b, h] = scale * m.max(axis=1)
    return out


# ---------------------------------------------------------------------------
# one decode step with cache append (per-sequence lengths)
# ---------------------------------------------------------------------------

def _append_inputs(B, Hq, Hkv, Lc, d, seed):
    """bf16-representable draws (float64 arrays) for q, k_new, v_new and the caches."""
    rng = np.random.default_rng(seed)
    draw = lambda *sh: torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).to(
        torch.bfloat16).to(torch.float64).numpy()
    return dict(q=draw(B, Hq, d), k_new=draw(B, Hkv, d), v_new=draw(B, Hkv, d),
                k_cache=draw(B, Hkv, Lc, d), v_cache=draw(B, Hkv, Lc, d))


def _run_append(x, lens, S, scale, dev=None):
    dev = dev or {n: _to_dev(a, "bf16") for n, a in x.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    B, Hq, d = x["q"].shape
    po = torch.empty((B, Hq, S, d), device="cuda")
    pl = torch.empty((B, Hq, S), device="cuda")
    o, lse = attn.attn_decode_append(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                                     dev["v_cache"], sl, S, scale, part_o=po, part_lse=pl)
    torch.cuda.synchronize()
    return dev, o.cpu().numpy(), lse.cpu().numpy(), po.cpu().numpy(), pl.cpu().numpy()


APPEND = [
    (4, 32, 8, 600, 128, 16, [0, 1, 299, 599]),
    (3, 12, 4, 257, 64, 7, [256, 100, 31]),
    (2, 16, 1, 40, 128, 16, [2, 39]),           # more splits than keys, G = 16
    (1, 8, 8, 4096, 64, 16, [4095]),            # full cache, G = 1
    (2, 12, 4, 3000, 128, 2, [2999, 1500]),     # G = 3, 1500-key chunks (several passes)
]


@pytest.mark.parametrize("B,Hq,Hkv,Lc,d,S,lens", APPEND,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Lc{c[3]}_d{c[4]}_S{c[5]}" for c in APPEND])
def test_decode_append(B, Hq, Hkv, Lc, d, S, lens):
    print(f"\n[case] decode_append B={B} Hq={Hq} Hkv={Hkv} Lc={Lc} d={d} S={S} lens={lens}", flush=True)
    x = _append_inputs(B, Hq, Hkv, Lc, d, seed=Lc + d)
    scale = d ** -0.5
    dev, o, lse, po, pl = _run_append(x, lens, S, scale)
    ro, rl, rkc, rvc = oracle.attn_decode_append(x["q"], x["k_new"], x["v_new"], x["k_cache"],
                                                 x["v_cache"], lens, scale)
    assert float(np.abs(o - ro).max()) <= 1e-2
    assert float(np.abs(lse - rl).max()) <= 1e-3
    # the cache after the append, bit for bit: row n replaced, every other row untouched
    assert np.array_equal(dev["k_cache"].double().cpu().numpy(), rkc)
    assert np.array_equal(dev["v_cache"].double().cpu().numpy(), rvc)
    # the split partials: the oracle's split decode over each sequence's n + 1 keys
    for b, n in enumerate(lens):
        rpo, rpl = oracle.attn_decode(x["q"][b:b + 1], rkc[b:b + 1, :, :n + 1], rvc[b:b + 1, :, :n + 1],
                                      scale, S)
        empty = np.isneginf(rpl[0])
        assert np.array_equal(np.isneginf(pl[b]), empty)
        assert float(np.abs(pl[b][~empty] - rpl[0][~empty]).max()) <= 1e-3
        assert float(np.abs(po[b] - rpo[0]).max()) <= 1e-2


# seeded random decode shapes (ATTN_SWEEP_N / ATTN_SWEEP_SEED as for the training sweep):
# split decode then merge, against the oracle's split decode, its merge and the
# unsplit last row; and the append step with per-sequence lengths


def _decode_sweep_cases(n, seed):
    rng = np.random.default_rng(seed + 1)
    cases = []
    for _ in range(n):
        d = int(rng.choice([16, 32, 64, 128], p=[0.1, 0.1, 0.4, 0.4]))
        dtype = "f32" if rng.random() < 0.15 else "bf16"
        Hkv = int(rng.integers(1, 9))
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 16]))
        cases.append((int(rng.integers(1, 4)), G * Hkv, Hkv, int(rng.integers(1, 5000)), d,
                      int(rng.integers(1, 41)), dtype))
    return cases


def _append_sweep_cases(n, seed):
    rng = np.random.default_rng(seed + 2)
    cases = []
    for _ in range(n):
        B = int(rng.integers(1, 6))
        Hkv = int(rng.integers(1, 9))
        Lc = int(rng.integers(1, 5000))
        lens = [int(v) for v in rng.integers(0, Lc, size=B)]
        cases.append((B, int(rng.choice([1, 2, 3, 4, 6, 8, 16])) * Hkv, Hkv, Lc,
                      int(rng.choice([64, 128])), int(rng.integers(1, 33)), lens))
    return cases


_NS = int(os.environ.get("ATTN_SWEEP_N", "24"))
_SEED = int(os.environ.get("ATTN_SWEEP_SEED", "20261203"))
DECODE_SWEEP = _decode_sweep_cases(max(8, _NS // 2), _SEED)
APPEND_SWEEP = _append_sweep_cases(max(6, _NS // 4), _SEED)


@pytest.mark.parametrize("B,Hq,Hkv,L,d,S,dtype", DECODE_SWEEP,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_L{c[3]}_d{c[4]}_S{c[5]}_{c[6]}" for c in DECODE_SWEEP])
def test_decode_sweep(B, Hq, Hkv, L, d, S, dtype):
    test_decode_shapes(B, Hq, Hkv, L, d, S, dtype)


@pytest.mark.parametrize("B,Hq,Hkv,Lc,d,S,lens", APPEND_SWEEP,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Lc{c[3]}_d{c[4]}_S{c[5]}" for c in APPEND_SWEEP])
def test_decode_append_sweep(B, Hq, Hkv, Lc, d, S, lens):
    test_decode_append(B, Hq, Hkv, Lc, d, S, lens)


def test_decode_append_invalid_lengths_and_two_steps():
    """Lengths outside [0, L_cap) give NaN outputs and leave that cache alone; a
    second step (lengths + 1, new tokens) continues from the first."""
    B, Hq, Hkv, Lc, d, S = 4, 8, 2, 50, 128, 5
    scale = d ** -0.5
    x = _append_inputs(B, Hq, Hkv, Lc, d, seed=5)
    lens = [-1, 50, 7, 49]
    dev, o, lse, _, _ = _run_append(x, lens, S, scale)
    assert np.all(np.isnan(o[:2])) and np.all(np.isnan(lse[:2]))
    assert np.all(np.isfinite(o[2:])) and np.all(np.isfinite(lse[2:]))
    ro, rl, rkc, rvc = oracle.attn_decode_append(x["q"], x["k_new"], x["v_new"], x["k_cache"],
                                                 x["v_cache"], lens, scale)
    assert np.array_equal(dev["k_cache"].double().cpu().numpy(), rkc)
    assert np.array_equal(dev["v_cache"].double().cpu().numpy(), rvc)
    assert float(np.abs(o[2:] - ro[2:]).max()) <= 1e-2
    # step 2 on the updated caches, valid lengths only
    x2 = _append_inputs(B, Hq, Hkv, Lc, d, seed=6)
    x2["k_cache"], x2["v_cache"] = rkc, rvc
    lens2 = [0, 10, 8, 48]
    dev2 = {n: _to_dev(x2[n], "bf16") for n in ("q", "k_new", "v_new")}
    dev2["k_cache"], dev2["v_cache"] = dev["k_cache"], dev["v_cache"]
    _, o2, l2, _, _ = _run_append(x2, lens2, S, scale, dev=dev2)
    ro2, rl2, rkc2, rvc2 = oracle.attn_decode_append(x2["q"], x2["k_new"], x2["v_new"], rkc, rvc,
                                                     lens2, scale)
    assert float(np.abs(o2 - ro2).max()) <= 1e-2 and float(np.abs(l2 - rl2).max()) <= 1e-3
    assert np.array_equal(dev2["k_cache"].double().cpu().numpy(), rkc2)


def test_merge_all_empty():
    po = torch.zeros((1, 3, 4, 64), device="cuda")
    pl = torch.full((1, 3, 4), float("-inf"), device="cuda")
    o, lse = attn.attn_lse_merge(po, pl)
    torch.cuda.synchronize()
    assert torch.all(o == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


MERGE_SPLITS = [1, 5, 16, 32, 33, 100]


@pytest.mark.parametrize("S", MERGE_SPLITS)
def test_merge_split_counts(S):
    """The merge alone on seeded partials (some chunks empty: lse = -inf, o = 0)
    against the oracle's merge, on both sides of the 32-split fast path."""
    print(f"\n[case] lse_merge S={S}", flush=True)
    rng = np.random.default_rng(4000 + S)
    B, Hq, d = 2, 5, 128
    po = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    pl = (3.0 * rng.standard_normal((B, Hq, S))).astype(np.float32)
    empty = rng.random((B, Hq, S)) < 0.3
    empty[0, 0, :] = S > 1                    # one row with a single live chunk
    empty[0, 0, -1] = False
    pl[empty] = -np.inf
    po[empty] = 0.0
    o, lse = attn.attn_lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(po, pl)
    assert float(np.abs(o.cpu().numpy() - ro).max()) <= 1e-5
    gl = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))   # rows whose chunks are all empty
    live = np.isfinite(rl)
    assert float(np.abs(gl[live] - rl[live]).max()) <= 1e-5


def test_invalid_call_leaves_outputs_untouched():
    q = torch.zeros((1, 3, 8, 64), device="cuda", dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 8, 64), device="cuda", dtype=torch.bfloat16)
    o = torch.full((1, 3, 8, 64), 7.0, device="cuda")
    lse = torch.full((1, 3, 8), 7.0, device="cuda")
    with pytest.raises(attn.AttnError):
        attn.attn_fwd(q, k, k, o=o, lse=lse)          # Hq % Hkv != 0
    torch.cuda.synchronize()
    assert torch.all(o == 7.0).item() and torch.all(lse == 7.0).item()


MERGED = [
    # B, Hq, Hkv, L, d, n_splits, dtype  (first call), second call uses L2
    (1, 32, 8, 4096, 128, 16, "bf16", 777),
    (2, 8, 2, 1000, 64, 7, "bf16", 64),
    (1, 4, 4, 5, 128, 8, "bf16", 3),         # empty chunks
    (1, 16, 1, 300, 128, 3, "bf16", 299),
    (1, 4, 2, 513, 64, 16, "f32", 100),      # generic decode kernel
    (1, 6, 3, 77, 32, 3, "bf16", 40),        # generic decode kernel (d = 32)
]


@pytest.mark.parametrize("B,Hq,Hkv,L,d,S,dtype,L2", MERGED,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_L{c[3]}_d{c[4]}_S{c[5]}_{c[6]}" for c in MERGED])
def test_decode_merged_two_calls(B, Hq, Hkv, L, d, S, dtype, L2):
    """Decode + merge in one call equals the oracle on two calls in a row reusing
    the outputs (the second on a shorter cache)."""
    for Lc in (L, L2):
        print(f"\n[case] decode_merged B={B} Hq={Hq} Hkv={Hkv} L={Lc} d={d} S={S} {dtype}", flush=True)
        cfg = W.DecodeConfig("adhoc", dtype, B, Hq, Hkv, Lc, d, S, seed=Lc * 3 + d)
        x = W.decode_inputs(cfg)
        g = {n: _to_dev(a, dtype) for n, a in x.items()}
        o, lse, po, pl = attn.attn_decode_merged(g["q"], g["k_cache"], g["v_cache"], S, scale=cfg.scale)
        torch.cuda.synchronize()
        rpo, rpl = oracle.attn_decode(x["q"], x["k_cache"], x["v_cache"], cfg.scale, S)
        ro, rl = oracle.lse_merge(rpo, rpl)
        tol_o, tol_l = (1e-5, 1e-5) if dtype == "f32" else (1e-2, 1e-3)
        assert float(np.abs(o.cpu().numpy() - ro).max()) <= tol_o
        assert float(np.abs(lse.cpu().numpy() - rl).max()) <= tol_l
        assert float(np.abs(po.cpu().numpy() - rpo).max()) <= tol_o


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [
    (4, 12, 4, 1024, 64, True),     # the 4 x 1024 training shape: one launch, 3-way head split
    (2, 8, 2, 333, 64, True),       # ragged tail, 4-way head split
    (1, 6, 3, 200, 64, False),
    (1, 8, 2, 300, 128, True),      # d = 128: two kernels side by side
])
def test_bwd_grads_stage(B, Hq, Hkv, N, d, causal):
    """preprocess + attn_bwd_grads against the oracle (bf16 tolerances)."""
    cfg = W.TrainConfig("grads", "bf16", B, Hq, Hkv, N, d, seed=21)
    print(f"\n[case] grads B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    x = W.train_inputs(cfg)
    g = {n: _to_dev(a, "bf16") for n, a in x.items()}
    o, lse = attn.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=cfg.scale)
    delta = attn.attn_bwd_preprocess(o, g["dout"])
    dq, dk, dv = attn.attn_bwd_grads(g["q"], g["k"], g["v"], lse, g["dout"], delta, causal,
                                     cfg.scale)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]
    ref = _oracle_fwd_bwd(x, causal, cfg.scale)
    _check(got, ref, "bf16", label=f"grads B{B} H{Hq}x{Hkv} N{N} d{d} c{int(causal)}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["stages", "grads", "attn_bwd"])
def test_graph_replay_matches_eager(mode, d):
    """The whole path captured in a HIP graph: every replay equals the eager run.
    The backward is the preprocess then the dK/dV and dQ stages ("stages"),
    attn_bwd_grads ("grads") or attn_bwd; at d = 128 attn_bwd_grads runs the dQ
    kernel then the dK/dV kernel, and attn_bwd runs the dQ kernel that computes
    the row terms, then the dK/dV kernel; at d = 64 both are one launch
    (attn_bwd_grads after a zero-fill launch of dk and dv)."""
    cfg = W.TrainConfig("graph", "bf16", 1, 8, 2, 320, d, seed=11)
    x = W.train_inputs(cfg)
    g = {n: _to_dev(a, "bf16") for n, a in x.items()}
    dc = W.DecodeConfig("graphdec", "bf16", 1, 8, 2, 700, 128, 5, seed=12)
    xd = W.decode_inputs(dc)
    gd = {n: _to_dev(a, "bf16") for n, a in xd.items()}
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    f32 = dict(device="cuda", dtype=torch.float32)
    o, lse = torch.empty((B, Hq, N, d), **f32), torch.empty((B, Hq, N), **f32)
    delta = torch.empty((B, Hq, N), **f32)
    dq, dk, dv = (torch.empty((B, Hq, N, d), **f32), torch.empty((B, Hkv, N, d), **f32),
                  torch.empty((B, Hkv, N, d), **f32))
    po, pl = torch.empty((1, 8, 5, 128), **f32), torch.empty((1, 8, 5), **f32)
    do_, dl = torch.empty((1, 8, 128), **f32), torch.empty((1, 8), **f32)
    ws = torch.empty(max(256, attn.attn_bwd_workspace_bytes(1, B, Hq, Hkv, N, d)), device="cuda",
                     dtype=torch.uint8)

    def step():
        attn.attn_fwd(g["q"], g["k"], g["v"], True, cfg.scale, o=o, lse=lse)
        attn.attn_bwd_preprocess(o, g["dout"], delta=delta)
        if mode == "attn_bwd":
            attn.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["dout"], True, cfg.scale, dq=dq, dk=dk,
                          dv=dv, workspace=ws)
        elif mode == "grads":
            attn.attn_bwd_grads(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, cfg.scale,
                                dq=dq, dk=dk, dv=dv)
        else:
            attn.attn_bwd_dkdv(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, cfg.scale,
                               dk=dk, dv=dv)
            attn.attn_bwd_dq(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, cfg.scale, dq=dq)
        attn.attn_decode_merged(gd["q"], gd["k_cache"], gd["v_cache"], 5, dc.scale,
                                part_o=po, part_lse=pl, o=do_, lse=dl)

    outs = (o, lse, dq, dk, dv, do_, dl)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, e) in enumerate(zip(outs, eager)):
            if i in (3, 4):      # dk, dv: atomics across query heads, last-bit differences
                assert torch.allclose(a, e, rtol=0, atol=1e-5 * float(e.abs().max())), \
                    f"replay {rep} differs from the eager run"
            else:
                assert torch.equal(a, e), f"replay {rep} differs from the eager run"


_FRESH_CAPTURE = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import attention_causal_gqa_flash_amd as attn
from attention_causal_gqa_flash_amd import workloads as W
x = W.random_train(1, 8, 2, 320, 128, seed=31, dout_scale=0.1)
g = {n: torch.from_numpy(a).cuda().to(torch.bfloat16) for n, a in x.items()}
f32 = dict(device="cuda", dtype=torch.float32)
lse = torch.from_numpy(np.random.default_rng(1).standard_normal((1, 8, 320)).astype(np.float32) + 6).cuda()
delta = torch.from_numpy(np.random.default_rng(2).standard_normal((1, 8, 320)).astype(np.float32) * 0.1).cuda()
outs = [torch.empty((1, 8, 320, 128), **f32), torch.empty((1, 2, 320, 128), **f32),
        torch.empty((1, 2, 320, 128), **f32)]
def call():
    attn.attn_bwd_grads(g["q"], g["k"], g["v"], lse, g["dout"], delta, True, 0.088,
                        dq=outs[0], dk=outs[1], dv=outs[2])
torch.cuda.synchronize()
s = torch.cuda.Stream()
graph = torch.cuda.CUDAGraph()
with torch.cuda.stream(s):
    with torch.cuda.graph(graph, stream=s):
        call()                  # the library's first call in this process
for t in outs:
    t.fill_(float("nan"))
torch.cuda.synchronize()
graph.replay()
torch.cuda.synchronize()
replayed = [t.clone() for t in outs]
call()
torch.cuda.synchronize()
# dq is bitwise deterministic; on this small grid dk and dv sum the query heads
# of a group with f32 atomics (last-bit differences between runs)
assert all(torch.isfinite(a).all() for a in replayed), "replay left non-finite values"
assert torch.equal(replayed[0], outs[0]), "dq of the replay differs from the eager call"
for a, e in zip(replayed[1:], outs[1:]):
    assert torch.allclose(a, e, rtol=0, atol=1e-5 * float(e.abs().max())), "dk/dv of the replay differ"
print("fresh-process capture ok", flush=True)
"""


def test_capture_as_first_call_in_fresh_process():
    """attn_bwd_grads at d = 128 captured into a graph as the library's very first call
    in a process: the library creates nothing lazily (no streams, events or other
    state), so the capture holds all of its work and the replay equals an eager call."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("\n[case] fresh-process capture of attn_bwd_grads d=128", flush=True)
    r = subprocess.run([sys.executable, "-c", _FRESH_CAPTURE, root], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0 and "fresh-process capture ok" in r.stdout, r.stdout + r.stderr


# ---------------------------------------------------------------------------
# strided layouts: q, k, v in one fused [B][N][Hq + 2 Hkv][d] projection buffer
# (interleaved heads), o, dout, dq, dk, dv as views of buffers of their own
# ---------------------------------------------------------------------------

STRIDED = [
    # B, Hq, Hkv, Nq, Nk, d, causal, dtype, o_dtype, with_dlse
    (2, 8, 2, 300, 300, 128, True, "bf16", "f32", False),    # d = 128: dQ with row terms, paired dK/dV
    (1, 32, 8, 512, 512, 128, True, "bf16", "f32", True),
    (2, 12, 4, 333, 333, 64, True, "bf16", "f32", False),     # d = 64: one-launch gradients
    (1, 8, 2, 200, 700, 64, True, "bf16", "bf16", True),      # chunk against a cache, bf16 o
    (1, 4, 2, 100, 257, 128, False, "bf16", "bf16", False),
    (1, 4, 2, 65, 65, 32, True, "f32", "f32", True),          # generic kernels
    (2, 2, 1, 40, 90, 16, True, "f32", "f32", False),
]


def _fused_views(x, B, Hq, Hkv, Nq, Nk, d, dtype):
    """q, k, v as strided views of one [B][N][Hq + 2 Hkv][d] buffer (q in its last Nq rows)."""
    H3 = Hq + 2 * Hkv
    buf = torch.zeros((B, Nk, H3, d), dtype=dtype, device="cuda")
    buf[:, :, :Hq] = torch.from_numpy(np.ascontiguousarray(x["q"].transpose(0, 2, 1, 3))).to(dtype).cuda()
    buf[:, :, Hq:Hq + Hkv] = torch.from_numpy(np.ascontiguousarray(x["k"].transpose(0, 2, 1, 3))).to(dtype).cuda()
    buf[:, :, Hq + Hkv:] = torch.from_numpy(np.ascontiguousarray(x["v"].transpose(0, 2, 1, 3))).to(dtype).cuda()
    q = buf[:, Nk - Nq:, :Hq].transpose(1, 2)
    k = buf[:, :, Hq:Hq + Hkv].transpose(1, 2)
    v = buf[:, :, Hq + Hkv:].transpose(1, 2)
    return buf, q, k, v


def _interleaved(B, H, N, d, dtype, fill):
    """A [B][H][N][d] view of a [B][N][H + 1][d] buffer filled with `fill` (one spare head per
    row, so that writes outside the view would show)."""
    buf = torch.full((B, N, H + 1, d), fill, dtype=dtype, device="cuda")
    return buf, buf[:, :, :H].transpose(1, 2)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype,o_dtype,with_dlse", STRIDED,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}"
                              f"_{c[7]}_o{c[8]}{'_dlse' if c[9] else ''}" for c in STRIDED])
def test_strided_layouts(B, Hq, Hkv, Nq, Nk, d, causal, dtype, o_dtype, with_dlse):
    print(f"\n[case] strided B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype} "
          f"o={o_dtype} dlse={with_dlse}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    odt = torch.bfloat16 if o_dtype == "bf16" else torch.float32
    x = W.random_train(B, Hq, Hkv, Nk, d, dtype=dtype, seed=11 * Nq + Nk + d, dout_scale=0.1)
    qn = np.ascontiguousarray(x["q"][:, :, Nk - Nq:])
    don = np.ascontiguousarray(x["dout"][:, :, Nk - Nq:])
    scale = float(np.float32(d ** -0.5))
    _, q, k, v = _fused_views(x, B, Hq, Hkv, Nq, Nk, d, tdt)
    assert not q.is_contiguous() and q.stride(3) == 1
    obuf, o = _interleaved(B, Hq, Nq, d, odt, 7.0)
    o, lse = attn.attn_fwd_strided(q, k, v, causal, scale, o=o)
    dobuf, dout = _interleaved(B, Hq, Nq, d, tdt, 0.0)
    dout.copy_(torch.from_numpy(don).to(tdt).cuda())
    dl = (torch.from_numpy(np.random.default_rng(Nq).standard_normal((B, Hq, Nq)).astype(np.float32) * 0.3).cuda()
          if with_dlse else None)
    bufs = [_interleaved(B, Hq, Nq, d, torch.float32, 7.0), _interleaved(B, Hkv, Nk, d, torch.float32, 7.0),
            _interleaved(B, Hkv, Nk, d, torch.float32, 7.0)]
    dq, dk, dv = attn.attn_bwd_strided(q, k, v, o, lse, dout, causal, scale, dq=bufs[0][1], dk=bufs[1][1],
                                       dv=bufs[2][1], dlse=dl)
    torch.cuda.synchronize()
    # nothing outside the views was written (the spare head of every row keeps its fill)
    for buf in (obuf, bufs[0][0], bufs[1][0], bufs[2][0]):
        assert bool((buf[:, :, -1] == 7.0).all())
    # the same kernels on contiguous copies: o, lse and dq bit for bit (dk, dv may take
    # atomics there, so to their last bits)
    gq, gk, gv, gdo = (t.contiguous() for t in (q, k, v, dout))
    o2, lse2 = attn.attn_fwd_ex(gq, gk, gv, causal, scale, o_dtype=odt)
    dq2, dk2, dv2 = attn.attn_bwd_ex(gq, gk, gv, o2, lse2, gdo, causal, scale, dlse=dl)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous(), o2) and torch.equal(lse, lse2)
    assert torch.equal(dq.contiguous(), dq2)
    for a, b in ((dk, dk2), (dv, dv2)):
        assert torch.allclose(a.contiguous(), b, rtol=0, atol=1e-5 * float(b.abs().max()))
    # and the oracle's tolerances
    got = [t.contiguous().float().cpu().numpy().astype(np.float64) for t in (o, lse, dq, dk, dv)]
    ro, rl = oracle.attn_fwd(qn, x["k"], x["v"], causal, scale)
    if dl is None:
        rdq, rdk, rdv = oracle.attn_bwd(qn, x["k"], x["v"], don, causal, scale)
    else:
        rdq, rdk, rdv = oracle.attn_bwd_dlse(qn, x["k"], x["v"], don, dl.cpu().numpy().astype(np.float64),
                                             causal, scale)
    if o_dtype == "bf16":
        # o rounded to bf16: half a unit in the last place (2^-9 relative) on top of the bound
        assert float(np.abs(got[0] - ro).max()) <= 1e-2 + 2.0 ** -9 * float(np.abs(ro).max())
        got[0] = ro
    _check(got, (ro, rl, rdq, rdk, rdv), dtype, label=f"strided Nq{Nq} Nk{Nk} d{d}")


# seeded random shapes for the strided and the rotary entry points (ATTN_SWEEP_N /
# ATTN_SWEEP_SEED as for the training sweep), through the tests above

def _layout_sweep_cases(n, seed, salt, max_work=1e9):
    rng = np.random.default_rng(seed + salt)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([16, 32, 64, 128], p=[0.1, 0.1, 0.4, 0.4]))
        dtype = "f32" if (d <= 32 and rng.random() < 0.5) or rng.random() < 0.1 else "bf16"
        Hkv = int(rng.integers(1, 7))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 4))
        Nk = int(rng.integers(2, 1200))
        Nq = Nk if rng.random() < 0.5 else int(rng.integers(2, Nk + 1))
        causal = bool(rng.random() < 0.75)
        o_dtype = "bf16" if dtype == "bf16" and rng.random() < 0.3 else "f32"
        dlse = bool(rng.random() < 0.3)
        if B * G * Hkv * Nq * Nk * d > max_work:
            continue
        cases.append((B, G * Hkv, Hkv, Nq, Nk, d, causal, dtype, o_dtype, dlse))
    return cases


STRIDED_SWEEP = _layout_sweep_cases(max(6, _NS // 4), _SEED, 3)
ROPE_SWEEP = [c[:8] + c[9:] for c in _layout_sweep_cases(max(6, _NS // 4), _SEED, 4)]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype,o_dtype,with_dlse", STRIDED_SWEEP,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}_{c[7]}"
                              f"_o{c[8]}{'_dlse' if c[9] else ''}" for c in STRIDED_SWEEP])
def test_strided_sweep(B, Hq, Hkv, Nq, Nk, d, causal, dtype, o_dtype, with_dlse):
    test_strided_layouts(B, Hq, Hkv, Nq, Nk, d, causal, dtype, o_dtype, with_dlse)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,dtype,with_dlse", ROPE_SWEEP,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}_{c[7]}"
                              f"{'_dlse' if c[8] else ''}" for c in ROPE_SWEEP])
def test_attn_rope_sweep(B, Hq, Hkv, Nq, Nk, d, causal, dtype, with_dlse):
    test_attn_rope(B, Hq, Hkv, Nq, Nk, d, causal, dtype, with_dlse)
