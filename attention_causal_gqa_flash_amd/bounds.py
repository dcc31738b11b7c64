"""Time floors of the path's kernels from their tile sizes, and the best tile.

A traffic bound and the best tile from one optimisation over tile sizes ("A
compiler that derives GPU kernels matches hand-tuned code", the paragraph on how
fast a kernel could possibly run: the floor must stay below every measured
time).  The pages do not print that program; this module takes its plainest
reading for the tiled kernels here.  For one launch of a kernel with a given
tiling, each of five quantities bounds the time from below:

  mfma   matrix-core flop the tiling performs (whole tiles, so the masked parts
         of diagonal tiles count) / the dense bf16 peak;
  mem    compulsory bytes (every input read once, every output written once)
         / the peak of the memory level that can hold them: the 256 MB
         last-level cache when they fit (a kernel that follows its producer
         finds its inputs there), HBM otherwise;
  l2     bytes the tiling moves from L2 into the CUs (operand tiles re-read per
         work item) / the L2-to-CU peak;
  lds    bytes the waves read from LDS (each wave owns 32 rows of the 32x32
         matrix-core blocks and reads every operand tile it multiplies) / the
         LDS peak;
  chain  the largest work item's flop / one CU's share of the matrix-core peak
         (a work item runs on one CU).

The floor is the largest of the five.  Smaller tiles shorten the chain and
waste less of the diagonal but re-read more from L2; the best tile is the
feasible tile (multiples of the 32-row matrix-core block, its LDS and register
footprint within one CU) with the least floor, found by enumerating the
power-of-two tile lattice.  Per-tile fixed costs (barriers, row reductions,
the exponentials' latency) are not in the floor: it bounds, it does not
predict.  All figures are in microseconds.  Host arithmetic only: nothing here
launches or times a kernel.
"""
from __future__ import annotations

CUS = 256
CLOCK_HZ = 2.4e9
PEAK_MFMA = 2516.6e12             # dense bf16 flop/s (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_MFMA_CU = PEAK_MFMA / CUS
PEAK_HBM = 8.0e12                 # B/s
PEAK_LLC = 17.2e12                # B/s, the 256 MB last-level (Infinity) cache
LLC_BYTES = 256 * 1024 * 1024
PEAK_L2 = CUS * 64 * CLOCK_HZ     # 64 B/clk per CU from L2 (16 x 128 B/clk per XCD): 39.3 TB/s
PEAK_LDS = CUS * 256 * CLOCK_HZ   # 256 B/clk per CU (ds_read_b128 measured 230 B/clk at 16 waves)
LDS_BYTES = 160 * 1024            # per CU
VGPR_BYTES = 4 * 512 * 64 * 4     # per CU: 4 SIMDs x 512 registers x 64 lanes x 4 B

_POW2 = (32, 64, 128, 256)


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def _floor(terms: dict) -> dict:
    us = {k: v * 1e6 for k, v in terms.items()}
    return {"floor_us": round(max(us.values()), 3), "terms_us": {k: round(v, 3) for k, v in us.items()}}


def _mem(nbytes: int, resident: bool | None = None) -> float:
    """Seconds to move the compulsory bytes; resident=None: they fit the last-level cache or not."""
    if resident is None:
        resident = nbytes <= LLC_BYTES
    return nbytes / (PEAK_LLC if resident else PEAK_HBM)


def _visible(r1: int, Nk: int, off: int, causal: bool) -> int:
    """Keys seen by query rows below r1 (query row i at key position i + off)."""
    return min(Nk, r1 + off) if causal else Nk


def fwd(B, Hq, Hkv, Nq, Nk, d, causal=True, BM=128, BN=64, esz=2) -> dict:
    """Forward: a work item is BM query rows of one head streaming BN-key tiles."""
    off = Nk - Nq
    flop = l2 = lds = chain = 0
    for t in range(_ceil(Nq, BM)):
        vis = _ceil(_visible(min(Nq, (t + 1) * BM), Nk, off, causal), BN) * BN
        f = BM * vis * 4 * d
        flop += f
        chain = max(chain, f)
        l2 += BM * d * esz + vis * d * 2 * esz + BM * (4 * d + 4)
        lds += (BM // 32) * vis * d * 2 * esz          # K and V tiles, per wave
    hbm = B * Hq * Nq * d * esz + 2 * B * Hkv * Nk * d * esz + B * Hq * Nq * (4 * d + 4)
    r = _floor({"mfma": B * Hq * flop / PEAK_MFMA, "mem": _mem(hbm),
                "l2": B * Hq * l2 / PEAK_L2, "lds": B * Hq * lds / PEAK_LDS,
                "chain": chain / PEAK_MFMA_CU})
    r["tile"] = {"BM": BM, "BN": BN}
    return r


def fwd_fits(d, BM, BN, esz=2) -> bool:
    lds = 2 * 2 * BN * d * esz                      # K and V tiles, double-buffered
    regs = BM * d * 4 + BM * d * esz + BM * BN * 4  # O accumulator, Q operand, scores
    return lds <= LDS_BYTES and regs <= VGPR_BYTES


def _dkdv_terms(B, Hq, Hkv, Nq, Nk, d, causal, BKV, SR, hs, esz=2):
    G, off = Hq // Hkv, Nk - Nq
    Gs = G // hs
    nq_r = _ceil(Nq, SR) * SR
    flop = l2 = lds = chain = 0
    for kt in range(_ceil(Nk, BKV)):
        q0 = (max(kt * BKV - off, 0) // SR) * SR if causal else 0
        rows = Gs * (nq_r - q0)
        f = rows * BKV * 8 * d                      # S, dP, dV, dK
        flop += f * hs
        chain = max(chain, f)
        l2 += hs * (BKV * d * 2 * esz + rows * (2 * d * esz + 8) + BKV * d * 8)
        # per 32-key wave: Q and dO rows for the scores, and again transposed
        lds += hs * (BKV // 32) * rows * (4 * d * esz + 8)
    return B * Hkv * flop, B * Hkv * l2, B * Hkv * lds, chain


def _dq_terms(B, Hq, Hkv, Nq, Nk, d, causal, BQ, BN, esz=2):
    off = Nk - Nq
    flop = l2 = lds = chain = 0
    for t in range(_ceil(Nq, BQ)):
        vis = _ceil(_visible(min(Nq, (t + 1) * BQ), Nk, off, causal), BN) * BN
        f = BQ * vis * 6 * d                        # S, dP (recomputed), dQ
        flop += f
        chain = max(chain, f)
        l2 += BQ * (2 * d * esz + 8) + vis * d * 2 * esz + BQ * d * 4
        lds += (BQ // 32) * vis * 3 * d * esz       # K, V for the scores, K again for dQ
    return B * Hq * flop, B * Hq * l2, B * Hq * lds, chain


def _bwd_hbm(B, Hq, Hkv, Nq, Nk, d, esz=2, dq=True, dkdv=True):
    rd = B * Hq * Nq * (2 * d * esz + 8) + 2 * B * Hkv * Nk * d * esz      # Q, dO, lse, D; K, V
    wr = (B * Hq * Nq * d * 4 if dq else 0) + (2 * B * Hkv * Nk * d * 4 if dkdv else 0)
    return rd + wr


def bwd_dkdv(B, Hq, Hkv, Nq, Nk, d, causal=True, BKV=64, SR=128, hs=1) -> dict:
    """dK/dV: a work item is BKV keys of one kv head against the query rows of G/hs heads."""
    flop, l2, lds, chain = _dkdv_terms(B, Hq, Hkv, Nq, Nk, d, causal, BKV, SR, hs)
    r = _floor({"mfma": flop / PEAK_MFMA, "mem": _mem(_bwd_hbm(B, Hq, Hkv, Nq, Nk, d, dq=False)),
                "l2": l2 / PEAK_L2, "lds": lds / PEAK_LDS, "chain": chain / PEAK_MFMA_CU})
    r["tile"] = {"BKV": BKV, "SR": SR, "hs": hs}
    return r


def bwd_dq(B, Hq, Hkv, Nq, Nk, d, causal=True, BQ=128, BN=64) -> dict:
    """dQ: a work item is BQ query rows of one head streaming BN-key tiles."""
    flop, l2, lds, chain = _dq_terms(B, Hq, Hkv, Nq, Nk, d, causal, BQ, BN)
    r = _floor({"mfma": flop / PEAK_MFMA, "mem": _mem(_bwd_hbm(B, Hq, Hkv, Nq, Nk, d, dkdv=False)),
                "l2": l2 / PEAK_L2, "lds": lds / PEAK_LDS, "chain": chain / PEAK_MFMA_CU})
    r["tile"] = {"BQ": BQ, "BN": BN}
    return r


def bwd_grads(B, Hq, Hkv, Nq, Nk, d, causal=True, BKV=64, SR=128, hs=1, BQ=128, BN=64) -> dict:
    """Both gradient kinds in one launch: their work items share the CUs."""
    f1, l1, s1, c1 = _dkdv_terms(B, Hq, Hkv, Nq, Nk, d, causal, BKV, SR, hs)
    f2, l2, s2, c2 = _dq_terms(B, Hq, Hkv, Nq, Nk, d, causal, BQ, BN)
    r = _floor({"mfma": (f1 + f2) / PEAK_MFMA, "mem": _mem(_bwd_hbm(B, Hq, Hkv, Nq, Nk, d)),
                "l2": (l1 + l2) / PEAK_L2, "lds": (s1 + s2) / PEAK_LDS,
                "chain": max(c1, c2) / PEAK_MFMA_CU})
    r["tile"] = {"BKV": BKV, "SR": SR, "hs": hs, "BQ": BQ, "BN": BN}
    return r


def dkdv_fits(d, BKV, SR, esz=2) -> bool:
    lds = 2 * SR * (2 * d * esz + 8)                         # Q, dO, lse, D, double-buffered
    regs = BKV * d * 8 + BKV * d * 2 * esz + 2 * SR * BKV * 4  # dK, dV; K, V; S, dP
    return lds <= LDS_BYTES and regs <= VGPR_BYTES


def dq_fits(d, BQ, BN, esz=2) -> bool:
    lds = 2 * 2 * BN * d * esz
    regs = BQ * d * 4 + BQ * d * 2 * esz + 2 * BQ * BN * 4
    return lds <= LDS_BYTES and regs <= VGPR_BYTES


def decode(B, Hq, Hkv, L, d, n_splits, esz=2, resident=None) -> dict:
    """Split-KV decode: a work item is one split of one kv head's cache for its G query heads
    (resident=False: the caches come from HBM, as when calls rotate over more caches than the
    last-level cache holds)."""
    G, C = Hq // Hkv, _ceil(L, n_splits)
    flop = B * Hkv * n_splits * G * C * 4 * d
    parts = B * Hq * n_splits * (d + 1) * 4
    hbm = 2 * B * Hkv * L * d * esz + B * Hq * d * esz + 2 * parts + B * Hq * (d + 1) * 4
    item_bytes = C * d * 2 * esz
    r = _floor({"mfma": flop / PEAK_MFMA, "mem": _mem(hbm, resident),
                "l2": (2 * B * Hkv * L * d * esz + parts) / PEAK_L2,
                "chain": item_bytes / (PEAK_L2 / CUS)})
    r["tile"] = {"splits": n_splits}
    return r


def preprocess(B, Hq, Hkv, N, d, zero_dkdv: bool, esz=2) -> dict:
    """D = rowsum(dO o O): O (f32) and dO read, D written; dK/dV zero-filled when split."""
    hbm = B * Hq * N * (d * 4 + d * esz + 4) + (2 * B * Hkv * N * d * 4 if zero_dkdv else 0)
    r = _floor({"mem": _mem(hbm)})
    r["tile"] = {}
    return r


def best_fwd(B, Hq, Hkv, Nq, Nk, d, causal=True) -> dict:
    cands = [fwd(B, Hq, Hkv, Nq, Nk, d, causal, BM, BN) for BM in _POW2 for BN in _POW2
             if fwd_fits(d, BM, BN)]
    return min(cands, key=lambda r: r["floor_us"])


def _divisors(n):
    return [c for c in range(1, n + 1) if n % c == 0]


def best_bwd_grads(B, Hq, Hkv, Nq, Nk, d, causal=True) -> dict:
    G = Hq // Hkv
    best = None
    for BKV in _POW2:
        for SR in _POW2:
            if not dkdv_fits(d, BKV, SR):
                continue
            for hs in _divisors(G):
                for BQ in _POW2:
                    for BN in _POW2:
                        if not dq_fits(d, BQ, BN):
                            continue
                        r = bwd_grads(B, Hq, Hkv, Nq, Nk, d, causal, BKV, SR, hs, BQ, BN)
                        if best is None or r["floor_us"] < best["floor_us"]:
                            best = r
    return best


def best_bwd_dkdv(B, Hq, Hkv, Nq, Nk, d, causal=True) -> dict:
    cands = [bwd_dkdv(B, Hq, Hkv, Nq, Nk, d, causal, BKV, SR, hs) for BKV in _POW2 for SR in _POW2
             for hs in _divisors(Hq // Hkv) if dkdv_fits(d, BKV, SR)]
    return min(cands, key=lambda r: r["floor_us"])


def best_bwd_dq(B, Hq, Hkv, Nq, Nk, d, causal=True) -> dict:
    cands = [bwd_dq(B, Hq, Hkv, Nq, Nk, d, causal, BQ, BN) for BQ in _POW2 for BN in _POW2
             if dq_fits(d, BQ, BN)]
    return min(cands, key=lambda r: r["floor_us"])


def best_decode(B, Hq, Hkv, L, d, resident=None) -> dict:
    return min((decode(B, Hq, Hkv, L, d, S, resident=resident) for S in (1, 2, 4, 8, 16, 32, 64, 128)),
               key=lambda r: r["floor_us"])


def head_split(B, Hq, Hkv, Nk, cus=CUS, BKV=64) -> int:
    """The dK/dV head split the library picks: the smallest divisor c of G with
    B * Hkv * (key tiles) * c >= 2 * cus (else G)."""
    G = Hq // Hkv
    base = _ceil(Nk, BKV) * B * Hkv
    hs = 1
    for c in _divisors(G):
        hs = c
        if base * c >= 2 * cus:
            break
    return hs


def fwd_tile(B, Hq, Nq, d, cus=CUS) -> dict:
    """The forward tile the library picks: 128 query rows, or 64 with the key
    split on small grids (32-key tiles at d = 64)."""
    items = _ceil(Nq, 128) * B * Hq
    split = items < 2 * cus if d == 64 else items < cus
    if not split:
        return {"BM": 128, "BN": 64}
    return {"BM": 64, "BN": 32 if d == 64 else 64}
