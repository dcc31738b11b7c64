"""The time floors of bounds.py (host arithmetic, CPU only)."""
import os
import re

import pytest

from attention_causal_gqa_flash_amd import bounds as BD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fwd_flop_closed_form():
    # causal, BM = BN: query tile t computes (t + 1) whole key tiles
    B, H, N, d, T = 2, 3, 512, 64, 128
    r = BD.fwd(B, H, H, N, N, d, True, T, T)
    n = N // T
    flop = B * H * sum(T * (t + 1) * T for t in range(n)) * 4 * d
    assert r["terms_us"]["mfma"] == pytest.approx(flop / BD.PEAK_MFMA * 1e6, abs=1e-3)
    assert r["terms_us"]["chain"] == pytest.approx(T * N * 4 * d / BD.PEAK_MFMA_CU * 1e6, abs=1e-3)
    # full attention: every tile sees every key
    full = BD.fwd(B, H, H, N, N, d, False, T, T)
    assert full["terms_us"]["mfma"] == pytest.approx(B * H * N * N * 4 * d / BD.PEAK_MFMA * 1e6, abs=1e-3)


def test_floor_is_the_largest_term_and_causal_is_cheaper():
    for args in ((4, 12, 4, 1024, 1024, 64), (1, 32, 8, 4096, 4096, 128), (1, 8, 2, 300, 700, 128)):
        for fn in (BD.fwd, BD.bwd_dq, BD.bwd_dkdv, BD.bwd_grads):
            c, f = fn(*args, True), fn(*args, False)
            assert c["floor_us"] == max(c["terms_us"].values())
            assert c["floor_us"] <= f["floor_us"]


def test_smaller_tiles_trade_chain_for_l2():
    a = BD.fwd(1, 32, 8, 4096, 4096, 128, True, 64, 64)
    b = BD.fwd(1, 32, 8, 4096, 4096, 128, True, 256, 64)
    assert a["terms_us"]["chain"] < b["terms_us"]["chain"]
    assert a["terms_us"]["l2"] > b["terms_us"]["l2"]


def test_memory_level():
    # 27.5 MB (O f32 and dO read, D written, dK/dV zero-filled) fits the
    # last-level cache; a decode that rotates over more
    # caches than it holds reads HBM
    small = BD.preprocess(4, 12, 4, 1024, 64, True)
    assert small["floor_us"] == pytest.approx((4 * 12 * 1024 * (64 * 4 + 64 * 2 + 4) + 2 * 4 * 4 * 1024 * 64 * 4) / BD.PEAK_LLC * 1e6, abs=1e-3)
    dec = BD.decode(1, 32, 8, 4096, 128, 16, resident=False)
    assert dec["terms_us"]["mem"] > 16_777_216 / BD.PEAK_HBM * 1e6


def test_library_tile_choices():
    assert BD.fwd_tile(4, 12, 1024, 64) == {"BM": 64, "BN": 32}       # key split on 768 items
    assert BD.fwd_tile(1, 32, 4096, 128) == {"BM": 128, "BN": 64}
    assert BD.fwd_tile(1, 32, 512, 128) == {"BM": 64, "BN": 64}
    assert BD.head_split(4, 12, 4, 1024) == 3
    assert BD.head_split(1, 32, 8, 4096) == 1
    assert BD.head_split(1, 32, 8, 4096, BKV=128) == 2   # the d = 128 kernel's 128-key tiles


def test_best_tile_is_feasible_and_no_worse():
    for B, Hq, Hkv, N, d in ((4, 12, 4, 1024, 64), (1, 32, 8, 4096, 128)):
        t = BD.fwd_tile(B, Hq, N, d)
        best = BD.best_fwd(B, Hq, Hkv, N, N, d)
        assert BD.fwd_fits(d, best["tile"]["BM"], best["tile"]["BN"])
        assert best["floor_us"] <= BD.fwd(B, Hq, Hkv, N, N, d, True, **t)["floor_us"]
        hs = BD.head_split(B, Hq, Hkv, N)
        g = BD.best_bwd_grads(B, Hq, Hkv, N, N, d)
        assert g["floor_us"] <= BD.bwd_grads(B, Hq, Hkv, N, N, d, True, 64, 128, hs, 128, 64)["floor_us"]


def _profile_avg_us(kernel_prefix):
    text = open(os.path.join(ROOT, "profiles", "kernels_gqa12x4_b4_n1024_d64.md")).read()
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0].startswith(kernel_prefix):
            return float(cells[2])
    return None


@pytest.mark.parametrize("kernel,floor", [
    ("fwd_mfma_kernel<64, 2, 32", lambda: BD.fwd(4, 12, 4, 1024, 1024, 64, True, 64, 32)),
    ("bwd_fused_kernel<64", lambda: BD.bwd_grads(4, 12, 4, 1024, 1024, 64, True, 64, 128, 3, 128, 64)),
    ("decode_mfma_kernel<128, false>", lambda: BD.decode(1, 32, 8, 4096, 128, 16, resident=False)),
])
def test_floor_below_the_recorded_kernel_time(kernel, floor):
    """The floor must stay below the measured time (the committed kernel-trace summary)."""
    avg = _profile_avg_us(kernel)
    if avg is None:
        pytest.skip(f"{kernel} not in the committed summary")
    assert floor()["floor_us"] < avg
