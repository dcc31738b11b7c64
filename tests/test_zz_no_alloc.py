"""attn_bwd_noalloc (no allocation, the row terms in the library's own device
array) against attn_bwd (caller workspace) and against the oracle, on two calls
in a row, the second with a smaller input, then a refusal of a shape beyond
the array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import attention_causal_gqa_flash_amd as attn
from attention_causal_gqa_flash_amd import workloads as W

pytestmark = pytest.mark.gpu


def _relF(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


CALLS = [
    # B, Hq, Hkv, N, d, dtype: the first call the larger one
    (2, 8, 2, 700, 128, "bf16"),
    (1, 4, 1, 300, 64, "bf16"),
]


def test_noalloc_matches_attn_bwd_two_calls():
    for B, Hq, Hkv, N, d, dtype in CALLS:
        print(f"\n[case] noalloc B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype}", flush=True)
        x = W.random_train(B, Hq, Hkv, N, d, dtype=dtype, seed=N + d, dout_scale=0.1)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        g = {n: torch.from_numpy(a).cuda().to(tdt) for n, a in x.items()}
        scale = d ** -0.5
        o, lse = attn.attn_fwd(g["q"], g["k"], g["v"], True, scale)
        ref = attn.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["dout"], True, scale)
        f32 = dict(device="cuda", dtype=torch.float32)
        outs = (torch.full((B, Hq, N, d), float("nan"), **f32),
                torch.full((B, Hkv, N, d), float("nan"), **f32),
                torch.full((B, Hkv, N, d), float("nan"), **f32))
        got = attn.attn_bwd_noalloc(g["q"], g["k"], g["v"], o, lse, g["dout"], True, scale,
                                    dq=outs[0], dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
        # the same kernels: dq bit for bit; dk, dv up to the order of atomic adds
        assert torch.equal(got[0], ref[0])
        for a, b in zip(got[1:], ref[1:]):
            assert torch.allclose(a, b, rtol=0, atol=1e-5 * float(b.abs().max()))
        # and the oracle's tolerance (bf16 inputs: relative Frobenius 2e-2)
        rdq, rdk, rdv = oracle.attn_bwd(x["q"], x["k"], x["v"], x["dout"], True, scale)
        for a, r in zip(got, (rdq, rdk, rdv)):
            assert _relF(a.cpu().numpy().astype(np.float64), r) <= 2e-2


def test_noalloc_refuses_shapes_beyond_its_array():
    L = attn.lib()
    P = ctypes.c_void_p(0x10000)
    # B * Hq * N = 2^20 + 64 query rows: more than the 4 MiB array holds
    rc = L.attn_bwd_noalloc(1, 1, 64, 8, (1 << 14) + 1, 64, 1, 0.125, *([P] * 9), None)
    assert rc == 3
