"""The C ABI of libattn.so, checked without a GPU.

The library must load, export every function that include/attn.h declares, and
refuse invalid calls with the documented status before touching the device.
Only refusal paths are exercised here: each call fails host-side validation,
so nothing is launched.  (Pointers used below are fake, aligned addresses; the
library never dereferences them on these paths.)
"""
import ctypes
import os
import re

import pytest

import attention_causal_gqa_flash_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = ctypes.c_void_p(0x10000)        # aligned, never dereferenced on refusal paths
MIS = ctypes.c_void_p(0x10004)      # misaligned
NUL = ctypes.c_void_p(0)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(attn.LIB_PATH):
        pytest.skip("libattn.so not built")
    return attn.lib()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("attn_fwd", "attn_fwd_kv", "attn_bwd", "attn_bwd_dlse", "attn_bwd_kv",
                     "attn_rope", "attn_fwd_rope", "attn_bwd_rope", "attn_fwd_ex", "attn_bwd_ex",
                     "attn_bwd_bf16grad", "attn_bwd_bf16grad_workspace_bytes",
                     "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
                     "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_grads",
                     "attn_bwd_grads_plan", "attn_decode", "attn_decode_append",
                     "attn_lse_merge", "attn_fwd_strided", "attn_bwd_strided",
                     "attn_bwd_noalloc", "attn_read_probe",
                     "attn_status_str", "attn_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), f"libattn.so does not export {name}"


def test_status_strings_and_version(L):
    assert attn.attn_abi_version() == 3
    assert attn.attn_status_str(OK) == "ok"
    assert "invalid" in attn.attn_status_str(INVALID)
    assert "unsupported" in attn.attn_status_str(UNSUPPORTED)
    assert "workspace" in attn.attn_status_str(WORKSPACE)
    assert attn.attn_status_str(99) == "unknown status"


def _fwd(L, dt=1, B=1, Hq=4, Hkv=2, N=64, d=64, causal=1, scale=0.125, ptrs=None):
    ptrs = ptrs or [P] * 5
    return L.attn_fwd(dt, B, Hq, Hkv, N, d, causal, scale, *ptrs, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID), (dict(N=0), INVALID),
    (dict(d=0), INVALID), (dict(B=-1), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(dt=2), INVALID), (dict(dt=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(d=8), UNSUPPORTED),
    (dict(Hq=70000, Hkv=1), UNSUPPORTED),
])
def test_fwd_refusals(L, kw, status):
    assert _fwd(L, **kw) == status


@pytest.mark.parametrize("which", range(5))
def test_fwd_refuses_null_or_misaligned(L, which):
    for bad in (NUL, MIS):
        ptrs = [P] * 5
        ptrs[which] = bad
        assert _fwd(L, ptrs=ptrs) == INVALID


def test_workspace_size(L):
    assert L.attn_bwd_workspace_bytes(1, 2, 12, 4, 1024, 64) == 2 * 12 * 1024 * 4
    assert L.attn_bwd_workspace_bytes(0, 1, 2, 1, 3, 16) == 256
    assert L.attn_bwd_workspace_bytes(1, 1, 6, 4, 64, 64) == 0     # Hq % Hkv != 0
    assert L.attn_bwd_workspace_bytes(1, 1, 4, 4, 64, 48) == 0     # unsupported d


def test_bf16grad_workspace_size(L):
    r256 = lambda x: (x + 255) // 256 * 256
    # row terms, then f32 dq [B,Hq,Nq,d], dk and dv [B,Hkv,Nk,d]
    B, Hq, Hkv, Nq, Nk, d = 2, 12, 4, 1000, 1024, 64
    want = r256(B * Hq * Nq * 4) + r256(B * Hq * Nq * d * 4) + 2 * r256(B * Hkv * Nk * d * 4)
    assert L.attn_bwd_bf16grad_workspace_bytes(1, B, Hq, Hkv, Nq, Nk, d) == want
    assert L.attn_bwd_bf16grad_workspace_bytes(0, 1, 2, 1, 3, 3, 16) == 256 + 512 + 2 * 256
    assert L.attn_bwd_bf16grad_workspace_bytes(1, 1, 4, 2, 65, 64, 64) == 0   # Nq > Nk
    assert L.attn_bwd_bf16grad_workspace_bytes(1, 1, 6, 4, 64, 64, 64) == 0   # Hq % Hkv != 0
    assert L.attn_bwd_bf16grad_workspace_bytes(1, 1, 4, 4, 64, 64, 48) == 0   # unsupported d


def _bwd_g(L, ws=P, ws_bytes=1 << 30, ptrs=None, **kw):
    a = dict(dt=1, o_dt=0, B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=64, causal=1, scale=0.125)
    a.update(kw)
    ptrs = ptrs or [P] * 10
    return L.attn_bwd_bf16grad(a["dt"], a["o_dt"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                               a["causal"], a["scale"], *ptrs, ws, ws_bytes, NUL)


def test_bf16grad_refusals(L):
    # every refusal is decided on the host, before any launch
    assert _bwd_g(L, o_dt=7) == INVALID
    assert _bwd_g(L, Nq=65) == INVALID
    assert _bwd_g(L, Hq=5) == INVALID
    assert _bwd_g(L, d=96) == UNSUPPORTED
    for which in (7, 8, 9):          # dq, dk, dv
        ptrs = [P] * 10
        ptrs[which] = MIS
        assert _bwd_g(L, ptrs=ptrs) == INVALID
    ptrs = [P] * 10
    ptrs[6] = MIS                    # dlse misaligned
    assert _bwd_g(L, ptrs=ptrs) == INVALID
    need = L.attn_bwd_bf16grad_workspace_bytes(1, 1, 4, 2, 64, 64, 64)
    assert _bwd_g(L, ws_bytes=need - 1) == WORKSPACE
    assert _bwd_g(L, ws=MIS) == WORKSPACE


def _bwd(L, ws=P, ws_bytes=1 << 20, ptrs=None, **kw):
    a = dict(dt=1, B=1, Hq=4, Hkv=2, N=64, d=64, causal=1, scale=0.125)
    a.update(kw)
    ptrs = ptrs or [P] * 9
    return L.attn_bwd(a["dt"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"],
                      *ptrs, ws, ws_bytes, NUL)


def test_bwd_refusals(L):
    assert _bwd(L, Hq=5, Hkv=2) == INVALID
    assert _bwd(L, d=96) == UNSUPPORTED
    assert _bwd(L, scale=float("-inf")) == INVALID
    for which in range(9):
        ptrs = [P] * 9
        ptrs[which] = NUL
        assert _bwd(L, ptrs=ptrs) == INVALID
    need = L.attn_bwd_workspace_bytes(1, 1, 4, 2, 64, 64)
    assert _bwd(L, ws_bytes=need - 1) == WORKSPACE
    assert _bwd(L, ws=NUL) == WORKSPACE
    assert _bwd(L, ws=MIS) == WORKSPACE


def _dec(lib_, ptrs=None, **kw):
    a = dict(dt=1, B=1, Hq=32, Hkv=8, L=4096, d=128, scale=0.088, S=16)
    a.update(kw)
    ptrs = ptrs or [P] * 5
    return lib_.attn_decode(a["dt"], a["B"], a["Hq"], a["Hkv"], a["L"], a["d"], a["scale"], a["S"],
                            *ptrs, NUL)


def test_decode_refusals(L):
    assert _dec(L, S=0) == INVALID
    assert _dec(L, S=-3) == INVALID
    assert _dec(L, L=0) == INVALID
    assert _dec(L, Hq=12, Hkv=8) == INVALID
    assert _dec(L, Hq=34, Hkv=2) == UNSUPPORTED      # group of 17 query heads
    assert _dec(L, d=80) == UNSUPPORTED
    assert _dec(L, scale=float("nan")) == INVALID
    for which in range(5):
        ptrs = [P] * 5
        ptrs[which] = MIS
        assert _dec(L, ptrs=ptrs) == INVALID


def test_merge_refusals(L):
    assert L.attn_lse_merge(0, 4, 2, 64, P, P, P, P, NUL) == INVALID
    assert L.attn_lse_merge(1, 4, 0, 64, P, P, P, P, NUL) == INVALID
    assert L.attn_lse_merge(1, 4, 2, 12, P, P, P, P, NUL) == UNSUPPORTED
    assert L.attn_lse_merge(1, 4, 2, 64, NUL, P, P, P, NUL) == INVALID
    assert L.attn_lse_merge(1, 4, 2, 64, P, P, P, MIS, NUL) == INVALID


def test_bwd_stage_refusals(L):
    assert L.attn_bwd_preprocess(1, 0, 4, 64, 64, P, P, P, NUL) == INVALID
    assert L.attn_bwd_preprocess(1, 1, 4, 64, 40, P, P, P, NUL) == UNSUPPORTED
    assert L.attn_bwd_preprocess(1, 1, 4, 64, 64, P, P, MIS, NUL) == INVALID
    args = [1, 1, 4, 2, 64, 64, 1, 0.125]
    assert L.attn_bwd_dkdv(1, 1, 4, 3, 64, 64, 1, 0.125, *([P] * 8), NUL) == INVALID
    assert L.attn_bwd_dkdv(*args, *([P] * 7), NUL, NUL) == INVALID
    assert L.attn_bwd_dq(1, 1, 4, 2, 64, 64, 1, float("nan"), *([P] * 7), NUL) == INVALID
    assert L.attn_bwd_dq(*args, *([P] * 6), MIS, NUL) == INVALID
    assert L.attn_bwd_grads(1, 1, 4, 3, 64, 64, 1, 0.125, *([P] * 9), NUL) == INVALID
    assert L.attn_bwd_grads(1, 1, 4, 2, 64, 40, 1, 0.125, *([P] * 9), NUL) == UNSUPPORTED
    for which in range(9):
        ptrs = [P] * 9
        ptrs[which] = MIS
        assert L.attn_bwd_grads(*args, *ptrs, NUL) == INVALID
        ptrs[which] = NUL
        assert L.attn_bwd_grads(*args, *ptrs, NUL) == INVALID


def test_bwd_dlse_refusals(L):
    args = [1, 1, 4, 2, 64, 64, 1, 0.125]
    ws, nb = P, ctypes.c_size_t(1 << 20)
    for which in range(10):
        ptrs = [P] * 10
        ptrs[which] = MIS
        assert L.attn_bwd_dlse(*args, *ptrs, ws, nb, NUL) == INVALID
    assert L.attn_bwd_dlse(*args, *([P] * 6), NUL, *([P] * 3), ws, nb, NUL) == INVALID   # no dlse
    assert L.attn_bwd_dlse(*args, *([P] * 10), ws, ctypes.c_size_t(16), NUL) == WORKSPACE
    assert L.attn_bwd_dlse(1, 1, 4, 3, 64, 64, 1, 0.125, *([P] * 10), ws, nb, NUL) == INVALID


def test_fwd_kv_refusals(L):
    def call(Nq=32, Nk=64, d=64, scale=0.125, ptrs=None):
        ptrs = ptrs or [P] * 5
        return L.attn_fwd_kv(1, 1, 4, 2, Nq, Nk, d, 1, scale, *ptrs, NUL)
    assert call(Nq=0) == INVALID
    assert call(Nq=65) == INVALID                   # more queries than keys
    assert call(Nk=-1) == INVALID
    assert call(d=48) == UNSUPPORTED
    assert call(scale=float("inf")) == INVALID
    for which in range(5):
        ptrs = [P] * 5
        ptrs[which] = MIS
        assert call(ptrs=ptrs) == INVALID


def test_bwd_kv_refusals(L):
    def call(Nq=32, Nk=64, d=64, scale=0.125, ptrs=None, nb=1 << 20, dt=1):
        ptrs = ptrs or [P] * 10
        return L.attn_bwd_kv(dt, 1, 4, 2, Nq, Nk, d, 1, scale, *ptrs, P, ctypes.c_size_t(nb), NUL)
    assert call(Nq=0) == INVALID
    assert call(Nq=65) == INVALID                   # more queries than keys
    assert call(Nk=-1) == INVALID
    assert call(d=48) == UNSUPPORTED
    assert call(dt=2) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(nb=16) == WORKSPACE                 # below 4 heads x 32 rows x 4 bytes
    for which in range(10):
        ptrs = [P] * 10
        ptrs[which] = MIS
        assert call(ptrs=ptrs) == INVALID
        if which != 6:                              # dlse may be null
            ptrs[which] = NUL
            assert call(ptrs=ptrs) == INVALID


def test_ex_refusals(L):
    def fwd(o_dt=1, Nq=32, Nk=64, ptrs=None):
        ptrs = ptrs or [P] * 5
        return L.attn_fwd_ex(1, o_dt, 1, 4, 2, Nq, Nk, 64, 1, 0.125, *ptrs, NUL)
    assert fwd(o_dt=2) == INVALID
    assert fwd(o_dt=-1) == INVALID
    assert fwd(Nq=65) == INVALID
    for which in range(5):
        ptrs = [P] * 5
        ptrs[which] = MIS
        assert fwd(ptrs=ptrs) == INVALID

    def bwd(o_dt=1, Nq=32, Nk=64, ptrs=None, nb=1 << 20):
        ptrs = ptrs or [P] * 10
        return L.attn_bwd_ex(1, o_dt, 1, 4, 2, Nq, Nk, 64, 1, 0.125, *ptrs, P, ctypes.c_size_t(nb), NUL)
    assert bwd(o_dt=7) == INVALID
    assert bwd(Nq=65) == INVALID
    assert bwd(nb=16) == WORKSPACE
    for which in range(10):
        ptrs = [P] * 10
        ptrs[which] = MIS
        assert bwd(ptrs=ptrs) == INVALID


def test_rope_refusals(L):
    def rope(dt=1, B=1, H=2, N=8, d=64, pos0=0, base=1e4, x=P, y=P):
        return L.attn_rope(dt, B, H, N, d, pos0, base, 0, x, y, NUL)
    assert rope(B=0) == INVALID
    assert rope(N=0) == INVALID
    assert rope(dt=3) == INVALID
    assert rope(d=48) == UNSUPPORTED
    assert rope(base=0.0) == INVALID
    assert rope(base=-2.0) == INVALID
    assert rope(base=float("inf")) == INVALID
    assert rope(pos0=1 << 41) == INVALID
    assert rope(x=MIS) == INVALID
    assert rope(y=NUL) == INVALID

    def fwd(Nq=32, Nk=64, base=1e4, ptrs=None):
        ptrs = ptrs or [P] * 7
        return L.attn_fwd_rope(1, 1, 4, 2, Nq, Nk, 64, 1, 0.125, base, *ptrs, NUL)
    assert fwd(Nq=65) == INVALID
    assert fwd(base=0.0) == INVALID
    for which in range(7):
        ptrs = [P] * 7
        ptrs[which] = MIS
        assert fwd(ptrs=ptrs) == INVALID

    def bwd(Nq=32, Nk=64, base=1e4, ptrs=None, nb=1 << 20):
        ptrs = ptrs or [P] * 10
        return L.attn_bwd_rope(1, 1, 4, 2, Nq, Nk, 64, 1, 0.125, base, *ptrs, P, ctypes.c_size_t(nb), NUL)
    assert bwd(Nq=65) == INVALID
    assert bwd(base=float("nan")) == INVALID
    assert bwd(nb=16) == WORKSPACE
    for which in range(10):
        ptrs = [P] * 10
        ptrs[which] = MIS
        assert bwd(ptrs=ptrs) == INVALID


def test_decode_append_refusals(L):
    def call(dt=1, B=2, Hq=8, Hkv=2, Lc=64, d=128, scale=0.088, S=4, ptrs=None, lens=P):
        ptrs = ptrs or [P] * 5
        return L.attn_decode_append(dt, B, Hq, Hkv, Lc, d, scale, S, *ptrs, lens, P, P, P, P, NUL)
    assert call(B=0) == INVALID
    assert call(Hq=6, Hkv=4) == INVALID
    assert call(S=0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(dt=0) == UNSUPPORTED                 # f32: no append kernel
    assert call(d=32) == UNSUPPORTED
    assert call(scale=0.0) == UNSUPPORTED
    assert call(Hq=34, Hkv=2) == UNSUPPORTED         # group of 17 heads
    # a head's cache must stay addressable by 32-bit buffer offsets
    assert call(Lc=(1 << 31) // 256) == UNSUPPORTED
    assert call(lens=NUL) == INVALID
    assert call(lens=ctypes.c_void_p(0x10002)) == INVALID
    for which in range(5):
        ptrs = [P] * 5
        ptrs[which] = MIS
        assert call(ptrs=ptrs) == INVALID
    assert L.attn_decode_append(1, 2, 8, 2, 64, 128, 0.088, 4, *([P] * 6), P, P, P, MIS, NUL) == INVALID


def _plan(L, dt, B, Hq, Hkv, Nq, Nk, d, scale, causal=1):
    g, b = ctypes.c_int(-1), ctypes.c_int(-1)
    one = L.attn_bwd_grads_plan(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, ctypes.byref(g),
                                ctypes.byref(b))
    return one, g.value, b.value


def test_bwd_grads_plan_query(L):
    """Whether the gradient stage is one kernel (host-side answer, no device work)."""
    assert _plan(L, 1, 4, 12, 4, 1024, 1024, 64, 0.125)[0] == 1
    assert _plan(L, 1, 1, 32, 8, 4096, 4096, 128, 0.088)[0] == 0     # d = 128: two kernels
    assert _plan(L, 1, 1, 32, 8, 512, 512, 128, 0.088)[0] == 1       # ... except on small grids
    assert _plan(L, 1, 1, 32, 8, 128, 128, 128, 0.088)[0] == 1
    assert _plan(L, 0, 4, 12, 4, 1024, 1024, 64, 0.125)[0] == 0      # f32: row-wise kernels
    assert _plan(L, 1, 4, 12, 4, 1024, 1024, 64, 0.0)[0] == 0        # scale 0: row-wise
    assert _plan(L, 1, 4, 12, 4, 1024, 1024, 40, 0.125) == (0, 0, 0)  # unsupported head dim
    assert _plan(L, 1, 4, 12, 4, 0, 0, 64, 0.125) == (0, 0, 0)
    assert _plan(L, 1, 4, 12, 4, 1024, 1000, 64, 0.125) == (0, 0, 0)  # Nk < Nq
    assert _plan(L, 1, 4, 12, 4, 1024, 1024, 64, float("nan")) == (0, 0, 0)


# The one-launch plan is a kernel argument of at most 48 block groups.  The
# dK/dV side splits a group wherever the key tiles' head split changes, so
# before the caps shrank, cross-length shapes such as 12/1 heads at Nq = 3008
# against Nk = 3072 planned 49 groups and wrote past the plan's arrays.
PLAN_SHAPES = [(1, 12, 1, nq, nk) for nk in (3072, 6016, 9024) for nq in (nk - 64, nk - 1, nk - 500)] + \
    [(B, Hq, Hkv, nq, nk) for B in (1, 2, 4) for Hq, Hkv in ((12, 1), (12, 4), (24, 2), (60, 1), (8, 8))
     for nk in (256, 1000, 2048, 4097) for nq in (1, nk // 3, nk - 7, nk)]


@pytest.mark.parametrize("causal", [1, 0])
def test_bwd_grads_plan_fits(L, causal):
    for B, Hq, Hkv, nq, nk in PLAN_SHAPES:
        one, groups, blocks = _plan(L, 1, B, Hq, Hkv, nq, nk, 64, 0.125, causal)
        assert one == 1, (B, Hq, Hkv, nq, nk)
        assert 1 <= groups <= 48, (B, Hq, Hkv, nq, nk, groups)
        # every dK/dV key tile and dQ query tile of every head is one block at least
        nkt, nqt = (nk + 63) // 64, (nq + 127) // 128
        assert blocks >= nkt * B * Hkv + nqt * B * Hq, (B, Hq, Hkv, nq, nk, blocks)
        assert blocks % 8 == 0


def test_no_unexpected_exports(L):
    """Only the declared attn_* functions are exported with C linkage."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    c_names = {n for n in exported if n.startswith("attn_")}
    assert c_names == set(_declared_functions())


def test_decode_merged_refusals(L):
    args = [1, 1, 32, 8, 4096, 128, 0.088, 16]
    assert L.attn_decode_merged(1, 1, 32, 8, 4096, 128, 0.088, 0, *([P] * 7), NUL) == INVALID
    assert L.attn_decode_merged(1, 1, 32, 8, 4096, 96, 0.088, 16, *([P] * 7), NUL) == UNSUPPORTED
    assert L.attn_decode_merged(1, 1, 34, 8, 4096, 128, 0.088, 16, *([P] * 7), NUL) == INVALID
    assert L.attn_decode_merged(*args, *([P] * 6), MIS, NUL) == INVALID
    assert L.attn_decode_merged(*args, NUL, *([P] * 6), NUL) == INVALID


_Layout = attn.AttnLayout


@pytest.mark.parametrize("lay", [
    (0, 64, 64), (4096, 0, 64), (4096, 64, 32),          # non-positive strides, a row shorter than d
    (4096, 64, 68), (4100, 64, 64), (4096, 68, 64),       # bf16 strides not a multiple of 16 bytes
    (1 << 40, 64, 1 << 31),                               # a row stride past 2^31 - 1
])
def test_strided_refuses_bad_layouts(L, lay):
    bad = _Layout(*lay)
    rc = L.attn_fwd_strided(1, 0, 1, 4, 2, 64, 64, 64, 1, 0.125, P, ctypes.byref(bad), P, None, P, None,
                            P, None, P, NUL)
    assert rc == INVALID
    # the same layout on dout (bf16, the rules of the input dtype)
    rc = L.attn_bwd_strided(1, 0, 1, 4, 2, 64, 64, 64, 1, 0.125, P, None, P, None, P, None, P, None, P,
                            P, ctypes.byref(bad), None, P, None, P, None, P, None, P, 1 << 20, NUL)
    assert rc == INVALID


def test_strided_refusals_like_the_contiguous_forms(L):
    ok = _Layout(64 * 8 * 64, 64, 8 * 64)
    # Nk < Nq, a bad output dtype, a misaligned pointer: refused before the layouts matter
    assert L.attn_fwd_strided(1, 0, 1, 4, 2, 64, 32, 64, 1, 0.125, P, ctypes.byref(ok), P, None, P, None,
                              P, None, P, NUL) == INVALID
    assert L.attn_fwd_strided(1, 5, 1, 4, 2, 64, 64, 64, 1, 0.125, P, None, P, None, P, None, P, None,
                              P, NUL) == INVALID
    assert L.attn_fwd_strided(1, 0, 1, 4, 2, 64, 64, 64, 1, 0.125, MIS, None, P, None, P, None, P, None,
                              P, NUL) == INVALID
    assert L.attn_bwd_strided(1, 0, 1, 4, 2, 64, 64, 64, 1, 0.125, P, None, P, None, P, None, P, None, P,
                              P, None, None, P, None, P, None, P, None, P, 8, NUL) == WORKSPACE
