"""CPU double-precision oracle for causal grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library neither links nor
calls it, and it shares no code with the HIP path.

This module is a thin ctypes wrapper over ``attn_oracle.c``: it converts numpy
arrays to contiguous float64 and passes pointers.  All arithmetic is in the C
file, which states the definition it follows and the passage behind each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source into a shared library with gcc.

    Built with -O2 and without fast-math, so double-precision semantics hold.
    """
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what}: oracle returned status {rc}")


def _shapes(q, k):
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k disagree in batch or head dimension")
    return B, Hq, Hkv, Nq, Nk, d


class Oracle:
    """ctypes view of one built oracle library (the default one, or a test variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_attn_fwd.argtypes = [i, i, i, i, i, i, i, d, _D, _D, _D, _D, _D]
        lib.oracle_attn_bwd.argtypes = [i, i, i, i, i, i, i, d, _D, _D, _D, _D, _D, _D, _D]
        lib.oracle_attn_bwd_dlse.argtypes = [i, i, i, i, i, i, i, d] + [_D] * 8
        lib.oracle_attn_fwd_dual.argtypes = [i, i, i, i, i, i, i, d] + [_D] * 10
        lib.oracle_dual_xsinx.argtypes = [d, _D, _D]
        lib.oracle_attn_decode.argtypes = [i, i, i, i, i, d, i, _D, _D, _D, _D, _D]
        lib.oracle_lse_merge.argtypes = [i, i, i, i, _D, _D, _D, _D]
        lib.oracle_state_combine.argtypes = [i, d, d, _D, d, d, _D, _D, _D, _D]
        lib.oracle_state_combine.restype = None
        lib.oracle_attn_decode_append.argtypes = [i, i, i, i, i, d, _D, _D, _D, _D, _D,
                                                  ctypes.POINTER(ctypes.c_int), _D, _D]
        lib.oracle_rope.argtypes = [i, i, i, i, ctypes.c_long, d, i, _D, _D]
        for name in ("oracle_attn_fwd", "oracle_attn_bwd", "oracle_attn_bwd_dlse", "oracle_attn_fwd_dual",
                     "oracle_rope",
                     "oracle_dual_xsinx", "oracle_attn_decode", "oracle_lse_merge",
                     "oracle_attn_decode_append", "oracle_abi_version", "oracle_num_threads"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def rope(self, x, pos0: int, base: float, inverse: bool = False):
        """Rotary positions on x [B,H,N,d] (row n at position pos0 + n); inverse: the transposed
        rotation."""
        x = _f64(x)
        B, H, N, d = x.shape
        y = np.empty_like(x)
        _check(self.lib.oracle_rope(B, H, N, d, int(pos0), float(base), int(inverse), _p(x), _p(y)),
               "rope")
        return y

    def attn_fwd(self, q, k, v, causal: bool, scale: float):
        """Returns (o [B,Hq,Nq,d], lse [B,Hq,Nq]) in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
        o = np.empty_like(q)
        lse = np.empty((B, Hq, Nq))
        _check(self.lib.oracle_attn_fwd(B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale),
                                        _p(q), _p(k), _p(v), _p(o), _p(lse)), "attn_fwd")
        return o, lse

    def attn_bwd(self, q, k, v, dout, causal: bool, scale: float):
        """Returns (dq, dk, dv) in float64 for the upstream gradient dout of o."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        _check(self.lib.oracle_attn_bwd(B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale),
                                        _p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv)),
               "attn_bwd")
        return dq, dk, dv

    def attn_bwd_dlse(self, q, k, v, dout, dlse, causal: bool, scale: float):
        """Returns (dq, dk, dv) for upstream gradients dout of o and dlse [B,Hq,Nq] of lse."""
        q, k, v, dout, dlse = _f64(q), _f64(k), _f64(v), _f64(dout), _f64(dlse)
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
        if dlse.shape != (B, Hq, Nq):
            raise ValueError("dlse shape mismatch")
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        _check(self.lib.oracle_attn_bwd_dlse(B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale),
                                             _p(q), _p(k), _p(v), _p(dout), _p(dlse), _p(dq),
                                             _p(dk), _p(dv)), "attn_bwd_dlse")
        return dq, dk, dv

    def attn_fwd_dual(self, q, tq, k, tk, v, tv, causal: bool, scale: float):
        """Forward on dual numbers: returns (o, o_tangent, lse, lse_tangent)."""
        q, tq, k, tk, v, tv = (_f64(x) for x in (q, tq, k, tk, v, tv))
        B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
        o, to = np.empty_like(q), np.empty_like(q)
        lse, tlse = np.empty((B, Hq, Nq)), np.empty((B, Hq, Nq))
        _check(self.lib.oracle_attn_fwd_dual(B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale),
                                             _p(q), _p(tq), _p(k), _p(tk), _p(v), _p(tv),
                                             _p(o), _p(to), _p(lse), _p(tlse)), "attn_fwd_dual")
        return o, to, lse, tlse

    def dual_xsinx(self, x: float):
        """f(x) = x sin x on a dual number: returns (value, derivative)."""
        val, der = ctypes.c_double(), ctypes.c_double()
        _check(self.lib.oracle_dual_xsinx(float(x), ctypes.byref(val), ctypes.byref(der)),
               "dual_xsinx")
        return val.value, der.value

    def attn_decode(self, q, k_cache, v_cache, scale: float, n_splits: int):
        """q [B,Hq,d], caches [B,Hkv,L,d] -> (part_o [B,Hq,S,d], part_lse [B,Hq,S])."""
        q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
        B, Hq, d = q.shape
        _, Hkv, L, _ = kc.shape
        po = np.empty((B, Hq, n_splits, d))
        pl = np.empty((B, Hq, n_splits))
        _check(self.lib.oracle_attn_decode(B, Hq, Hkv, L, d, float(scale), int(n_splits),
                                           _p(q), _p(kc), _p(vc), _p(po), _p(pl)), "attn_decode")
        return po, pl

    def attn_decode_append(self, q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float):
        """One decode step with cache append: q [B,Hq,d], k_new/v_new [B,Hkv,d], caches
        [B,Hkv,Lcap,d], seq_lens [B] -> (o [B,Hq,d], lse [B,Hq], k_cache', v_cache') with the
        caches returned as updated copies (the inputs are not modified)."""
        q, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
        kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
        lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        B, Hq, d = q.shape
        _, Hkv, Lcap, _ = kc.shape
        if kn.shape != (B, Hkv, d) or vn.shape != (B, Hkv, d) or lens.shape != (B,):
            raise ValueError("k_new, v_new or seq_lens shape mismatch")
        o = np.empty((B, Hq, d))
        lse = np.empty((B, Hq))
        _check(self.lib.oracle_attn_decode_append(
            B, Hq, Hkv, Lcap, d, float(scale), _p(q), _p(kn), _p(vn), _p(kc), _p(vc),
            lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), _p(o), _p(lse)), "attn_decode_append")
        return o, lse, kc, vc

    def lse_merge(self, part_o, part_lse):
        """part_o [B,Hq,S,d], part_lse [B,Hq,S] -> (o [B,Hq,d], lse [B,Hq])."""
        po, pl = _f64(part_o), _f64(part_lse)
        B, Hq, S, d = po.shape
        o = np.empty((B, Hq, d))
        lse = np.empty((B, Hq))
        _check(self.lib.oracle_lse_merge(B, Hq, S, d, _p(po), _p(pl), _p(o), _p(lse)),
               "lse_merge")
        return o, lse

    def state_combine(self, s1, s2):
        """Combine two online-softmax states (m, l, a); returns a new (m, l, a)."""
        m1, l1, a1 = s1
        m2, l2, a2 = s2
        a1, a2 = _f64(a1), _f64(a2)
        a = np.empty_like(a1)
        m, l = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_state_combine(a1.shape[0], float(m1), float(l1), _p(a1), float(m2),
                                      float(l2), _p(a2), ctypes.byref(m), ctypes.byref(l), _p(a))
        return m.value, l.value, a


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def attn_fwd(q, k, v, causal, scale):
    return default().attn_fwd(q, k, v, causal, scale)


def attn_bwd(q, k, v, dout, causal, scale):
    return default().attn_bwd(q, k, v, dout, causal, scale)


def rope(x, pos0, base, inverse=False):
    return default().rope(x, pos0, base, inverse)


def attn_fwd_rope(q, k, v, causal, scale, base):
    """Attention of rotated q (positions Nk - Nq + i) and rotated k (positions j)."""
    Nq, Nk = q.shape[2], k.shape[2]
    return default().attn_fwd(rope(q, Nk - Nq, base), rope(k, 0, base), v, causal, scale)


def attn_bwd_rope(q, k, v, dout, causal, scale, base, dlse=None):
    """Gradients with respect to the unrotated q and k: the attention backward at the rotated
    inputs, carried back through the rotations by their transposes."""
    Nq, Nk = q.shape[2], k.shape[2]
    qr, kr = rope(q, Nk - Nq, base), rope(k, 0, base)
    if dlse is None:
        dq, dk, dv = attn_bwd(qr, kr, v, dout, causal, scale)
    else:
        dq, dk, dv = attn_bwd_dlse(qr, kr, v, dout, dlse, causal, scale)
    return rope(dq, Nk - Nq, base, inverse=True), rope(dk, 0, base, inverse=True), dv


def attn_bwd_dlse(q, k, v, dout, dlse, causal, scale):
    return default().attn_bwd_dlse(q, k, v, dout, dlse, causal, scale)


def attn_fwd_dual(q, tq, k, tk, v, tv, causal, scale):
    return default().attn_fwd_dual(q, tq, k, tk, v, tv, causal, scale)


def dual_xsinx(x):
    return default().dual_xsinx(x)


def attn_decode(q, k_cache, v_cache, scale, n_splits):
    return default().attn_decode(q, k_cache, v_cache, scale, n_splits)


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale):
    return default().attn_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale)


def lse_merge(part_o, part_lse):
    return default().lse_merge(part_o, part_lse)


def state_combine(s1, s2):
    return default().state_combine(s1, s2)
