"""Causal grouped-query flash attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (declared in
``include/attn.h``).  It only marshals arguments: it checks tensor shapes and
dtypes, allocates output tensors with torch (device memory is torch's
plumbing), and passes raw device pointers and the current HIP stream to the
library.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
           "attn_bwd_grads", "attn_bwd_grads_single_launch", "attn_decode_append", "attn_fwd_kv",
           "attn_bwd_dlse", "attn_bwd_kv", "attn_rope", "attn_fwd_rope", "attn_bwd_rope",
           "attn_fwd_ex", "attn_bwd_ex",
           "attn_bwd_dkdv", "attn_bwd_dq", "attn_decode", "attn_lse_merge",
           "attn_decode_merged",
           "attn_status_str", "attn_abi_version", "AttnError", "lib", "LIB_PATH",
           "ATTN_F32", "ATTN_BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32 = 0
ATTN_BF16 = 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
          3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}

_lib = None


class AttnError(RuntimeError):
    """A non-OK status returned by libattn.so."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({attn_status_str(status)})")


def lib() -> ctypes.CDLL:
    """The loaded libattn.so, with argument types declared (loads on first use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    i, f, p, sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.attn_fwd.argtypes = [i, i, i, i, i, i, i, f, p, p, p, p, p, p]
    L.attn_fwd.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [i, i, i, i, i, i, i, f] + [p] * 9 + [p, sz, p]
    L.attn_bwd.restype = i
    L.attn_bwd_preprocess.argtypes = [i, i, i, i, i, p, p, p, p]
    L.attn_bwd_preprocess.restype = i
    L.attn_bwd_dkdv.argtypes = [i, i, i, i, i, i, i, f] + [p] * 9
    L.attn_bwd_dkdv.restype = i
    L.attn_bwd_dq.argtypes = [i, i, i, i, i, i, i, f] + [p] * 8
    L.attn_bwd_grads.argtypes = [i, i, i, i, i, i, i, f] + [p] * 10
    L.attn_bwd_grads.restype = i
    L.attn_bwd_dlse.argtypes = [i, i, i, i, i, i, i, f] + [p] * 10 + [p, sz, p]
    L.attn_bwd_dlse.restype = i
    L.attn_fwd_kv.argtypes = [i, i, i, i, i, i, i, i, f, p, p, p, p, p, p]
    L.attn_fwd_kv.restype = i
    L.attn_bwd_kv.argtypes = [i, i, i, i, i, i, i, i, f] + [p] * 10 + [p, sz, p]
    L.attn_bwd_kv.restype = i
    dbl, ll = ctypes.c_double, ctypes.c_longlong
    L.attn_fwd_ex.argtypes = [i, i, i, i, i, i, i, i, i, f, p, p, p, p, p, p]
    L.attn_fwd_ex.restype = i
    L.attn_bwd_ex.argtypes = [i, i, i, i, i, i, i, i, i, f] + [p] * 10 + [p, sz, p]
    L.attn_bwd_ex.restype = i
    L.attn_rope.argtypes = [i, i, i, i, i, ll, dbl, i, p, p, p]
    L.attn_rope.restype = i
    L.attn_fwd_rope.argtypes = [i, i, i, i, i, i, i, i, f, dbl] + [p] * 7 + [p]
    L.attn_fwd_rope.restype = i
    L.attn_bwd_rope.argtypes = [i, i, i, i, i, i, i, i, f, dbl] + [p] * 10 + [p, sz, p]
    L.attn_bwd_rope.restype = i
    L.attn_decode_append.argtypes = [i, i, i, i, i, i, f, i] + [p] * 10 + [p]
    L.attn_decode_append.restype = i
    L.attn_bwd_grads_single_launch.argtypes = [i, i, i, f]
    L.attn_bwd_grads_single_launch.restype = i
    L.attn_bwd_dq.restype = i
    L.attn_decode.argtypes = [i, i, i, i, i, i, f, i, p, p, p, p, p, p]
    L.attn_decode.restype = i
    L.attn_decode_merged.argtypes = [i, i, i, i, i, i, f, i] + [p] * 7 + [p]
    L.attn_decode_merged.restype = i
    L.attn_lse_merge.argtypes = [i, i, i, i, p, p, p, p, p]
    L.attn_lse_merge.restype = i
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_abi_version.argtypes = []
    L.attn_abi_version.restype = i
    _lib = L
    return L


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def attn_abi_version() -> int:
    return int(lib().attn_abi_version())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported input dtype {t.dtype}; use float32 or bfloat16")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check(fn: str, rc: int):
    if rc != 0:
        raise AttnError(fn, rc)


def attn_fwd(q, k, v, causal: bool = True, scale: float | None = None, o=None, lse=None,
             stream=None):
    """Forward.  q [B,Hq,N,d], k/v [B,Hkv,N,d] (float32 or bfloat16) -> (o f32, lse f32)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, Hkv, N, d] with q's batch, length, head dim and dtype")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if o is None:
        o = torch.empty((B, Hq, N, d), device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((B, Hq, N), device=q.device, dtype=torch.float32)
    rc = lib().attn_fwd(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), scale,
                        _ptr(q), _ptr(k), _ptr(v), _ptr(_dev(o, "o")), _ptr(_dev(lse, "lse")),
                        _stream(stream))
    _check("attn_fwd", rc)
    return o, lse


def attn_bwd_workspace_bytes(dtype_code: int, B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(int(dtype_code), B, Hq, Hkv, N, d))


def attn_bwd(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, dlse=None):
    """Backward.  Returns (dq, dk, dv), all float32, for the upstream gradient dout of o
    (and, with dlse [B,Hq,N] float32, of lse: attn_bwd_dlse)."""
    if dlse is not None:
        return attn_bwd_dlse(q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv, workspace,
                             stream)
    return _bwd_call("attn_bwd", q, k, v, o, lse, dout, None, causal, scale, dq, dk, dv, workspace,
                     stream)


def attn_bwd_dlse(q, k, v, o, lse, dout, dlse, causal: bool = True, scale: float | None = None,
                  dq=None, dk=None, dv=None, workspace=None, stream=None):
    """attn_bwd with an upstream gradient dlse [B,Hq,N] float32 of lse as well."""
    return _bwd_call("attn_bwd_dlse", q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv,
                     workspace, stream)


def attn_bwd_kv(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
                dq=None, dk=None, dv=None, workspace=None, stream=None, dlse=None):
    """Backward of attn_fwd_kv: q, dout [B,Hq,Nq,d] against k, v [B,Hkv,Nk,d] (Nk >= Nq, the
    queries at the last Nq positions), o, lse from attn_fwd_kv, dlse [B,Hq,Nq] float32 or None.
    Returns (dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d]), all float32."""
    return _bwd_call("attn_bwd_kv", q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv,
                     workspace, stream)


def _bwd_call(fn, q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv, workspace, stream,
              base=None):
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (dout, "dout")):
        _dev(t, n)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if fn not in ("attn_bwd_kv", "attn_bwd_rope", "attn_bwd_ex") and Nk != Nq:
        raise ValueError(f"{fn} needs as many keys as queries (attn_bwd_kv takes Nk > Nq)")
    if dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must match q in shape and dtype")
    if (o.dtype != torch.float32 and fn != "attn_bwd_ex") or lse.dtype != torch.float32:
        raise ValueError("o and lse must be the float32 outputs of the forward")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    code = _dtype_code(q)
    if dq is None:
        dq = torch.empty((B, Hq, Nq, d), device=q.device, dtype=torch.float32)
    if dk is None:
        dk = torch.empty((B, Hkv, Nk, d), device=q.device, dtype=torch.float32)
    if dv is None:
        dv = torch.empty((B, Hkv, Nk, d), device=q.device, dtype=torch.float32)
    nbytes = attn_bwd_workspace_bytes(code, B, Hq, Hkv, Nq, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    if dlse is not None:
        if dlse.dtype != torch.float32 or tuple(dlse.shape) != (B, Hq, Nq):
            raise ValueError("dlse must be float32 of the shape of lse")
        dlse_p = _ptr(_dev(dlse, "dlse"))
    elif fn == "attn_bwd_dlse":
        raise ValueError("attn_bwd_dlse needs dlse")
    else:
        dlse_p = None
    head = ((code, _dtype_code(o)) if fn == "attn_bwd_ex" else (code,)) + (B, Hq, Hkv) + \
        ((Nq, Nk) if fn in ("attn_bwd_kv", "attn_bwd_rope", "attn_bwd_ex") else (Nq,)) + \
        (d, int(bool(causal)), scale) + ((float(base),) if fn == "attn_bwd_rope" else ()) + \
        (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout))
    tail = (_ptr(_dev(dq, "dq")), _ptr(_dev(dk, "dk")), _ptr(_dev(dv, "dv")), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    rc = getattr(lib(), fn)(*head, *((dlse_p,) if fn != "attn_bwd" else ()), *tail)
    _check(fn, rc)
    return dq, dk, dv


def attn_bwd_preprocess(o, dout, delta=None, stream=None):
    """Stage 1 of the backward: delta [B,Hq,N] f32 = rowwise dout . o."""
    torch = _torch()
    _dev(o, "o")
    _dev(dout, "dout")
    B, Hq, N, d = dout.shape
    if delta is None:
        delta = torch.empty((B, Hq, N), device=dout.device, dtype=torch.float32)
    rc = lib().attn_bwd_preprocess(_dtype_code(dout), B, Hq, N, d, _ptr(o), _ptr(dout),
                                   _ptr(_dev(delta, "delta")), _stream(stream))
    _check("attn_bwd_preprocess", rc)
    return delta


def attn_bwd_dkdv(q, k, v, lse, dout, delta, causal=True, scale=None, dk=None, dv=None,
                  stream=None):
    """Stage 2 of the backward: (dk, dv) f32."""
    torch = _torch()
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if dk is None:
        dk = torch.empty((B, Hkv, N, d), device=q.device, dtype=torch.float32)
    if dv is None:
        dv = torch.empty((B, Hkv, N, d), device=q.device, dtype=torch.float32)
    rc = lib().attn_bwd_dkdv(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), scale,
                             _ptr(_dev(q, "q")), _ptr(_dev(k, "k")), _ptr(_dev(v, "v")),
                             _ptr(_dev(lse, "lse")), _ptr(_dev(dout, "dout")),
                             _ptr(_dev(delta, "delta")), _ptr(_dev(dk, "dk")), _ptr(_dev(dv, "dv")),
                             _stream(stream))
    _check("attn_bwd_dkdv", rc)
    return dk, dv


def attn_bwd_dq(q, k, v, lse, dout, delta, causal=True, scale=None, dq=None, stream=None):
    """Stage 3 of the backward: dq f32."""
    torch = _torch()
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if dq is None:
        dq = torch.empty((B, Hq, N, d), device=q.device, dtype=torch.float32)
    rc = lib().attn_bwd_dq(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), scale,
                           _ptr(_dev(q, "q")), _ptr(_dev(k, "k")), _ptr(_dev(v, "v")),
                           _ptr(_dev(lse, "lse")), _ptr(_dev(dout, "dout")),
                           _ptr(_dev(delta, "delta")), _ptr(_dev(dq, "dq")), _stream(stream))
    _check("attn_bwd_dq", rc)
    return dq


def attn_fwd_kv(q, k, v, causal: bool = True, scale: float | None = None, o=None, lse=None,
                stream=None):
    """Forward of q [B,Hq,Nq,d] against k, v [B,Hkv,Nk,d] (Nk >= Nq, queries at the last Nq
    positions) -> (o [B,Hq,Nq,d] f32, lse [B,Hq,Nq] f32)."""
    torch = _torch()
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if o is None:
        o = torch.empty((B, Hq, Nq, d), device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), device=q.device, dtype=torch.float32)
    rc = lib().attn_fwd_kv(_dtype_code(q), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
                           _ptr(_dev(q, "q")), _ptr(_dev(k, "k")), _ptr(_dev(v, "v")),
                           _ptr(_dev(o, "o")), _ptr(_dev(lse, "lse")), _stream(stream))
    _check("attn_fwd_kv", rc)
    return o, lse


def attn_fwd_ex(q, k, v, causal: bool = True, scale: float | None = None, o_dtype=None, o=None,
                lse=None, stream=None):
    """The general forward: q [B,Hq,Nq,d] against k, v [B,Hkv,Nk,d] (Nk >= Nq), o in o_dtype
    (torch.float32, the default, or torch.bfloat16).  Returns (o, lse)."""
    torch = _torch()
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if o is None:
        o = torch.empty((B, Hq, Nq, d), device=q.device, dtype=o_dtype)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), device=q.device, dtype=torch.float32)
    rc = lib().attn_fwd_ex(_dtype_code(q), _dtype_code(o), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                           scale, _ptr(_dev(q, "q")), _ptr(_dev(k, "k")), _ptr(_dev(v, "v")),
                           _ptr(_dev(o, "o")), _ptr(_dev(lse, "lse")), _stream(stream))
    _check("attn_fwd_ex", rc)
    return o, lse


def attn_bwd_ex(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None, dq=None,
                dk=None, dv=None, workspace=None, stream=None, dlse=None):
    """The general backward: o from attn_fwd_ex in either dtype, dlse optional."""
    return _bwd_call("attn_bwd_ex", q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv,
                     workspace, stream)


def attn_rope(x, pos0: int, base: float, inverse: bool = False, y=None, stream=None):
    """Rotary positions on x [B,H,N,d] (row n at position pos0 + n) into y (default: a new
    tensor; y may be x).  inverse: the transposed rotation."""
    torch = _torch()
    B, H, N, d = x.shape
    if y is None:
        y = torch.empty_like(x)
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("y must match x in shape and dtype")
    rc = lib().attn_rope(_dtype_code(x), B, H, N, d, int(pos0), float(base), int(bool(inverse)),
                         _ptr(_dev(x, "x")), _ptr(_dev(y, "y")), _stream(stream))
    _check("attn_rope", rc)
    return y


def attn_fwd_rope(q, k, v, causal: bool = True, scale: float | None = None, base: float = 10000.0,
                  q_rot=None, k_rot=None, o=None, lse=None, stream=None):
    """Forward over rotated q (row i at position Nk - Nq + i) and k (row j at j).
    Returns (o, lse, q_rot, k_rot); attn_bwd_rope takes q_rot and k_rot."""
    torch = _torch()
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    q_rot = torch.empty_like(q) if q_rot is None else q_rot
    k_rot = torch.empty_like(k) if k_rot is None else k_rot
    if o is None:
        o = torch.empty((B, Hq, Nq, d), device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), device=q.device, dtype=torch.float32)
    rc = lib().attn_fwd_rope(_dtype_code(q), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
                             float(base), _ptr(_dev(q, "q")), _ptr(_dev(k, "k")), _ptr(_dev(v, "v")),
                             _ptr(_dev(q_rot, "q_rot")), _ptr(_dev(k_rot, "k_rot")),
                             _ptr(_dev(o, "o")), _ptr(_dev(lse, "lse")), _stream(stream))
    _check("attn_fwd_rope", rc)
    return o, lse, q_rot, k_rot


def attn_bwd_rope(q_rot, k_rot, v, o, lse, dout, causal: bool = True, scale: float | None = None,
                  base: float = 10000.0, dq=None, dk=None, dv=None, workspace=None, stream=None,
                  dlse=None):
    """Backward of attn_fwd_rope: (dq, dk, dv) with respect to the unrotated q, k and v."""
    return _bwd_call("attn_bwd_rope", q_rot, k_rot, v, o, lse, dout, dlse, causal, scale, dq, dk,
                     dv, workspace, stream, base=base)


def attn_bwd_grads(q, k, v, lse, dout, delta, causal=True, scale=None, dq=None, dk=None, dv=None,
                   stream=None):
    """Stages 2 and 3 of the backward as attn_bwd runs them: (dq, dk, dv) f32."""
    torch = _torch()
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if dq is None:
        dq = torch.empty((B, Hq, N, d), device=q.device, dtype=torch.float32)
    if dk is None:
        dk = torch.empty((B, Hkv, N, d), device=q.device, dtype=torch.float32)
    if dv is None:
        dv = torch.empty((B, Hkv, N, d), device=q.device, dtype=torch.float32)
    rc = lib().attn_bwd_grads(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), scale,
                              _ptr(_dev(q, "q")), _ptr(_dev(k, "k")), _ptr(_dev(v, "v")),
                              _ptr(_dev(lse, "lse")), _ptr(_dev(dout, "dout")),
                              _ptr(_dev(delta, "delta")), _ptr(_dev(dq, "dq")),
                              _ptr(_dev(dk, "dk")), _ptr(_dev(dv, "dv")), _stream(stream))
    _check("attn_bwd_grads", rc)
    return dq, dk, dv


def attn_bwd_grads_single_launch(dtype_code: int, N: int, d: int, scale: float) -> bool:
    """Whether attn_bwd_grads runs as one kernel for this dtype code, N, d, scale."""
    return bool(lib().attn_bwd_grads_single_launch(int(dtype_code), int(N), int(d), float(scale)))


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, n_splits: int,
                       scale: float | None = None, part_o=None, part_lse=None, o=None, lse=None,
                       stream=None):
    """One decode step with cache append.  q [B,Hq,d], k_new/v_new [B,Hkv,d], caches
    [B,Hkv,L_cap,d] (row seq_lens[b] is written), seq_lens int32 [B] on the device
    -> (o [B,Hq,d], lse [B,Hq]) f32."""
    torch = _torch()
    B, Hq, d = q.shape
    Hkv, L_cap = k_cache.shape[1], k_cache.shape[2]
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError(f"seq_lens must be int32 of shape ({B},)")
    if part_o is None:
        part_o = torch.empty((B, Hq, n_splits, d), device=q.device, dtype=torch.float32)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, n_splits), device=q.device, dtype=torch.float32)
    if o is None:
        o = torch.empty((B, Hq, d), device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((B, Hq), device=q.device, dtype=torch.float32)
    rc = lib().attn_decode_append(_dtype_code(q), B, Hq, Hkv, L_cap, d, scale, int(n_splits),
                                  _ptr(_dev(q, "q")), _ptr(_dev(k_new, "k_new")),
                                  _ptr(_dev(v_new, "v_new")), _ptr(_dev(k_cache, "k_cache")),
                                  _ptr(_dev(v_cache, "v_cache")), _ptr(_dev(seq_lens, "seq_lens")),
                                  _ptr(_dev(part_o, "part_o")), _ptr(_dev(part_lse, "part_lse")),
                                  _ptr(_dev(o, "o")), _ptr(_dev(lse, "lse")), _stream(stream))
    _check("attn_decode_append", rc)
    return o, lse


def attn_decode(q, k_cache, v_cache, n_splits: int, scale: float | None = None,
                part_o=None, part_lse=None, stream=None):
    """Split-KV decode.  q [B,Hq,d], caches [B,Hkv,L,d] -> (part_o [B,Hq,S,d], part_lse [B,Hq,S])."""
    torch = _torch()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    B, Hq, d = q.shape
    _, Hkv, L, _ = k_cache.shape
    if v_cache.shape != k_cache.shape or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("caches must be [B, Hkv, L, d] with q's dtype")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if part_o is None:
        part_o = torch.empty((B, Hq, n_splits, d), device=q.device, dtype=torch.float32)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, n_splits), device=q.device, dtype=torch.float32)
    rc = lib().attn_decode(_dtype_code(q), B, Hq, Hkv, L, d, scale, int(n_splits),
                           _ptr(q), _ptr(k_cache), _ptr(v_cache),
                           _ptr(_dev(part_o, "part_o")), _ptr(_dev(part_lse, "part_lse")),
                           _stream(stream))
    _check("attn_decode", rc)
    return part_o, part_lse


def attn_decode_merged(q, k_cache, v_cache, n_splits: int, scale: float | None = None,
                       part_o=None, part_lse=None, o=None, lse=None, stream=None):
    """Split-KV decode and the LSE merge in one call.

    Returns (o [B,Hq,d], lse [B,Hq], part_o, part_lse).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    B, Hq, d = q.shape
    _, Hkv, L, _ = k_cache.shape
    if v_cache.shape != k_cache.shape or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("caches must be [B, Hkv, L, d] with q's dtype")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    f32 = dict(device=q.device, dtype=torch.float32)
    part_o = torch.empty((B, Hq, n_splits, d), **f32) if part_o is None else part_o
    part_lse = torch.empty((B, Hq, n_splits), **f32) if part_lse is None else part_lse
    o = torch.empty((B, Hq, d), **f32) if o is None else o
    lse = torch.empty((B, Hq), **f32) if lse is None else lse
    rc = lib().attn_decode_merged(_dtype_code(q), B, Hq, Hkv, L, d, scale, int(n_splits),
                                  _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(_dev(part_o, "part_o")), _ptr(_dev(part_lse, "part_lse")),
                                  _ptr(_dev(o, "o")), _ptr(_dev(lse, "lse")), _stream(stream))
    _check("attn_decode_merged", rc)
    return o, lse, part_o, part_lse


def attn_lse_merge(part_o, part_lse, o=None, lse=None, stream=None):
    """Merge split partials: part_o [B,Hq,S,d], part_lse [B,Hq,S] -> (o [B,Hq,d], lse [B,Hq])."""
    torch = _torch()
    _dev(part_o, "part_o")
    _dev(part_lse, "part_lse")
    B, Hq, S, d = part_o.shape
    if o is None:
        o = torch.empty((B, Hq, d), device=part_o.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((B, Hq), device=part_o.device, dtype=torch.float32)
    rc = lib().attn_lse_merge(B, Hq, S, d, _ptr(part_o), _ptr(part_lse), _ptr(_dev(o, "o")),
                              _ptr(_dev(lse, "lse")), _stream(stream))
    _check("attn_lse_merge", rc)
    return o, lse
