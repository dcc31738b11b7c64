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
           "attn_bwd_grads", "attn_bwd_grads_plan", "attn_decode_append", "attn_fwd_kv",
           "attn_bwd_dlse", "attn_bwd_kv", "attn_rope", "attn_fwd_rope", "attn_bwd_rope",
           "attn_fwd_ex", "attn_bwd_ex", "attn_bwd_bf16grad", "attn_bwd_bf16grad_workspace_bytes",
           "attn_bwd_dkdv", "attn_bwd_dq", "attn_decode", "attn_lse_merge",
           "attn_decode_merged", "attn_read_probe", "attn_bwd_noalloc", "attn_fwd_strided",
           "attn_bwd_strided", "AttnLayout",
           "attn_status_str", "attn_abi_version", "AttnError", "lib", "LIB_PATH",
           "ATTN_F32", "ATTN_BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32 = 0
ATTN_BF16 = 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
          3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}

_lib = None


class AttnLayout(ctypes.Structure):
    """Element strides of a [B][H][N][d] tensor whose head dim is contiguous (attn_layout)."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


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
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m attention_causal_gqa_flash_amd.build first")
    L = ctypes.CDLL(LIB_PATH)
    i, f, p, sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.attn_fwd.argtypes = [i, i, i, i, i, i, i, f, p, p, p, p, p, p]
    L.attn_fwd.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [i, i, i, i, i, i, i, f] + [p] * 9 + [p, sz, p]
    L.attn_bwd.restype = i
    L.attn_bwd_noalloc.argtypes = [i, i, i, i, i, i, i, f] + [p] * 9 + [p]
    L.attn_bwd_noalloc.restype = i
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
    L.attn_bwd_bf16grad_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_bwd_bf16grad_workspace_bytes.restype = sz
    L.attn_bwd_bf16grad.argtypes = [i, i, i, i, i, i, i, i, i, f] + [p] * 10 + [p, sz, p]
    L.attn_bwd_bf16grad.restype = i
    L.attn_rope.argtypes = [i, i, i, i, i, ll, dbl, i, p, p, p]
    L.attn_rope.restype = i
    L.attn_fwd_rope.argtypes = [i, i, i, i, i, i, i, i, f, dbl] + [p] * 7 + [p]
    L.attn_fwd_rope.restype = i
    L.attn_bwd_rope.argtypes = [i, i, i, i, i, i, i, i, f, dbl] + [p] * 10 + [p, sz, p]
    L.attn_bwd_rope.restype = i
    L.attn_decode_append.argtypes = [i, i, i, i, i, i, f, i] + [p] * 10 + [p]
    L.attn_decode_append.restype = i
    ip = ctypes.POINTER(ctypes.c_int)
    L.attn_bwd_grads_plan.argtypes = [i, i, i, i, i, i, i, i, f, ip, ip]
    L.attn_bwd_grads_plan.restype = i
    L.attn_bwd_dq.restype = i
    L.attn_decode.argtypes = [i, i, i, i, i, i, f, i, p, p, p, p, p, p]
    L.attn_decode.restype = i
    L.attn_decode_merged.argtypes = [i, i, i, i, i, i, f, i] + [p] * 7 + [p]
    L.attn_decode_merged.restype = i
    L.attn_lse_merge.argtypes = [i, i, i, i, p, p, p, p, p]
    L.attn_lse_merge.restype = i
    lp = ctypes.POINTER(AttnLayout)
    L.attn_fwd_strided.argtypes = [i] * 8 + [i, f, p, lp, p, lp, p, lp, p, lp, p, p]
    L.attn_fwd_strided.restype = i
    L.attn_bwd_strided.argtypes = [i] * 8 + [i, f, p, lp, p, lp, p, lp, p, lp, p, p, lp, p,
                                             p, lp, p, lp, p, lp, p, sz, p]
    L.attn_bwd_strided.restype = i
    L.attn_read_probe.argtypes = [p, sz, p, p]
    L.attn_read_probe.restype = i
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


def _expect(t, shape, dtype, name, like=None):
    """t must be a contiguous device tensor of this shape and dtype (on like's device)."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, got {t.device}")
    return t


def _out(t, shape, dtype, name, like, stream):
    """The caller's output tensor (checked), or a new one.  A new tensor is
    allocated on the stream the call is enqueued on, so that torch's caching
    allocator does not hand its memory to other streams while the kernels may
    still be using it."""
    if t is not None:
        return _expect(t, shape, dtype, name, like)
    torch = _torch()
    if stream is None:
        return torch.empty(shape, device=like.device, dtype=dtype)
    with torch.cuda.stream(stream):
        return torch.empty(shape, device=like.device, dtype=dtype)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check(fn: str, rc: int):
    if rc != 0:
        raise AttnError(fn, rc)


def _qkv(q, k, v, square: bool):
    """Shapes of q [B,Hq,Nq,d] and k, v [B,Hkv,Nk,d] (same dtype, device); square: Nk == Nq."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _dtype_code(q)
    _expect(k, (B, Hkv, Nk, d), q.dtype, "k", q)
    _expect(v, (B, Hkv, Nk, d), q.dtype, "v", q)
    if square and Nk != Nq:
        raise ValueError("k and v must have as many rows as q (the Nq < Nk form is attn_fwd_kv / "
                         "attn_bwd_kv)")
    return B, Hq, Hkv, Nq, Nk, d


def _scale(scale, d):
    return float(d) ** -0.5 if scale is None else float(scale)


def attn_fwd(q, k, v, causal: bool = True, scale: float | None = None, o=None, lse=None,
             stream=None):
    """Forward.  q [B,Hq,N,d], k/v [B,Hkv,N,d] (float32 or bfloat16) -> (o f32, lse f32)."""
    torch = _torch()
    B, Hq, Hkv, N, _, d = _qkv(q, k, v, square=True)
    o = _out(o, (B, Hq, N, d), torch.float32, "o", q, stream)
    lse = _out(lse, (B, Hq, N), torch.float32, "lse", q, stream)
    rc = lib().attn_fwd(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), _scale(scale, d),
                        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream))
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


_KV_FORMS = ("attn_bwd_kv", "attn_bwd_rope", "attn_bwd_ex")


def _bwd_call(fn, q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv, workspace, stream,
              base=None):
    torch = _torch()
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v, square=fn not in _KV_FORMS)
    _expect(dout, (B, Hq, Nq, d), q.dtype, "dout", q)
    if fn == "attn_bwd_ex":
        _dev(o, "o")
        _dtype_code(o)
        _expect(o, (B, Hq, Nq, d), None, "o", q)
    else:
        _expect(o, (B, Hq, Nq, d), torch.float32, "o (the float32 output of the forward)", q)
    _expect(lse, (B, Hq, Nq), torch.float32, "lse", q)
    scale = _scale(scale, d)
    code = _dtype_code(q)
    dq = _out(dq, (B, Hq, Nq, d), torch.float32, "dq", q, stream)
    dk = _out(dk, (B, Hkv, Nk, d), torch.float32, "dk", q, stream)
    dv = _out(dv, (B, Hkv, Nk, d), torch.float32, "dv", q, stream)
    nbytes = attn_bwd_workspace_bytes(code, B, Hq, Hkv, Nq, d)
    if workspace is None:
        workspace = _out(None, (max(nbytes, 256),), torch.uint8, "workspace", q, stream)
    else:
        _dev(workspace, "workspace")
    if dlse is not None:
        dlse_p = _ptr(_expect(dlse, (B, Hq, Nq), torch.float32, "dlse", q))
    elif fn == "attn_bwd_dlse":
        raise ValueError("attn_bwd_dlse needs dlse")
    else:
        dlse_p = None
    head = ((code, _dtype_code(o)) if fn == "attn_bwd_ex" else (code,)) + (B, Hq, Hkv) + \
        ((Nq, Nk) if fn in _KV_FORMS else (Nq,)) + \
        (d, int(bool(causal)), scale) + ((float(base),) if fn == "attn_bwd_rope" else ()) + \
        (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout))
    tail = (_ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    rc = getattr(lib(), fn)(*head, *((dlse_p,) if fn != "attn_bwd" else ()), *tail)
    _check(fn, rc)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
                     dq=None, dk=None, dv=None, stream=None):
    """attn_bwd without a workspace: the row terms live in the library's own device array
    (B*Hq*N <= 2^20; calls that overlap on one device race).  Pass dq, dk, dv to keep the
    call free of allocations."""
    torch = _torch()
    B, Hq, Hkv, N, _, d = _qkv(q, k, v, square=True)
    _expect(dout, (B, Hq, N, d), q.dtype, "dout", q)
    _expect(o, (B, Hq, N, d), torch.float32, "o (the float32 output of the forward)", q)
    _expect(lse, (B, Hq, N), torch.float32, "lse", q)
    dq = _out(dq, (B, Hq, N, d), torch.float32, "dq", q, stream)
    dk = _out(dk, (B, Hkv, N, d), torch.float32, "dk", q, stream)
    dv = _out(dv, (B, Hkv, N, d), torch.float32, "dv", q, stream)
    rc = lib().attn_bwd_noalloc(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)),
                                _scale(scale, d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream))
    _check("attn_bwd_noalloc", rc)
    return dq, dk, dv


def attn_bwd_preprocess(o, dout, delta=None, stream=None):
    """Stage 1 of the backward: delta [B,Hq,N] f32 = rowwise dout . o."""
    torch = _torch()
    _dev(dout, "dout")
    if dout.dim() != 4:
        raise ValueError("dout must be [B, Hq, N, d]")
    B, Hq, N, d = dout.shape
    _expect(o, (B, Hq, N, d), torch.float32, "o", dout)
    delta = _out(delta, (B, Hq, N), torch.float32, "delta", dout, stream)
    rc = lib().attn_bwd_preprocess(_dtype_code(dout), B, Hq, N, d, _ptr(o), _ptr(dout),
                                   _ptr(delta), _stream(stream))
    _check("attn_bwd_preprocess", rc)
    return delta


def _stage_inputs(q, k, v, lse, dout, delta):
    torch = _torch()
    B, Hq, Hkv, N, _, d = _qkv(q, k, v, square=True)
    _expect(lse, (B, Hq, N), torch.float32, "lse", q)
    _expect(dout, (B, Hq, N, d), q.dtype, "dout", q)
    _expect(delta, (B, Hq, N), torch.float32, "delta", q)
    return B, Hq, Hkv, N, d


def attn_bwd_dkdv(q, k, v, lse, dout, delta, causal=True, scale=None, dk=None, dv=None,
                  stream=None):
    """Stage 2 of the backward: (dk, dv) f32."""
    torch = _torch()
    B, Hq, Hkv, N, d = _stage_inputs(q, k, v, lse, dout, delta)
    dk = _out(dk, (B, Hkv, N, d), torch.float32, "dk", q, stream)
    dv = _out(dv, (B, Hkv, N, d), torch.float32, "dv", q, stream)
    rc = lib().attn_bwd_dkdv(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), _scale(scale, d),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                             _ptr(dk), _ptr(dv), _stream(stream))
    _check("attn_bwd_dkdv", rc)
    return dk, dv


def attn_bwd_dq(q, k, v, lse, dout, delta, causal=True, scale=None, dq=None, stream=None):
    """Stage 3 of the backward: dq f32."""
    torch = _torch()
    B, Hq, Hkv, N, d = _stage_inputs(q, k, v, lse, dout, delta)
    dq = _out(dq, (B, Hq, N, d), torch.float32, "dq", q, stream)
    rc = lib().attn_bwd_dq(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), _scale(scale, d),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                           _ptr(dq), _stream(stream))
    _check("attn_bwd_dq", rc)
    return dq


def attn_bwd_grads(q, k, v, lse, dout, delta, causal=True, scale=None, dq=None, dk=None, dv=None,
                   stream=None):
    """Stages 2 and 3 of the backward as attn_bwd runs them: (dq, dk, dv) f32."""
    torch = _torch()
    B, Hq, Hkv, N, d = _stage_inputs(q, k, v, lse, dout, delta)
    dq = _out(dq, (B, Hq, N, d), torch.float32, "dq", q, stream)
    dk = _out(dk, (B, Hkv, N, d), torch.float32, "dk", q, stream)
    dv = _out(dv, (B, Hkv, N, d), torch.float32, "dv", q, stream)
    rc = lib().attn_bwd_grads(_dtype_code(q), B, Hq, Hkv, N, d, int(bool(causal)), _scale(scale, d),
                              _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                              _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream))
    _check("attn_bwd_grads", rc)
    return dq, dk, dv


def attn_fwd_kv(q, k, v, causal: bool = True, scale: float | None = None, o=None, lse=None,
                stream=None):
    """Forward of q [B,Hq,Nq,d] against k, v [B,Hkv,Nk,d] (Nk >= Nq, queries at the last Nq
    positions) -> (o [B,Hq,Nq,d] f32, lse [B,Hq,Nq] f32)."""
    torch = _torch()
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v, square=False)
    o = _out(o, (B, Hq, Nq, d), torch.float32, "o", q, stream)
    lse = _out(lse, (B, Hq, Nq), torch.float32, "lse", q, stream)
    rc = lib().attn_fwd_kv(_dtype_code(q), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                           _scale(scale, d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                           _stream(stream))
    _check("attn_fwd_kv", rc)
    return o, lse


def attn_fwd_ex(q, k, v, causal: bool = True, scale: float | None = None, o_dtype=None, o=None,
                lse=None, stream=None):
    """The general forward: q [B,Hq,Nq,d] against k, v [B,Hkv,Nk,d] (Nk >= Nq), o in o_dtype
    (torch.float32, the default, or torch.bfloat16).  Returns (o, lse)."""
    torch = _torch()
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v, square=False)
    if o is not None and o_dtype is None:
        o_dtype = o.dtype
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if o_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"unsupported output dtype {o_dtype}; use float32 or bfloat16")
    o = _out(o, (B, Hq, Nq, d), o_dtype, "o", q, stream)
    lse = _out(lse, (B, Hq, Nq), torch.float32, "lse", q, stream)
    rc = lib().attn_fwd_ex(_dtype_code(q), _dtype_code(o), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                           _scale(scale, d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                           _stream(stream))
    _check("attn_fwd_ex", rc)
    return o, lse


def attn_bwd_ex(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None, dq=None,
                dk=None, dv=None, workspace=None, stream=None, dlse=None):
    """The general backward: o from attn_fwd_ex in either dtype, dlse optional."""
    return _bwd_call("attn_bwd_ex", q, k, v, o, lse, dout, dlse, causal, scale, dq, dk, dv,
                     workspace, stream)


def attn_bwd_bf16grad_workspace_bytes(dtype_code: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                                      d: int) -> int:
    return int(lib().attn_bwd_bf16grad_workspace_bytes(int(dtype_code), B, Hq, Hkv, Nq, Nk, d))


def attn_bwd_bf16grad(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
                      dq=None, dk=None, dv=None, workspace=None, stream=None, dlse=None):
    """attn_bwd_ex with the gradients in bfloat16 (each the float32 gradient rounded to
    nearest even).  Returns (dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d]), all bfloat16."""
    torch = _torch()
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v, square=False)
    _expect(dout, (B, Hq, Nq, d), q.dtype, "dout", q)
    _dev(o, "o")
    _expect(o, (B, Hq, Nq, d), None, "o", q)
    _expect(lse, (B, Hq, Nq), torch.float32, "lse", q)
    scale = _scale(scale, d)
    code = _dtype_code(q)
    dq = _out(dq, (B, Hq, Nq, d), torch.bfloat16, "dq", q, stream)
    dk = _out(dk, (B, Hkv, Nk, d), torch.bfloat16, "dk", q, stream)
    dv = _out(dv, (B, Hkv, Nk, d), torch.bfloat16, "dv", q, stream)
    dlse_p = None if dlse is None else _ptr(_expect(dlse, (B, Hq, Nq), torch.float32, "dlse", q))
    nbytes = attn_bwd_bf16grad_workspace_bytes(code, B, Hq, Hkv, Nq, Nk, d)
    if workspace is None:
        workspace = _out(None, (max(nbytes, 256),), torch.uint8, "workspace", q, stream)
    else:
        _dev(workspace, "workspace")
    rc = lib().attn_bwd_bf16grad(code, _dtype_code(o), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), dlse_p,
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_bwd_bf16grad", rc)
    return dq, dk, dv


def attn_rope(x, pos0: int, base: float, inverse: bool = False, y=None, stream=None):
    """Rotary positions on x [B,H,N,d] (row n at position pos0 + n) into y (default: a new
    tensor; y may be x).  inverse: the transposed rotation."""
    _dev(x, "x")
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    y = _out(y, tuple(x.shape), x.dtype, "y", x, stream)
    rc = lib().attn_rope(_dtype_code(x), B, H, N, d, int(pos0), float(base), int(bool(inverse)),
                         _ptr(x), _ptr(y), _stream(stream))
    _check("attn_rope", rc)
    return y


def attn_fwd_rope(q, k, v, causal: bool = True, scale: float | None = None, base: float = 10000.0,
                  q_rot=None, k_rot=None, o=None, lse=None, stream=None):
    """Forward over rotated q (row i at position Nk - Nq + i) and k (row j at j).
    Returns (o, lse, q_rot, k_rot); attn_bwd_rope takes q_rot and k_rot."""
    torch = _torch()
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v, square=False)
    q_rot = _out(q_rot, tuple(q.shape), q.dtype, "q_rot", q, stream)
    k_rot = _out(k_rot, tuple(k.shape), k.dtype, "k_rot", q, stream)
    o = _out(o, (B, Hq, Nq, d), torch.float32, "o", q, stream)
    lse = _out(lse, (B, Hq, Nq), torch.float32, "lse", q, stream)
    rc = lib().attn_fwd_rope(_dtype_code(q), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                             _scale(scale, d), float(base), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(q_rot), _ptr(k_rot), _ptr(o), _ptr(lse), _stream(stream))
    _check("attn_fwd_rope", rc)
    return o, lse, q_rot, k_rot


def attn_bwd_rope(q_rot, k_rot, v, o, lse, dout, causal: bool = True, scale: float | None = None,
                  base: float = 10000.0, dq=None, dk=None, dv=None, workspace=None, stream=None,
                  dlse=None):
    """Backward of attn_fwd_rope: (dq, dk, dv) with respect to the unrotated q, k and v."""
    return _bwd_call("attn_bwd_rope", q_rot, k_rot, v, o, lse, dout, dlse, causal, scale, dq, dk,
                     dv, workspace, stream, base=base)


def attn_bwd_grads_plan(dtype_code: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                        causal: bool, scale: float):
    """(one_kernel, groups, blocks): whether attn_bwd_grads (and the gradient part of attn_bwd /
    attn_bwd_kv) runs as one kernel for this shape, and its plan's block groups and grid size."""
    g, b = ctypes.c_int(0), ctypes.c_int(0)
    one = lib().attn_bwd_grads_plan(int(dtype_code), int(B), int(Hq), int(Hkv), int(Nq), int(Nk),
                                    int(d), int(bool(causal)), float(scale), ctypes.byref(g),
                                    ctypes.byref(b))
    return bool(one), int(g.value), int(b.value)


def _decode_inputs(q, k_cache, v_cache, cache_name="caches"):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, Hkv, L, d]")
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _dtype_code(q)
    _expect(k_cache, (B, Hkv, L, d), q.dtype, "k_cache", q)
    _expect(v_cache, (B, Hkv, L, d), q.dtype, "v_cache", q)
    return B, Hq, Hkv, L, d


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, n_splits: int,
                       scale: float | None = None, part_o=None, part_lse=None, o=None, lse=None,
                       stream=None):
    """One decode step with cache append.  q [B,Hq,d], k_new/v_new [B,Hkv,d], caches
    [B,Hkv,L_cap,d] (row seq_lens[b] is written), seq_lens int32 [B] on the device
    -> (o [B,Hq,d], lse [B,Hq]) f32."""
    torch = _torch()
    B, Hq, Hkv, L_cap, d = _decode_inputs(q, k_cache, v_cache)
    _expect(k_new, (B, Hkv, d), q.dtype, "k_new", q)
    _expect(v_new, (B, Hkv, d), q.dtype, "v_new", q)
    _expect(seq_lens, (B,), torch.int32, "seq_lens", q)
    S = int(n_splits)
    part_o = _out(part_o, (B, Hq, S, d), torch.float32, "part_o", q, stream)
    part_lse = _out(part_lse, (B, Hq, S), torch.float32, "part_lse", q, stream)
    o = _out(o, (B, Hq, d), torch.float32, "o", q, stream)
    lse = _out(lse, (B, Hq), torch.float32, "lse", q, stream)
    rc = lib().attn_decode_append(_dtype_code(q), B, Hq, Hkv, L_cap, d, _scale(scale, d), S,
                                  _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(seq_lens), _ptr(part_o), _ptr(part_lse),
                                  _ptr(o), _ptr(lse), _stream(stream))
    _check("attn_decode_append", rc)
    return o, lse


def attn_decode(q, k_cache, v_cache, n_splits: int, scale: float | None = None,
                part_o=None, part_lse=None, stream=None):
    """Split-KV decode.  q [B,Hq,d], caches [B,Hkv,L,d] -> (part_o [B,Hq,S,d], part_lse [B,Hq,S])."""
    torch = _torch()
    B, Hq, Hkv, L, d = _decode_inputs(q, k_cache, v_cache)
    S = int(n_splits)
    part_o = _out(part_o, (B, Hq, S, d), torch.float32, "part_o", q, stream)
    part_lse = _out(part_lse, (B, Hq, S), torch.float32, "part_lse", q, stream)
    rc = lib().attn_decode(_dtype_code(q), B, Hq, Hkv, L, d, _scale(scale, d), S,
                           _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(part_o), _ptr(part_lse),
                           _stream(stream))
    _check("attn_decode", rc)
    return part_o, part_lse


def attn_decode_merged(q, k_cache, v_cache, n_splits: int, scale: float | None = None,
                       part_o=None, part_lse=None, o=None, lse=None, stream=None):
    """Split-KV decode and the LSE merge in one call.

    Returns (o [B,Hq,d], lse [B,Hq], part_o, part_lse).
    """
    torch = _torch()
    B, Hq, Hkv, L, d = _decode_inputs(q, k_cache, v_cache)
    S = int(n_splits)
    part_o = _out(part_o, (B, Hq, S, d), torch.float32, "part_o", q, stream)
    part_lse = _out(part_lse, (B, Hq, S), torch.float32, "part_lse", q, stream)
    o = _out(o, (B, Hq, d), torch.float32, "o", q, stream)
    lse = _out(lse, (B, Hq), torch.float32, "lse", q, stream)
    rc = lib().attn_decode_merged(_dtype_code(q), B, Hq, Hkv, L, d, _scale(scale, d), S,
                                  _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(part_o),
                                  _ptr(part_lse), _ptr(o), _ptr(lse), _stream(stream))
    _check("attn_decode_merged", rc)
    return o, lse, part_o, part_lse


def attn_lse_merge(part_o, part_lse, o=None, lse=None, stream=None):
    """Merge split partials: part_o [B,Hq,S,d], part_lse [B,Hq,S] -> (o [B,Hq,d], lse [B,Hq])."""
    torch = _torch()
    _dev(part_o, "part_o")
    if part_o.dim() != 4:
        raise ValueError("part_o must be [B, Hq, S, d]")
    B, Hq, S, d = part_o.shape
    _expect(part_o, (B, Hq, S, d), torch.float32, "part_o")
    _expect(part_lse, (B, Hq, S), torch.float32, "part_lse", part_o)
    o = _out(o, (B, Hq, d), torch.float32, "o", part_o, stream)
    lse = _out(lse, (B, Hq), torch.float32, "lse", part_o, stream)
    rc = lib().attn_lse_merge(B, Hq, S, d, _ptr(part_o), _ptr(part_lse), _ptr(o), _ptr(lse),
                              _stream(stream))
    _check("attn_lse_merge", rc)
    return o, lse


def attn_read_probe(src, out=None, stream=None):
    """Read every byte of the contiguous device tensor src once (a bandwidth reference for
    decode); out: a device int32 tensor of one element (written only on a sentinel match)."""
    torch = _torch()
    _dev(src, "src")
    out = _out(out, (1,), torch.int32, "out", src, stream)
    nbytes = src.numel() * src.element_size()
    rc = lib().attn_read_probe(_ptr(src), nbytes, _ptr(out), _stream(stream))
    _check("attn_read_probe", rc)
    return out


def _strided(t, shape, dtype, name, like):
    """A device tensor of this shape and dtype whose last dim is contiguous (any other
    strides); returns its AttnLayout."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, got {t.device}")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous last (head) dimension")
    return AttnLayout(t.stride(0), t.stride(1), t.stride(2))


def attn_fwd_strided(q, k, v, causal: bool = True, scale: float | None = None, o_dtype=None, o=None,
                     lse=None, stream=None):
    """attn_fwd_ex over views of any strides: q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] and o may be
    strided views (e.g. x.view(B, N, H, d).transpose(1, 2) of a [B, N, H, d] tensor) whose
    head dim is contiguous.  A new o is contiguous.  Returns (o, lse)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    lq = _strided(q, (B, Hq, Nq, d), q.dtype, "q", q)
    lk = _strided(k, (B, Hkv, Nk, d), q.dtype, "k", q)
    lv = _strided(v, (B, Hkv, Nk, d), q.dtype, "v", q)
    if o is None:
        o = _out(None, (B, Hq, Nq, d), o_dtype or torch.float32, "o", q, stream)
    lo = _strided(o, (B, Hq, Nq, d), None, "o", q)
    lse = _out(lse, (B, Hq, Nq), torch.float32, "lse", q, stream)
    rc = lib().attn_fwd_strided(code, _dtype_code(o), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                                _scale(scale, d), _ptr(q), ctypes.byref(lq), _ptr(k), ctypes.byref(lk),
                                _ptr(v), ctypes.byref(lv), _ptr(o), ctypes.byref(lo), _ptr(lse),
                                _stream(stream))
    _check("attn_fwd_strided", rc)
    return o, lse


def attn_bwd_strided(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
                     dq=None, dk=None, dv=None, workspace=None, stream=None, dlse=None):
    """attn_bwd_ex over views of any strides (head dim contiguous): q, k, v, o, dout and the
    outputs dq, dk, dv (new ones are contiguous).  Returns (dq, dk, dv), float32."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    lay = [_strided(q, (B, Hq, Nq, d), q.dtype, "q", q),
           _strided(k, (B, Hkv, Nk, d), q.dtype, "k", q),
           _strided(v, (B, Hkv, Nk, d), q.dtype, "v", q),
           _strided(o, (B, Hq, Nq, d), None, "o", q)]
    _dtype_code(o)
    _expect(lse, (B, Hq, Nq), torch.float32, "lse", q)
    ldo = _strided(dout, (B, Hq, Nq, d), q.dtype, "dout", q)
    dq = dq if dq is not None else _out(None, (B, Hq, Nq, d), torch.float32, "dq", q, stream)
    dk = dk if dk is not None else _out(None, (B, Hkv, Nk, d), torch.float32, "dk", q, stream)
    dv = dv if dv is not None else _out(None, (B, Hkv, Nk, d), torch.float32, "dv", q, stream)
    louts = [_strided(dq, (B, Hq, Nq, d), torch.float32, "dq", q),
             _strided(dk, (B, Hkv, Nk, d), torch.float32, "dk", q),
             _strided(dv, (B, Hkv, Nk, d), torch.float32, "dv", q)]
    if dlse is not None:
        _expect(dlse, (B, Hq, Nq), torch.float32, "dlse", q)
    nbytes = attn_bwd_workspace_bytes(code, B, Hq, Hkv, Nq, d)
    if workspace is None:
        workspace = _out(None, (max(nbytes, 256),), torch.uint8, "workspace", q, stream)
    else:
        _dev(workspace, "workspace")
    rc = lib().attn_bwd_strided(code, _dtype_code(o), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                                _scale(scale, d), _ptr(q), ctypes.byref(lay[0]), _ptr(k),
                                ctypes.byref(lay[1]), _ptr(v), ctypes.byref(lay[2]), _ptr(o),
                                ctypes.byref(lay[3]), _ptr(lse), _ptr(dout), ctypes.byref(ldo),
                                None if dlse is None else _ptr(dlse), _ptr(dq), ctypes.byref(louts[0]),
                                _ptr(dk), ctypes.byref(louts[1]), _ptr(dv), ctypes.byref(louts[2]),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check("attn_bwd_strided", rc)
    return dq, dk, dv
