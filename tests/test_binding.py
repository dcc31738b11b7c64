"""The Python binding's argument checks, on the CPU.

The binding must refuse tensors whose shapes or dtypes do not match the call
(a k of another dtype, an o or lse from another call, outputs of the wrong
size) with ValueError / TypeError before it reaches the library: the kernels
trust the sizes they are given.  Here the device check is relaxed so that CPU
tensors stand in for device tensors, and the library is replaced by a stub
that fails the test if any call gets through.
"""
import pytest
import torch

import attention_causal_gqa_flash_amd as attn


class _NoLib:
    def __getattr__(self, name):
        raise AssertionError(f"the binding reached the library ({name}) with invalid arguments")


@pytest.fixture(autouse=True)
def cpu_stand_in(monkeypatch):
    def dev(t, name):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t
    monkeypatch.setattr(attn, "_dev", dev)
    monkeypatch.setattr(attn, "lib", lambda: _NoLib())
    monkeypatch.setattr(attn, "attn_bwd_workspace_bytes", lambda *a: 1024)
    monkeypatch.setattr(attn, "attn_bwd_bf16grad_workspace_bytes", lambda *a: 1024)


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


B, Hq, Hkv, N, d = 1, 4, 2, 16, 64


def _bwd_args(**over):
    a = dict(q=_t(B, Hq, N, d), k=_t(B, Hkv, N, d), v=_t(B, Hkv, N, d),
             o=_t(B, Hq, N, d, dtype=torch.float32), lse=_t(B, Hq, N, dtype=torch.float32),
             dout=_t(B, Hq, N, d))
    a.update(over)
    return a


@pytest.mark.parametrize("bad", [
    dict(k=_t(B, Hkv, N, d, dtype=torch.float32)),          # k in another dtype than q
    dict(v=_t(B, Hkv, N, d, dtype=torch.float32)),
    dict(v=_t(B, Hkv, N + 1, d)),                            # v not k's shape
    dict(k=_t(B + 1, Hkv, N, d), v=_t(B + 1, Hkv, N, d)),    # another batch
    dict(k=_t(B, Hkv, N, 32), v=_t(B, Hkv, N, 32)),          # another head dim
    dict(o=_t(B, Hq, N + 1, d, dtype=torch.float32)),        # o from another call
    dict(o=_t(B, Hq, N, d)),                                 # o not float32
    dict(lse=_t(B, Hq, N + 1, dtype=torch.float32)),         # lse from another call
    dict(lse=_t(B, Hq, N)),
    dict(dout=_t(B, Hq, N, d, dtype=torch.float32)),
    dict(dout=_t(B, Hq, N - 1, d)),
])
def test_bwd_refuses_mismatched_inputs(bad):
    with pytest.raises((ValueError, TypeError)):
        attn.attn_bwd(**_bwd_args(**bad))


@pytest.mark.parametrize("name,shape,dtype", [
    ("dq", (B, Hq, N, d + 1), torch.float32), ("dk", (B, Hkv + 1, N, d), torch.float32),
    ("dv", (B, Hkv, N, d), torch.bfloat16),
])
def test_bwd_refuses_wrong_outputs(name, shape, dtype):
    with pytest.raises(ValueError):
        attn.attn_bwd(**_bwd_args(), **{name: torch.zeros(shape, dtype=dtype)})


@pytest.mark.parametrize("bad", [
    dict(k=_t(B, Hkv, N, d, dtype=torch.float32)),
    dict(o=_t(B, Hq, N + 1, d, dtype=torch.float32)),        # o from another call
    dict(lse=_t(B, Hq, N)),
    dict(dout=_t(B, Hq, N - 1, d)),
    dict(dq=torch.zeros((B, Hq, N, d), dtype=torch.float32)),  # the gradients are bf16
    dict(dk=torch.zeros((B, Hkv + 1, N, d), dtype=torch.bfloat16)),
    dict(dlse=_t(B, Hq, N + 3, dtype=torch.float32)),
])
def test_bf16grad_refuses_mismatched_arguments(bad):
    with pytest.raises((ValueError, TypeError)):
        attn.attn_bwd_bf16grad(**_bwd_args(**bad))


def test_bwd_kv_forms_check_the_cross_length_shapes():
    a = _bwd_args(k=_t(B, Hkv, 2 * N, d), v=_t(B, Hkv, 2 * N, d))
    with pytest.raises(ValueError):
        attn.attn_bwd(**a)                                   # the square form refuses Nk != Nq
    with pytest.raises(ValueError):
        attn.attn_bwd_kv(**dict(a, lse=_t(B, Hq, 2 * N, dtype=torch.float32)))
    with pytest.raises(ValueError):
        attn.attn_bwd_kv(**a, dlse=_t(B, Hq, N + 3, dtype=torch.float32))


@pytest.mark.parametrize("bad", [
    dict(k=_t(B, Hkv, N, d, dtype=torch.float32)),
    dict(v=_t(B, Hkv, N, 32)),
    dict(o=_t(B, Hq, N, d, dtype=torch.float32)[:, :, :8]),
    dict(lse=_t(B, Hq, 2 * N, dtype=torch.float32)),
])
def test_fwd_refuses_mismatched_arguments(bad):
    a = dict(q=_t(B, Hq, N, d), k=_t(B, Hkv, N, d), v=_t(B, Hkv, N, d))
    a.update(bad)
    with pytest.raises(ValueError):
        attn.attn_fwd(**a)


def test_stage_and_decode_checks():
    q, k, v = _t(B, Hq, N, d), _t(B, Hkv, N, d), _t(B, Hkv, N, d)
    lse, delta = _t(B, Hq, N, dtype=torch.float32), _t(B, Hq, N, dtype=torch.float32)
    with pytest.raises(ValueError):
        attn.attn_bwd_dkdv(q, k, v, lse, _t(B, Hq, N, d), _t(B, Hq, N + 1, dtype=torch.float32))
    with pytest.raises(ValueError):
        attn.attn_bwd_dq(q, k, v, lse[:, :, :4].contiguous(), _t(B, Hq, N, d), delta)
    with pytest.raises(ValueError):
        attn.attn_bwd_grads(q, k, v, lse, _t(B, Hq, N, d), delta, dk=_t(B, Hkv, N, d))
    with pytest.raises(ValueError):
        attn.attn_bwd_preprocess(_t(B, Hq, N, d, dtype=torch.float32), _t(B, Hq, N + 1, d))
    qd, kc = _t(B, Hq, d), _t(B, Hkv, 100, d)
    with pytest.raises(ValueError):
        attn.attn_decode(qd, kc, _t(B, Hkv, 99, d), 4)
    with pytest.raises(ValueError):
        attn.attn_decode(qd, kc, kc, 4, part_o=_t(B, Hq, 5, d, dtype=torch.float32))
    with pytest.raises(ValueError):
        attn.attn_lse_merge(_t(B, Hq, 4, d, dtype=torch.float32), _t(B, Hq, 5, dtype=torch.float32))
    with pytest.raises(ValueError):
        attn.attn_decode_append(qd, _t(B, Hkv, d), _t(B, Hkv, d), kc, kc,
                                torch.zeros(B, dtype=torch.int64), 4)
