"""Pins for the CPU f64 oracle (no GPU).

The oracle is the reference every GPU result is compared with, so it is itself
checked here against things other than itself: values the pages print, hand
worked examples, closed forms, an independent textbook computation with numpy,
invariants of softmax attention, central finite differences and dual numbers.
Each check is chosen so that a plausible slip in the oracle (a dropped scale, a
wrong sign, an off-by-one mask, a transposed operand, a wrong head map) fails
at least one of them; ``test_oracle_mutants.py`` plants such slips and checks
that they are caught.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, Hq, Hkv, N, d, seed=0, Nk=None):
    Nk = N if Nk is None else Nk
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    do = rng.standard_normal((B, Hq, N, d))
    return q, k, v, do


def _textbook(q, k, v, causal, scale):
    """softmax(scale Q K^T + mask) V with numpy, one head at a time (G = 1)."""
    B, H, N, d = q.shape
    Nk = k.shape[2]
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if causal:
                mask = np.arange(Nk)[None, :] > np.arange(N)[:, None] + (Nk - N)
                s = np.where(mask, -np.inf, s)
            lse[b, h] = logsumexp(s, axis=1)
            p = np.exp(s - lse[b, h][:, None])
            o[b, h] = p @ v[b, h]
    return o, lse


# --------------------------------------------------------------------------
# values printed on the pages, and hand-worked examples
# --------------------------------------------------------------------------

def test_dual_xsinx_golden():
    rows = np.loadtxt(os.path.join(GOLDEN, "dual_xsinx.txt"))
    for x, val, der in rows:
        got_v, got_d = oracle.dual_xsinx(x)
        assert got_v == pytest.approx(val, abs=1e-15)
        assert got_d == pytest.approx(der, abs=1e-15)


def test_dual_xsinx_closed_form():
    for x in np.linspace(-4, 4, 33):
        v, d = oracle.dual_xsinx(x)
        assert v == pytest.approx(x * math.sin(x), abs=1e-15)
        assert d == pytest.approx(math.sin(x) + x * math.cos(x), abs=1e-14)


def _golden_worked():
    vals = {}
    with open(os.path.join(GOLDEN, "two_key_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *nums = line.split()
            vals[name] = np.array([float(x) for x in nums])
    return vals


def test_two_key_worked_example():
    g = _golden_worked()
    q = g["q"].reshape(1, 1, 2, 1)
    k = g["k"].reshape(1, 1, 2, 1)
    v = g["v"].reshape(1, 1, 2, 1)
    o, lse = oracle.attn_fwd(q, k, v, True, 1.0)
    np.testing.assert_allclose(o.ravel(), g["o"], atol=1e-14)
    np.testing.assert_allclose(lse.ravel(), g["lse"], atol=1e-14)
    dq, dk, dv = oracle.attn_bwd(q, k, v, g["dout"].reshape(1, 1, 2, 1), True, 1.0)
    np.testing.assert_allclose(dq.ravel(), g["dq"], atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), g["dk"], atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), g["dv"], atol=1e-14)


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_softmax_rows_sum_to_one(causal):
    # With d = Nk and V = identity, O row i is the probability row P_i itself.
    N = 24
    q = _rand((1, 2, N, N), 1)
    k = _rand((1, 1, N, N), 2)
    v = np.eye(N).reshape(1, 1, N, N)
    o, _ = oracle.attn_fwd(q, k, v, causal, 0.7)
    P = o[0]
    np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-14)
    assert (P >= 0).all()
    if causal:
        upper = np.triu(np.ones((N, N), bool), k=1)
        assert (P[:, upper] == 0).all()
        assert (P[:, ~upper] > 0).all()


def test_causal_row0_closed_form():
    q, k, v, _ = _qkv(2, 4, 2, 16, 8, seed=3)
    scale = 0.3
    o, lse = oracle.attn_fwd(q, k, v, True, scale)
    for h in range(4):
        g = h // 2
        np.testing.assert_array_equal(o[:, h, 0], v[:, g, 0])
        np.testing.assert_allclose(lse[:, h, 0], scale * np.einsum("bc,bc->b", q[:, h, 0], k[:, g, 0]),
                                   rtol=1e-15, atol=1e-15)


def test_constant_keys_closed_form():
    N, d, scale = 20, 6, 0.45
    q, _, v, _ = _qkv(1, 2, 1, N, d, seed=4)
    kvec = _rand((d,), 5)
    k = np.broadcast_to(kvec, (1, 1, N, d)).copy()
    o, lse = oracle.attn_fwd(q, k, v, True, scale)
    for i in range(N):
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(v[0, 0, : i + 1].mean(axis=0), (2, d)),
                                   rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], scale * q[0, :, i] @ kvec + math.log(i + 1),
                                   rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 4), (2, 3, 3, 17, 8), (1, 2, 2, 33, 16)])
def test_matches_numpy_textbook(causal, shape):
    B, Hq, Hkv, N, d = shape
    q, k, v, _ = _qkv(B, Hq, Hkv, N, d, seed=6)
    o, lse = oracle.attn_fwd(q, k, v, causal, 1.0 / math.sqrt(d))
    ot, lt = _textbook(q, k, v, causal, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(o, ot, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lt, rtol=1e-12, atol=1e-13)


def test_cross_length_bottom_right_mask():
    # Nq < Nk: query i sits at absolute position i + (Nk - Nq).
    q, k, v, _ = _qkv(1, 1, 1, 5, 4, seed=7, Nk=9)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.5)
    ot, lt = _textbook(q, k, v, True, 0.5)
    np.testing.assert_allclose(o, ot, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lt, rtol=1e-12, atol=1e-13)
    # the last query sees every key: equals the non-causal result
    on, ln = oracle.attn_fwd(q[:, :, -1:], k, v, False, 0.5)
    np.testing.assert_allclose(o[:, :, -1], on[:, :, 0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("G", [1, 2, 3, 4])
def test_gqa_equals_mha_with_repeated_kv(G):
    Hkv = 2
    q, k, v, _ = _qkv(2, Hkv * G, Hkv, 19, 8, seed=8)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.35)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    om, lm = oracle.attn_fwd(q, kr, vr, True, 0.35)
    np.testing.assert_array_equal(o, om)
    np.testing.assert_array_equal(lse, lm)
    # and the group map is contiguous: head h reads kv head h // G
    ot, lt = _textbook(q, kr, vr, True, 0.35)
    np.testing.assert_allclose(o, ot, rtol=1e-12, atol=1e-13)


def test_prefix_invariance():
    q, k, v, _ = _qkv(1, 2, 1, 64, 8, seed=9)
    o64, l64 = oracle.attn_fwd(q, k, v, True, 0.4)
    o32, l32 = oracle.attn_fwd(q[:, :, :32], k[:, :, :32], v[:, :, :32], True, 0.4)
    np.testing.assert_array_equal(o64[:, :, :32], o32)
    np.testing.assert_array_equal(l64[:, :, :32], l32)


def test_key_shift_invariance():
    q, k, v, _ = _qkv(1, 2, 1, 21, 8, seed=10)
    c = _rand((8,), 11)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.4)
    o2, lse2 = oracle.attn_fwd(q, k + c, v, True, 0.4)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 0.4 * np.einsum("bhnc,c->bhn", q, c), rtol=1e-11, atol=1e-11)


def test_value_linearity():
    q, k, v, _ = _qkv(1, 2, 1, 13, 4, seed=12)
    v2 = _rand(v.shape, 13)
    o1, _ = oracle.attn_fwd(q, k, v, True, 0.5)
    o2, _ = oracle.attn_fwd(q, k, v2, True, 0.5)
    o3, _ = oracle.attn_fwd(q, k, 2.0 * v - 3.0 * v2, True, 0.5)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.attn_fwd(q, k, v, causal, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 3), (1, 2, 2, 6, 4), (2, 3, 1, 4, 2)])
def test_bwd_central_finite_differences(causal, shape):
    B, Hq, Hkv, N, d = shape
    q, k, v, do = _qkv(B, Hq, Hkv, N, d, seed=14)
    scale = 0.6
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, causal, scale)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - g)) / max(1.0, np.max(np.abs(g)))
        assert err <= 1e-7, (name, err)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 1, 7, 4), (2, 4, 2, 11, 8), (1, 3, 1, 16, 16)])
def test_bwd_dual_numbers(causal, shape):
    B, Hq, Hkv, N, d = shape
    q, k, v, do = _qkv(B, Hq, Hkv, N, d, seed=15)
    tq, tk, tv = _rand(q.shape, 16), _rand(k.shape, 17), _rand(v.shape, 18)
    scale = 0.37
    o, to, lse, tlse = oracle.attn_fwd_dual(q, tq, k, tk, v, tv, causal, scale)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-14)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale)
    directional = float(np.sum(do * to))
    inner = float(np.sum(dq * tq) + np.sum(dk * tk) + np.sum(dv * tv))
    assert abs(directional - inner) <= 1e-12 * max(1.0, abs(directional))


def test_bwd_invariants():
    B, Hq, Hkv, N, d = 2, 6, 2, 23, 8
    q, k, v, do = _qkv(B, Hq, Hkv, N, d, seed=19)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True, 0.3)
    G = Hq // Hkv
    # causal row 0 has a single visible key: its dq is exactly zero
    assert np.all(dq[:, :, 0] == 0.0)
    # shift invariance in the keys: sum_j dk_j = 0 per kv head
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # rows of P sum to one: sum_j dv_j = sum over the group and rows of dO
    for g in range(Hkv):
        np.testing.assert_allclose(dv[:, g].sum(axis=1), do[:, g * G:(g + 1) * G].sum(axis=(1, 2)),
                                   rtol=1e-12, atol=1e-12)


def test_bwd_gqa_is_group_sum_of_mha():
    B, Hkv, G, N, d = 1, 2, 3, 12, 4
    q, k, v, do = _qkv(B, Hkv * G, Hkv, N, d, seed=20)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True, 0.5)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dqm, dkm, dvm = oracle.attn_bwd(q, kr, vr, do, True, 0.5)
    np.testing.assert_allclose(dq, dqm, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, dkm.reshape(B, Hkv, G, N, d).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dvm.reshape(B, Hkv, G, N, d).sum(axis=2), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk,causal", [(3, 7, True), (2, 5, False), (1, 6, True)])
def test_bwd_cross_length_finite_differences(Nq, Nk, causal):
    """Nq queries at the last Nq of Nk key positions: central differences of <o, dO>."""
    B, Hq, Hkv, d = 1, 2, 1, 3
    q, k, v, do = _qkv(B, Hq, Hkv, Nq, d, seed=50 + Nq + Nk, Nk=Nk)
    scale = 0.8
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = {"q": q, "k": k, "v": v}
            a[name] = xp
            lp = _loss(a["q"], a["k"], a["v"], do, causal, scale)
            a[name] = xm
            lm = _loss(a["q"], a["k"], a["v"], do, causal, scale)
            assert abs((lp - lm) / (2 * h) - g[idx]) <= 2e-6, (name, idx)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_cross_length_is_square_with_silent_prefix(causal):
    """The chunk's gradients equal those of the square problem over all Nk positions whose
    first Nk - Nq query rows (any values) receive dO = 0: those rows add nothing."""
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 5, 12, 6
    q, k, v, do = _qkv(B, Hq, Hkv, Nq, d, seed=60, Nk=Nk)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, 0.4)
    pre = _rand((B, Hq, Nk - Nq, d), 61)
    qf = np.concatenate([pre, q], axis=2)
    dof = np.concatenate([np.zeros_like(pre), do], axis=2)
    dqf, dkf, dvf = oracle.attn_bwd(qf, k, v, dof, causal, 0.4)
    np.testing.assert_allclose(dq, dqf[:, :, Nk - Nq:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, dkf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dvf, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# rotary positions
# --------------------------------------------------------------------------

def _rope_complex(x, pos0, base):
    """The rotation as complex multiplication: pair (x_i, x_{i+d/2}) is z = x_i + 1j x_{i+d/2},
    turned by exp(1j p base^(-2i/d)) at position p."""
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    p = pos0 + np.arange(x.shape[-2])[:, None]
    w = np.exp(1j * p * np.power(float(base), -2.0 * np.arange(h) / d)[None, :])
    y = z * w
    return np.concatenate([y.real, y.imag], axis=-1)


@pytest.mark.parametrize("pos0,base,d", [(0, 10000.0, 8), (5, 10000.0, 16), (4093, 500000.0, 64),
                                         (2, 3.0, 2)])
def test_rope_is_a_complex_turn(pos0, base, d):
    x = _rand((2, 3, 7, d), 70 + d)
    np.testing.assert_allclose(oracle.rope(x, pos0, base), _rope_complex(x, pos0, base),
                               rtol=1e-12, atol=1e-12)


def test_rope_identity_at_zero_and_norms_kept():
    x = _rand((1, 2, 9, 12), 71)
    y = oracle.rope(x, 0, 10000.0)
    assert np.array_equal(y[:, :, 0], x[:, :, 0])          # position 0: no turn
    h = 6
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2,
                               rtol=1e-12)


def test_rope_scores_depend_on_position_difference():
    q, k = _rand((1, 1, 1, 16), 72), _rand((1, 1, 1, 16), 73)
    base = 10000.0
    dots = [float(np.sum(oracle.rope(q, 7 + t, base) * oracle.rope(k, 3 + t, base))) for t in (0, 1, 50, 999)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)


def test_rope_inverse_is_transpose():
    x, y = _rand((2, 2, 5, 8), 74), _rand((2, 2, 5, 8), 75)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, 11, 1e4), 11, 1e4, inverse=True), x,
                               rtol=1e-13, atol=1e-13)
    lhs = float(np.sum(oracle.rope(x, 11, 1e4) * y))
    rhs = float(np.sum(x * oracle.rope(y, 11, 1e4, inverse=True)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("Nq,Nk,causal", [(4, 4, True), (3, 6, True), (4, 5, False)])
def test_attn_rope_gradient_finite_differences(Nq, Nk, causal):
    """Attention of rotated q and k: the composite's gradient by central differences."""
    B, Hq, Hkv, d, base = 1, 2, 1, 4, 100.0
    q, k, v, do = _qkv(B, Hq, Hkv, Nq, d, seed=80 + Nq + Nk, Nk=Nk)
    dq, dk, dv = oracle.attn_bwd_rope(q, k, v, do, causal, 0.6, base)

    def loss(a):
        return float(np.sum(oracle.attn_fwd_rope(a["q"], a["k"], a["v"], causal, 0.6, base)[0] * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = {"q": q, "k": k, "v": v}
            a[name] = xp
            lp = loss(a)
            a[name] = xm
            lm = loss(a)
            assert abs((lp - lm) / (2 * h) - g[idx]) <= 2e-6, (name, idx)


# --------------------------------------------------------------------------
# backward with an upstream gradient of lse
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Nq,Nk,causal", [(4, 4, True), (3, 7, True), (5, 5, False)])
def test_bwd_dlse_finite_differences(Nq, Nk, causal):
    """d/dx of <o, dO> + <lse, dlse> by central differences equals the backward."""
    B, Hq, Hkv, d = 1, 2, 1, 3
    rng = np.random.default_rng(41 + Nq + Nk)
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    do = rng.standard_normal((B, Hq, Nq, d))
    dl = rng.standard_normal((B, Hq, Nq))
    dq, dk, dv = oracle.attn_bwd_dlse(q, k, v, do, dl, causal, 0.7)

    def loss(a):
        o, lse = oracle.attn_fwd(a["q"], a["k"], a["v"], causal, 0.7)
        return float(np.sum(o * do) + np.sum(lse * dl))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = {"q": q, "k": k, "v": v}
            a[name] = xp
            lp = loss(a)
            a[name] = xm
            lm = loss(a)
            assert abs((lp - lm) / (2 * h) - g[idx]) <= 2e-6, (name, idx)


def test_bwd_dlse_zero_equals_bwd_and_lse_only_leaves_dv_zero():
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 5
    rng = np.random.default_rng(44)
    q, k, v = rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)), \
        rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    a = oracle.attn_bwd(q, k, v, do, True, 0.5)
    b = oracle.attn_bwd_dlse(q, k, v, do, np.zeros((B, Hq, N)), True, 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # only lse has an upstream gradient: v does not reach lse
    _, _, dv = oracle.attn_bwd_dlse(q, k, v, np.zeros_like(do), rng.standard_normal((B, Hq, N)),
                                    True, 0.5)
    assert np.all(dv == 0.0)


# --------------------------------------------------------------------------
# split-KV decode, the merge and the online-softmax monoid
# --------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 7, 64, 100])
def test_decode_split_invariance(L):
    B, Hq, Hkv, d = 2, 4, 2, 8
    rng = np.random.default_rng(21)
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, Hkv, L, d))
    vc = rng.standard_normal((B, Hkv, L, d))
    # unsplit definition: the one-row forward against every cached key
    o_ref, l_ref = oracle.attn_fwd(q[:, :, None], kc, vc, False, 0.35)
    for S in sorted({1, 2, 3, 16, L, L + 3}):
        po, pl = oracle.attn_decode(q, kc, vc, 0.35, S)
        o, lse = oracle.lse_merge(po, pl)
        np.testing.assert_allclose(o, o_ref[:, :, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse, l_ref[:, :, 0], rtol=1e-13, atol=1e-14)
        C = -(-L // S)
        for s in range(S):
            if s * C >= L:            # empty chunk: the identity
                assert np.all(pl[:, :, s] == -np.inf) and np.all(po[:, :, s] == 0.0)


def test_decode_equals_last_causal_row():
    B, Hq, Hkv, L, d = 1, 4, 1, 37, 8
    rng = np.random.default_rng(22)
    Q = rng.standard_normal((B, Hq, L, d))
    kc = rng.standard_normal((B, Hkv, L, d))
    vc = rng.standard_normal((B, Hkv, L, d))
    o, lse = oracle.attn_fwd(Q, kc, vc, True, 0.4)
    po, pl = oracle.attn_decode(Q[:, :, -1], kc, vc, 0.4, 5)
    od, ld = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(od, o[:, :, -1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ld, lse[:, :, -1], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# one decode step with cache append and per-sequence lengths
# --------------------------------------------------------------------------

def _append_inputs(B, Hq, Hkv, Lcap, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, d)), rng.standard_normal((B, Hkv, d)),
            rng.standard_normal((B, Hkv, d)), rng.standard_normal((B, Hkv, Lcap, d)),
            rng.standard_normal((B, Hkv, Lcap, d)))


def test_append_first_token_closed_form():
    """n = 0: the token attends to itself only, so o = v_new and lse = scale q.k_new."""
    B, Hq, Hkv, Lcap, d = 2, 6, 3, 5, 4
    q, kn, vn, kc, vc = _append_inputs(B, Hq, Hkv, Lcap, d, 31)
    o, lse, _, _ = oracle.attn_decode_append(q, kn, vn, kc, vc, [0, 0], 0.7)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(o[b, h], vn[b, h // G], rtol=1e-15, atol=1e-15)
            assert abs(lse[b, h] - 0.7 * float(q[b, h] @ kn[b, h // G])) < 1e-14


def test_append_identical_keys_closed_form():
    """All n + 1 keys equal: uniform weights, o = mean of the values, lse = s + ln(n + 1)."""
    B, Hq, Hkv, Lcap, d, n = 1, 2, 1, 9, 3, 6
    q, kn, vn, kc, vc = _append_inputs(B, Hq, Hkv, Lcap, d, 32)
    kc[:] = kn[:, :, None, :]
    o, lse, kc2, vc2 = oracle.attn_decode_append(q, kn, vn, kc, vc, [n], 1.3)
    mean_v = (vc[0, 0, :n].sum(axis=0) + vn[0, 0]) / (n + 1)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], mean_v, rtol=1e-13, atol=1e-14)
        assert abs(lse[0, h] - (1.3 * float(q[0, h] @ kn[0, 0]) + math.log(n + 1))) < 1e-13


def test_append_equals_last_causal_row_per_sequence():
    """Sequence b with n_b cached tokens: the step's output is the last row of a
    causal forward over the n_b + 1 tokens (cache rows then the new token)."""
    B, Hq, Hkv, Lcap, d = 3, 4, 2, 12, 8
    q, kn, vn, kc, vc = _append_inputs(B, Hq, Hkv, Lcap, d, 33)
    lens = [11, 0, 5]
    o, lse, _, _ = oracle.attn_decode_append(q, kn, vn, kc, vc, lens, 0.45)
    for b, n in enumerate(lens):
        K = np.concatenate([kc[b:b + 1, :, :n], kn[b:b + 1, :, None]], axis=2)
        V = np.concatenate([vc[b:b + 1, :, :n], vn[b:b + 1, :, None]], axis=2)
        Q = np.zeros((1, Hq, n + 1, d))
        Q[0, :, n] = q[b]
        of, lf = oracle.attn_fwd(Q, K, V, True, 0.45)
        np.testing.assert_allclose(o[b], of[0, :, n], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[b], lf[0, :, n], rtol=1e-13, atol=1e-14)
        # and against numpy's own softmax, head by head
        for h in range(Hq):
            sc = 0.45 * (K[0, h // (Hq // Hkv)] @ q[b, h])
            w = np.exp(sc - logsumexp(sc))
            np.testing.assert_allclose(o[b, h], w @ V[0, h // (Hq // Hkv)], rtol=1e-12, atol=1e-13)


def test_append_writes_row_n_only_and_rows_past_n_are_ignored():
    B, Hq, Hkv, Lcap, d = 2, 2, 2, 10, 4
    q, kn, vn, kc, vc = _append_inputs(B, Hq, Hkv, Lcap, d, 34)
    lens = [3, 9]
    o, lse, kc2, vc2 = oracle.attn_decode_append(q, kn, vn, kc, vc, lens, 0.5)
    for b, n in enumerate(lens):
        exp_k, exp_v = kc[b].copy(), vc[b].copy()
        exp_k[:, n], exp_v[:, n] = kn[b], vn[b]
        assert np.array_equal(kc2[b], exp_k) and np.array_equal(vc2[b], exp_v)
    # rows past n (and the stale row n) have no influence
    kp, vp = kc.copy(), vc.copy()
    kp[0, :, 3:], vp[0, :, 3:] = np.nan, 1e300
    o2, l2, _, _ = oracle.attn_decode_append(q, kn, vn, kp, vp, lens, 0.5)
    np.testing.assert_array_equal(o2[0], o[0])
    np.testing.assert_array_equal(l2[0], lse[0])


def test_append_invalid_length_is_reported():
    B, Hq, Hkv, Lcap, d = 3, 2, 1, 6, 4
    q, kn, vn, kc, vc = _append_inputs(B, Hq, Hkv, Lcap, d, 35)
    o, lse, kc2, vc2 = oracle.attn_decode_append(q, kn, vn, kc, vc, [-1, 6, 2], 0.5)
    assert np.all(np.isnan(o[:2])) and np.all(np.isnan(lse[:2]))
    assert np.array_equal(kc2[:2], kc[:2]) and np.array_equal(vc2[:2], vc[:2])
    assert np.all(np.isfinite(o[2])) and np.all(np.isfinite(lse[2]))


def test_merge_order_independent_and_identity():
    rng = np.random.default_rng(23)
    B, Hq, S, d = 1, 3, 9, 5
    po = rng.standard_normal((B, Hq, S, d))
    pl = rng.standard_normal((B, Hq, S)) * 4
    o, lse = oracle.lse_merge(po, pl)
    for _ in range(5):
        perm = rng.permutation(S)
        o2, l2 = oracle.lse_merge(po[:, :, perm], pl[:, :, perm])
        np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(l2, lse, rtol=1e-13, atol=1e-14)
    # adding empty chunks changes nothing
    po_e = np.concatenate([po, np.zeros((B, Hq, 2, d))], axis=2)
    pl_e = np.concatenate([pl, np.full((B, Hq, 2), -np.inf)], axis=2)
    o3, l3 = oracle.lse_merge(po_e, pl_e)
    np.testing.assert_allclose(o3, o, rtol=1e-15, atol=0)
    np.testing.assert_allclose(l3, lse, rtol=1e-15, atol=0)
    # all chunks empty
    o4, l4 = oracle.lse_merge(np.zeros((1, 1, 3, d)), np.full((1, 1, 3), -np.inf))
    assert np.all(o4 == 0) and np.all(l4 == -np.inf)


def _fold_tree(states, rng):
    """Combine a list of states in a random binary tree shape."""
    states = list(states)
    while len(states) > 1:
        i = int(rng.integers(0, len(states) - 1))
        merged = oracle.state_combine(states[i], states[i + 1])
        states[i:i + 2] = [merged]
    return states[0]


def test_online_monoid_order_and_tree_independence():
    rng = np.random.default_rng(24)
    n, d = 40, 6
    s = rng.standard_normal(n) * 3
    v = rng.standard_normal((n, d))
    # materialised softmax
    p = np.exp(s - s.max())
    p /= p.sum()
    o_ref = p @ v
    lse_ref = logsumexp(s)
    singles = [(s[j], 1.0, v[j]) for j in range(n)]
    for trial in range(8):
        perm = rng.permutation(n)
        m, l, a = _fold_tree([singles[j] for j in perm], rng)
        np.testing.assert_allclose(a / l, o_ref, rtol=1e-12, atol=1e-13)
        assert m + math.log(l) == pytest.approx(lse_ref, rel=1e-13, abs=1e-13)


def test_online_monoid_laws():
    rng = np.random.default_rng(25)
    d = 4
    ident = (-np.inf, 0.0, np.zeros(d))
    x = (1.5, 2.0, rng.standard_normal(d))
    y = (-0.5, 0.7, rng.standard_normal(d))
    z = (3.0, 1.1, rng.standard_normal(d))
    for left in (oracle.state_combine(ident, x), oracle.state_combine(x, ident)):
        assert left[0] == x[0] and left[1] == x[1]
        np.testing.assert_array_equal(left[2], x[2])
    a = oracle.state_combine(oracle.state_combine(x, y), z)
    b = oracle.state_combine(x, oracle.state_combine(y, z))
    assert a[0] == b[0]
    assert a[1] == pytest.approx(b[1], rel=1e-14)
    np.testing.assert_allclose(a[2], b[2], rtol=1e-14, atol=1e-15)
    c = oracle.state_combine(y, x)
    d_ = oracle.state_combine(x, y)
    assert c[0] == d_[0] and c[1] == pytest.approx(d_[1], rel=1e-15)
