"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/attn_oracle.c`` to a temporary directory, plants one
plausible slip (a dropped scale, a wrong sign, an off-by-one mask, a wrong
operand or head map, a dropped term), builds the copy and runs a compact
battery of the same kinds of pins as ``test_oracle.py``.  The battery must pass
on the real oracle and fail on every mutant.
"""
import math
import os
import shutil

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attn_oracle.c")

# (name, text to find, replacement, expected occurrences)
MUTANTS = [
    ("scale_dropped", "s *= scale;                                     /* step 1 */",
     "s *= 1.0;", 1),
    ("mask_off_by_one", "return !causal || j <= i + (Nk - Nq);", "return !causal || j < i + (Nk - Nq);", 1),
    ("mask_wrong_alignment", "return !causal || j <= i + (Nk - Nq);", "return !causal || j <= i;", 1),
    ("max_not_subtracted_lse", "lse_h[i] = m + log(l);", "lse_h[i] = log(l);", 1),
    ("ds_sign", "dS[i * Nk + j] = p * (dp - Di + gl);", "dS[i * Nk + j] = p * (Di - dp + gl);", 1),
    ("ds_drops_D", "dS[i * Nk + j] = p * (dp - Di + gl);", "dS[i * Nk + j] = p * (dp + gl);", 1),
    ("ds_dlse_sign", "dS[i * Nk + j] = p * (dp - Di + gl);", "dS[i * Nk + j] = p * (dp - Di - gl);", 1),
    ("dq_scale_dropped", "dqh[i * d + c] *= scale;", "dqh[i * d + c] *= 1.0;", 1),
    ("dk_scale_dropped", "dkg[j * d + c] += scale * s * qh[i * d + c];",
     "dkg[j * d + c] += s * qh[i * d + c];", 1),
    ("dv_wrong_operand", "dvg[j * d + c] += p * doh[i * d + c];", "dvg[j * d + c] += p * qh[i * d + c];", 1),
    ("dv_transposed_P", "double s = dS[i * Nk + j], p = P[i * Nk + j];",
     "double s = dS[i * Nk + j], p = P[j * Nk + i];", 1),
    ("bwd_dk_stride_of_queries", "double *dkg = dk + ((size_t)b * Hkv + g) * (size_t)Nk * d;",
     "double *dkg = dk + ((size_t)b * Hkv + g) * (size_t)Nq * d;", 1),
    ("dq_wrong_operand", "dqh[i * d + c] += s * kg[j * d + c];", "dqh[i * d + c] += s * vg[j * d + c];", 1),
    ("head_map_interleaved", "int g = h / G;", "int g = h % Hkv;", 5),
    ("decode_chunk_short", "long j0 = (long)s * C, j1 = j0 + C;", "long j0 = (long)s * C, j1 = j0 + C - 1;", 1),
    ("append_drops_new_key", "for (long j = 0; j <= n; ++j) {\n                double sc = 0.0;",
     "for (long j = 0; j < n; ++j) {\n                double sc = 0.0;", 1),
    ("append_wrong_row", "double *krow = kc + (((size_t)b * Hkv + g) * (size_t)Lcap + n) * d;",
     "double *krow = kc + (((size_t)b * Hkv + g) * (size_t)Lcap + (n + 1 < Lcap ? n + 1 : n)) * d;", 1),
    ("append_value_from_key", "vrow[c] = v_new[((size_t)b * Hkv + g) * d + c];",
     "vrow[c] = k_new[((size_t)b * Hkv + g) * d + c];", 1),
    ("rope_sine_sign", "double c = cos(a), s = sgn * sin(a);", "double c = cos(a), s = -sgn * sin(a);", 1),
    ("rope_frequency", "double theta = pow(base, -2.0 * i / d);", "double theta = pow(base, -1.0 * i / d);", 1),
    ("rope_position_offset_dropped", "long p = pos0 + r % N;", "long p = r % N;", 1),
    ("rope_pairs_adjacent", "double x0 = xr[i], x1 = xr[i + half];", "double x0 = xr[i], x1 = xr[i ^ 1];", 1),
    ("merge_not_normalised", "for (int c = 0; c < d; ++c) oo[c] /= W;", "", 1),
    ("merge_lse_drops_max", "lse[(size_t)b * Hq + h] = M + log(W);", "lse[(size_t)b * Hq + h] = log(W);", 1),
    ("combine_wrong_weight", "*l = l1 * w1 + l2 * w2;", "*l = l1 * w1 + l2 * w1;", 1),
    ("dual_product_rule", "return dl_make(a.v * b.v, a.v * b.e + a.e * b.v);",
     "return dl_make(a.v * b.v, a.v * b.e);", 1),
    ("dual_exp_rule", "double x = exp(a.v); return dl_make(x, x * a.e);",
     "double x = exp(a.v); return dl_make(x, a.e);", 1),
    ("no_max_subtraction", "double e = (Pi[j] == -INFINITY) ? 0.0 : exp(Pi[j] - m);",
     "double e = (Pi[j] == -INFINITY) ? 0.0 : exp(Pi[j]) * exp(-m);", 1),
]


def _textbook(q, k, v, causal, scale, G):
    B, Hq, N, d = q.shape
    k, v = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
            lse[b, h] = logsumexp(s, axis=1)
            o[b, h] = np.exp(s - lse[b, h][:, None]) @ v[b, h]
    return o, lse


def battery(O) -> list:
    """Returns the names of the pins that failed (empty on a correct oracle)."""
    failed = []
    rng = np.random.default_rng(99)

    def check(name, ok):
        if not ok:
            failed.append(name)

    # page-printed and closed-form dual values
    for x, val, der in ((0.0, 0.0, 0.0), (math.pi / 2, math.pi / 2, 1.0), (math.pi, 0.0, -math.pi)):
        v_, d_ = O.dual_xsinx(x)
        check("dual_golden", abs(v_ - val) < 1e-12 and abs(d_ - der) < 1e-12)

    # hand-worked two-key example
    q = np.array([1.0, 1.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, math.log(3)]).reshape(1, 1, 2, 1)
    v = np.array([4.0, 8.0]).reshape(1, 1, 2, 1)
    o, lse = O.attn_fwd(q, k, v, True, 1.0)
    check("worked_fwd", np.allclose(o.ravel(), [4, 7], atol=1e-12)
          and np.allclose(lse.ravel(), [0, math.log(4)], atol=1e-12))
    dq, dk, dv = O.attn_bwd(q, k, v, np.ones((1, 1, 2, 1)), True, 1.0)
    check("worked_bwd", np.allclose(dq.ravel(), [0, 0.75 * math.log(3)], atol=1e-12)
          and np.allclose(dk.ravel(), [-0.75, 0.75], atol=1e-12)
          and np.allclose(dv.ravel(), [1.25, 0.75], atol=1e-12))

    # textbook comparison with GQA (G = 2), scale != 1, and very large scores
    B, Hkv, G, N, d = 1, 2, 2, 9, 4
    q = rng.standard_normal((B, Hkv * G, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal(q.shape)
    for scale in (0.45, 300.0):
        o, lse = O.attn_fwd(q, k, v, True, scale)
        ot, lt = _textbook(q, k, v, True, scale, G)
        check("textbook", np.allclose(o, ot, rtol=1e-10, atol=1e-11)
              and np.allclose(lse, lt, rtol=1e-10, atol=1e-10))

    # cross-length causal mask: query i sits at absolute position i + (Nk - Nq)
    qx = rng.standard_normal((1, 1, 3, d))
    kx, vx = rng.standard_normal((1, 1, 7, d)), rng.standard_normal((1, 1, 7, d))
    sx = 0.5 * (qx[0, 0] @ kx[0, 0].T)
    sx = np.where(np.arange(7)[None, :] > np.arange(3)[:, None] + 4, -np.inf, sx)
    ox, lx = O.attn_fwd(qx, kx, vx, True, 0.5)
    check("cross_length", np.allclose(ox[0, 0], np.exp(sx - logsumexp(sx, axis=1)[:, None]) @ vx[0, 0],
                                      rtol=1e-11, atol=1e-12))

    # finite differences of the backward
    qs, ks, vs, dos = q[:, :2, :4], k[:, :1, :4], v[:, :1, :4], do[:, :2, :4]
    dq, dk, dv = O.attn_bwd(qs, ks, vs, dos, True, 0.6)
    h = 1e-6
    ok = True
    for which, x, g in (("q", qs, dq), ("k", ks, dk), ("v", vs, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = {"q": qs, "k": ks, "v": vs}
            a[which] = xp
            lp = np.sum(O.attn_fwd(a["q"], a["k"], a["v"], True, 0.6)[0] * dos)
            a[which] = xm
            lm = np.sum(O.attn_fwd(a["q"], a["k"], a["v"], True, 0.6)[0] * dos)
            ok = ok and abs((lp - lm) / (2 * h) - g[idx]) <= 1e-6
    check("finite_differences", ok)

    # dual-number directional derivative against the backward
    tq, tk, tv = (rng.standard_normal(x.shape) for x in (q, k, v))
    _, to, _, _ = O.attn_fwd_dual(q, tq, k, tk, v, tv, True, 0.45)
    dq, dk, dv = O.attn_bwd(q, k, v, do, True, 0.45)
    lhs = float(np.sum(do * to))
    rhs = float(np.sum(dq * tq) + np.sum(dk * tk) + np.sum(dv * tv))
    check("dual_vs_bwd", abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)))

    # upstream gradient of lse: the dual directional derivative of <o, dO> + <lse, dlse>
    dl = rng.standard_normal((B, Hkv * G, N))
    _, to2, _, tl2 = O.attn_fwd_dual(q, tq, k, tk, v, tv, True, 0.45)
    dq2, dk2, dv2 = O.attn_bwd_dlse(q, k, v, do, dl, True, 0.45)
    lhs2 = float(np.sum(do * to2) + np.sum(dl * tl2))
    rhs2 = float(np.sum(dq2 * tq) + np.sum(dk2 * tk) + np.sum(dv2 * tv))
    check("dual_vs_bwd_dlse", abs(lhs2 - rhs2) <= 1e-10 * max(1.0, abs(lhs2)))

    # cross-length backward: the square problem with dO = 0 on the first Nk - Nq rows
    qc, doc = q[:, :, 6:], do[:, :, 6:]
    dqc, dkc, dvc = O.attn_bwd(qc, k, v, doc, True, 0.45)
    dof = np.concatenate([np.zeros_like(do[:, :, :6]), doc], axis=2)
    dqf, dkf, dvf = O.attn_bwd(q, k, v, dof, True, 0.45)
    check("bwd_cross_length", dkc.shape == k.shape and np.allclose(dqc, dqf[:, :, 6:], rtol=1e-11, atol=1e-12)
          and np.allclose(dkc, dkf, rtol=1e-11, atol=1e-12) and np.allclose(dvc, dvf, rtol=1e-11, atol=1e-12))

    # rotary positions: a complex turn of each (x_i, x_{i+d/2}) pair by p base^(-2i/d)
    xr = rng.standard_normal((1, 2, 5, 8))
    z = xr[..., :4] + 1j * xr[..., 4:]
    w = np.exp(1j * (3 + np.arange(5))[:, None] * np.power(500.0, -2.0 * np.arange(4) / 8)[None, :])
    yz = z * w
    yr = O.rope(xr, 3, 500.0)
    check("rope", np.allclose(yr, np.concatenate([yz.real, yz.imag], axis=-1), rtol=1e-12, atol=1e-12)
          and np.allclose(O.rope(yr, 3, 500.0, True), xr, rtol=1e-12, atol=1e-12))

    # backward invariants
    check("bwd_invariants", np.allclose(dk.sum(axis=2), 0, atol=1e-10) and np.all(dq[:, :, 0] == 0))

    # decode: split count invariance, and equality with the last causal row
    L = 13
    Q = rng.standard_normal((1, 4, L, d))
    kc = rng.standard_normal((1, 2, L, d))
    vc = rng.standard_normal((1, 2, L, d))
    o_full, l_full = O.attn_fwd(Q, kc, vc, True, 0.5)
    ok = True
    for S in (1, 3, 13, 16):
        po, pl = O.attn_decode(Q[:, :, -1], kc, vc, 0.5, S)
        od, ld = O.lse_merge(po, pl)
        ok = ok and np.allclose(od, o_full[:, :, -1], rtol=1e-11, atol=1e-12) \
            and np.allclose(ld, l_full[:, :, -1], rtol=1e-11, atol=1e-12)
    check("decode", ok)

    # decode step with append: n = 0 closed form, last causal row, cache rows
    Bq, Hq2, Hkv2, Lc, d2 = 2, 4, 2, 8, 4
    qa = rng.standard_normal((Bq, Hq2, d2))
    kn, vn = rng.standard_normal((Bq, Hkv2, d2)), rng.standard_normal((Bq, Hkv2, d2))
    kca, vca = rng.standard_normal((Bq, Hkv2, Lc, d2)), rng.standard_normal((Bq, Hkv2, Lc, d2))
    oa, la, kc2, vc2 = O.attn_decode_append(qa, kn, vn, kca, vca, [0, 5], 0.6)
    ok = np.allclose(oa[0], np.repeat(vn[0], 2, axis=0), rtol=1e-14, atol=1e-14)
    K = np.concatenate([kca[1:2, :, :5], kn[1:2, :, None]], axis=2)
    V = np.concatenate([vca[1:2, :, :5], vn[1:2, :, None]], axis=2)
    for h in range(Hq2):
        sc = 0.6 * (K[0, h // 2] @ qa[1, h])
        ok = ok and np.allclose(oa[1, h], np.exp(sc - logsumexp(sc)) @ V[0, h // 2], rtol=1e-12)
        ok = ok and abs(la[1, h] - logsumexp(sc)) < 1e-12
    ok = ok and np.array_equal(kc2[1, :, 5], kn[1]) and np.array_equal(vc2[1, :, 5], vn[1]) \
        and np.array_equal(kc2[1, :, 6:], kca[1, :, 6:]) and np.array_equal(kc2[0, :, 1:], kca[0, :, 1:])
    check("decode_append", ok)

    # the online monoid: folds of singletons equal the materialised softmax
    s = rng.standard_normal(12) * 2
    vv = rng.standard_normal((12, 3))
    st = (s[0], 1.0, vv[0])
    for j in range(1, 12):
        st = O.state_combine(st, (s[j], 1.0, vv[j]))
    p = np.exp(s - logsumexp(s))
    check("monoid", np.allclose(st[2] / st[1], p @ vv, rtol=1e-12)
          and abs(st[0] + math.log(st[1]) - logsumexp(s)) < 1e-12)
    return failed


def test_battery_passes_on_the_oracle():
    assert battery(oracle.default()) == []


@pytest.mark.parametrize("name,find,repl,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, find, repl, count):
    text = open(SRC).read()
    assert text.count(find) == count, f"mutation site for {name} not found as expected"
    mutated = text.replace(find, repl)
    src = tmp_path / "attn_oracle.c"
    src.write_text(mutated)
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "liboracle_mutant.so"))
    failed = battery(oracle.Oracle(lib))
    assert failed, f"mutant {name} passed every pin"
    shutil.rmtree(tmp_path, ignore_errors=True)
