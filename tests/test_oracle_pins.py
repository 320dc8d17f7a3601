"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check below compares the oracle with something independent: a library
routine (torch's scaled-dot-product attention and forward-mode autodiff,
numpy's weighted covariance, numpy's least squares), a closed form worked out
by hand, or an invariant that follows from the definition in Eq. 2 of the page
"Parallax - Parameterized Local Linear Attention for Language Modeling"
(section "Core mechanism").  `test_planted_mistakes_are_caught` then plants
plausible mistakes in copies of the oracle and checks that at least one pin
fails for each.

CPU only; the whole file runs in seconds.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import parallax_oracle as po

HERE = os.path.dirname(os.path.abspath(__file__))


def _real_impl():
    return types.SimpleNamespace(prefill=po.prefill, decode=po.decode,
                                 explicit_row=po.explicit_row,
                                 prefill_explicit=po.prefill_explicit,
                                 prefill_rows=po.prefill_rows)


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _prefill_case(seed, B=1, H=2, L=24, dk=6, dv=6, rho_std=0.7):
    rng = np.random.default_rng(seed)
    return dict(q=_rand(rng, B, H, L, dk), k=_rand(rng, B, H, L, dk),
                v=_rand(rng, B, H, L, dv), rho=_rand(rng, B, H, L, dk, std=rho_std),
                gate=rng.uniform(0.2, 1.0, H))


def _sdpa(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal,
                                          scale=scale).numpy()


# --------------------------------------------------------------------- pins
def pin_rho_zero_is_softmax_attention(impl):
    """Section "Significance": with W_R = 0 (rho = 0) the layer is ordinary
    softmax attention; same with gate 0.  Reference: torch SDPA in fp64."""
    c = _prefill_case(1, dk=5, dv=7)
    sc = 0.37
    ref = _sdpa(c["q"], c["k"], c["v"], sc, causal=True)
    out = impl.prefill(c["q"], c["k"], c["v"], np.zeros_like(c["rho"]), c["gate"], scale=sc)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    out = impl.prefill(c["q"], c["k"], c["v"], c["rho"], np.zeros(2), scale=sc)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # decode attends every cached key: compare with non-causal SDPA
    rng = np.random.default_rng(2)
    q = _rand(rng, 2, 2, 1, 5)
    kc, vc = _rand(rng, 2, 2, 9, 5), _rand(rng, 2, 2, 9, 7)
    ref = _sdpa(q, kc, vc, sc, causal=False)[:, :, 0]
    out = impl.decode(q[:, :, 0], kc, vc, np.zeros((2, 2, 5)), np.ones(2), [9, 9], scale=sc)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_sigma_is_weighted_covariance(impl):
    """Sigma_KV (d_v x d_k) equals numpy's weighted cross-covariance block with
    the softmax weights as aweights and no Bessel correction."""
    rng = np.random.default_rng(3)
    n, dk, dv = 11, 4, 3
    q, K, V, rho = _rand(rng, dk), _rand(rng, n, dk), _rand(rng, n, dv), _rand(rng, dk)
    sc = 0.8
    _, o_sa, sigma = impl.explicit_row(q, K, V, rho, 1.0, sc)
    s = sc * K @ q
    w = np.exp(s - s.max())
    w /= w.sum()
    cov = np.cov(np.vstack([V.T, K.T]), aweights=w, bias=True)
    assert sigma.shape == (dv, dk)
    np.testing.assert_allclose(sigma, cov[:dv, dv:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(o_sa, np.average(V, axis=0, weights=w), rtol=0, atol=1e-13)


def pin_correction_is_score_tilt_derivative(impl):
    """Sigma rho is the derivative of softmax attention when every score s_j is
    tilted by t * r_j: d/dt sum_j softmax(s + t r)_j v_j = Cov_w(v, r).  Since
    r_j = <rho, k_j> and s_j = scale <q, k_j>, the tilt is q -> q + t rho/scale.
    Reference: torch.func.jvp through torch's fp64 SDPA (causal prefill and
    non-causal decode)."""
    c = _prefill_case(4, dk=6, dv=5, L=20)
    sc = 0.41
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    q, k, v, rho = map(t, (c["q"], c["k"], c["v"], c["rho"]))

    def att(x):
        return F.scaled_dot_product_attention(x, k, v, is_causal=True, scale=sc)

    o_sa, dir_deriv = torch.func.jvp(att, (q,), (rho / sc,))
    g = torch.from_numpy(c["gate"])[None, :, None, None]
    ref = (o_sa - g * dir_deriv).numpy()
    out = impl.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"], scale=sc)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)

    rng = np.random.default_rng(5)
    qd, rd = _rand(rng, 1, 3, 6), _rand(rng, 1, 3, 6, std=2.0)
    kc, vc = _rand(rng, 1, 3, 13, 6), _rand(rng, 1, 3, 13, 4)
    kt, vt = t(kc), t(vc)

    def att_d(x):
        return F.scaled_dot_product_attention(x, kt, vt, is_causal=False, scale=sc)

    o_sa, dd = torch.func.jvp(att_d, (t(qd[:, :, None]),), (t(rd[:, :, None] / sc),))
    ref = (o_sa - 0.6 * dd)[:, :, 0].numpy()
    out = impl.decode(qd, kc, vc, rd, np.full(3, 0.6), [13], scale=sc)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)


def pin_local_linear_regression(impl):
    """Section "Core mechanism": Parallax replaces the per-query optimal probe
    rho* (which needs a covariance inverse) by a learned one.  With the probe
    set to rho* = Sigma_KK^-1 (kbar - q) and gate 1, Eq. 2 must give the
    intercept of the softmax-weighted least-squares fit of v on (k - q): the
    local-linear estimate at q.  Reference: numpy lstsq and np.cov."""
    rng = np.random.default_rng(6)
    n, dk, dv = 40, 4, 3
    q, K, V = _rand(rng, dk), _rand(rng, n, dk), _rand(rng, n, dv)
    sc = 0.5
    s = sc * K @ q
    w = np.exp(s - s.max())
    w /= w.sum()
    kbar = np.average(K, axis=0, weights=w)
    s_kk = np.cov(K.T, aweights=w, bias=True)
    rho_star = np.linalg.solve(s_kk, kbar - q)
    X = np.hstack([np.ones((n, 1)), K - q])
    sw = np.sqrt(w)[:, None]
    coef = np.linalg.lstsq(sw * X, sw * V, rcond=None)[0]
    intercept = coef[0]
    out = impl.decode(q[None, None], K[None, None], V[None, None], rho_star[None, None],
                      np.ones(1), [n], scale=sc)[0, 0]
    np.testing.assert_allclose(out, intercept, rtol=0, atol=1e-10)


def pin_closed_forms(impl):
    """Closed forms worked from Eq. 2: one key gives o = v_0 exactly; two keys
    give o = o_SA - g w0 w1 (v0 - v1)(r0 - r1); identical keys give no
    correction and a uniform average; constant values give o = v."""
    c = _prefill_case(7, dk=5, dv=3)
    out = impl.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"])
    assert np.array_equal(out[:, :, 0], c["v"][:, :, 0])        # row 0 = v_0 exactly

    rng = np.random.default_rng(8)
    q, K, V, rho = _rand(rng, 5), _rand(rng, 2, 5), _rand(rng, 2, 3), _rand(rng, 5)
    sc, g = 0.9, 0.7
    s = sc * K @ q
    w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    w1 = 1.0 - w0
    r = K @ rho
    o_sa = w0 * V[0] + w1 * V[1]
    ref = o_sa - g * w0 * w1 * (V[0] - V[1]) * (r[0] - r[1])
    out = impl.decode(q[None, None], K[None, None], V[None, None], rho[None, None],
                      np.array([g]), [2], scale=sc)[0, 0]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)

    L = 12
    q = _rand(rng, 1, 1, L, 4)
    k = np.repeat(_rand(rng, 1, 1, 1, 4), L, axis=2)
    v = _rand(rng, 1, 1, L, 3)
    rho = _rand(rng, 1, 1, L, 4, std=3.0)
    out = impl.prefill(q, k, v, rho, np.ones(1))
    ref = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)

    v = np.repeat(_rand(rng, 1, 1, 1, 3), L, axis=2)
    k = _rand(rng, 1, 1, L, 4)
    out = impl.prefill(q, k, v, rho, np.ones(1))
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-12)


def pin_invariants(impl):
    """Invariants of Eq. 2: a common shift of all keys changes neither the
    weights nor the covariance; a shift of all values shifts the output; the
    correction is linear in rho and in g; and by Cauchy-Schwarz each component
    of Sigma rho is bounded by sqrt(Var_w(v_m) Var_w(r))."""
    c = _prefill_case(9, dk=5, dv=4, L=16)
    base = impl.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"])
    shift_k = np.random.default_rng(10).standard_normal(5) * 3
    out = impl.prefill(c["q"], c["k"] + shift_k, c["v"], c["rho"], c["gate"])
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-10)
    shift_v = np.arange(4) - 1.5
    out = impl.prefill(c["q"], c["k"], c["v"] + shift_v, c["rho"], c["gate"])
    np.testing.assert_allclose(out, base + shift_v, rtol=0, atol=1e-11)

    o_sa = impl.prefill(c["q"], c["k"], c["v"], 0 * c["rho"], c["gate"])
    corr = o_sa - base
    out = impl.prefill(c["q"], c["k"], c["v"], 2.5 * c["rho"], c["gate"])
    np.testing.assert_allclose(o_sa - out, 2.5 * corr, rtol=0, atol=1e-11)
    out = impl.prefill(c["q"], c["k"], c["v"], c["rho"], 0.5 * c["gate"])
    np.testing.assert_allclose(o_sa - out, 0.5 * corr, rtol=0, atol=1e-11)

    rng = np.random.default_rng(11)
    q, K, V, rho = _rand(rng, 6), _rand(rng, 30, 6), _rand(rng, 30, 4), _rand(rng, 6, std=2)
    out = impl.decode(q[None, None], K[None, None], V[None, None], rho[None, None],
                      np.ones(1), [30], scale=0.6)[0, 0]
    s = 0.6 * K @ q
    w = np.exp(s - s.max())
    w /= w.sum()
    r = K @ rho
    var_r = np.average((r - np.average(r, weights=w)) ** 2, weights=w)
    var_v = np.average((V - np.average(V, axis=0, weights=w)) ** 2, axis=0, weights=w)
    corr = np.average(V, axis=0, weights=w) - out
    assert np.all(np.abs(corr) <= np.sqrt(var_v * var_r) + 1e-12)


def pin_hand_cases(impl):
    """Exact rational results worked by hand (tests/golden/hand_cases.json)."""
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v, rho = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v", "rho"))
        g = np.array([c["gate"]])
        if c["kind"] == "decode":
            out = impl.decode(q[None, None], k[None, None], v[None, None], rho[None, None],
                              g, [k.shape[0]], scale=c["scale"])[0, 0]
        else:
            out = impl.prefill(q[None, None], k[None, None], v[None, None], rho[None, None],
                               g, scale=c["scale"])[0, 0]
        np.testing.assert_allclose(out, np.array(c["expected"]), rtol=0, atol=1e-13,
                                   err_msg=c["name"])


def pin_decode_matches_prefill_row(impl):
    """A decode over the first i+1 keys of a sequence is prefill row i."""
    c = _prefill_case(12, B=2, H=2, L=17, dk=4, dv=4)
    pre = impl.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"])
    for i in (0, 5, 16):
        dec = impl.decode(c["q"][:, :, i], c["k"], c["v"], c["rho"][:, :, i], c["gate"],
                          [i + 1, i + 1])
        np.testing.assert_allclose(dec, pre[:, :, i], rtol=0, atol=1e-12)


def pin_prefill_rows(impl):
    """The selected-rows checker (explicit form, one head at a time) against the
    score-tilt derivative of torch's fp64 causal SDPA (the independent reference
    of pin_correction_is_score_tilt_derivative), at rows 0, 1, a middle row and
    the last row of every head of a B=2, H=3 case whose heads have distinct
    gates; and against the expanded form on the same rows."""
    c = _prefill_case(16, B=2, H=3, L=21, dk=6, dv=5, rho_std=1.3)
    c["gate"] = np.array([0.25, 0.6, 1.1])
    sc = 0.47
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    q, k, v, rho = map(t, (c["q"], c["k"], c["v"], c["rho"]))

    def att(x):
        return F.scaled_dot_product_attention(x, k, v, is_causal=True, scale=sc)

    o_sa, dd = torch.func.jvp(att, (q,), (rho / sc,))
    ref = (o_sa - torch.from_numpy(c["gate"])[None, :, None, None] * dd).numpy()
    full = impl.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"], scale=sc)
    rows = [0, 1, 10, 20]
    for b in range(2):
        for h in range(3):
            got = impl.prefill_rows(c["q"], c["k"], c["v"], c["rho"], c["gate"], b, h, rows,
                                    scale=sc)
            assert got.shape == (len(rows), 5)
            np.testing.assert_allclose(got, ref[b, h, rows], rtol=0, atol=1e-12)
            np.testing.assert_allclose(got, full[b, h, rows], rtol=0, atol=1e-12)
    # the default scale is 1/sqrt(d_k)
    got = impl.prefill_rows(c["q"], c["k"], c["v"], c["rho"], c["gate"], 1, 2, [20])
    full = impl.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"], scale=1 / np.sqrt(6))
    np.testing.assert_allclose(got[0], full[1, 2, 20], rtol=0, atol=1e-12)


PINS = [pin_rho_zero_is_softmax_attention, pin_sigma_is_weighted_covariance,
        pin_correction_is_score_tilt_derivative, pin_local_linear_regression,
        pin_closed_forms, pin_invariants, pin_hand_cases, pin_decode_matches_prefill_row,
        pin_prefill_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_real_impl())


# ------------------------------------------------------- internal agreement
def test_explicit_and_expanded_forms_agree():
    c = _prefill_case(13, B=1, H=2, L=40, dk=8, dv=8)
    a = po.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"])
    b = po.prefill_explicit(c["q"], c["k"], c["v"], c["rho"], c["gate"])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    rng = np.random.default_rng(14)
    q, rho = _rand(rng, 2, 2, 8), _rand(rng, 2, 2, 8)
    kc, vc = _rand(rng, 2, 2, 50, 8), _rand(rng, 2, 2, 50, 8)
    a = po.decode(q, kc, vc, rho, np.ones(2), [50, 7])
    b = po.decode_explicit(q, kc, vc, rho, np.ones(2), [50, 7])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_decode_length_edge_cases():
    """Length 0 gives zeros; lengths are clamped to [0, Lmax]; cache rows past
    a sequence's length are never read (NaN there changes nothing)."""
    rng = np.random.default_rng(15)
    q, rho = _rand(rng, 3, 1, 4), _rand(rng, 3, 1, 4)
    kc, vc = _rand(rng, 3, 1, 6, 4), _rand(rng, 3, 1, 6, 4)
    kc[1, :, 3:] = np.nan
    vc[1, :, 3:] = np.nan
    out = po.decode(q, kc, vc, rho, np.ones(1), [0, 3, 99])
    assert np.all(out[0] == 0.0)
    assert np.all(np.isfinite(out[1]))
    ref = po.decode(q[2:], kc[2:], vc[2:], rho[2:], np.ones(1), [6])
    np.testing.assert_array_equal(out[2], ref[0])


# ---------------------------------------------------------- planted mistakes
def _mutant_prefill(kind):
    def prefill(q, k, v, rho, gate, scale=None, heads=None):
        q, k, v, rho, gate = map(po._f64, (q, k, v, rho, gate))
        B, H, L, dk = q.shape
        sc = 1 / np.sqrt(dk) if scale is None else scale
        out = np.empty(v.shape)
        for b in range(B):
            for h in range(H):
                S = sc * q[b, h] @ k[b, h].T
                off = 1 if kind == "mask_off_by_one" else 0
                mask = np.arange(L)[None, :] <= np.arange(L)[:, None] + off
                S = np.where(mask, S, -np.inf)
                W = np.exp(S - S.max(1, keepdims=True))
                W /= W.sum(1, keepdims=True)
                R = rho[b, h] @ k[b, h].T
                if kind == "scaled_r":
                    R = sc * R
                WR = W * R
                o_sa = W @ v[b, h]
                u = WR @ v[b, h]
                rbar = WR.sum(1, keepdims=True)
                if kind == "dropped_mean_term":
                    corr = u
                elif kind == "sign_flip":
                    corr = -(u - o_sa * rbar)
                elif kind == "gate_on_output":
                    out[b, h] = gate[h] * (o_sa - (u - o_sa * rbar))
                    continue
                else:
                    corr = u - o_sa * rbar
                out[b, h] = o_sa - gate[h] * corr
        return out
    return prefill


def _mutant_explicit_row(kind):
    def explicit_row(q_i, K, V, rho_i, g, scale):
        w = po.softmax_weights(q_i, K, scale)
        o_sa = w @ V
        kbar = w @ K
        if kind == "uncentred":
            sigma = V.T @ (w[:, None] * K)
        elif kind == "transposed":
            sigma = ((V - o_sa).T @ (w[:, None] * (K - kbar))).T
        else:
            sigma = (V - o_sa).T @ (w[:, None] * (K - kbar))
        # a shape mismatch raises, which also counts as a caught mistake
        return o_sa - g * (sigma @ rho_i), o_sa, sigma
    return explicit_row


def _mutant_decode(prefill_impl):
    """A decode built from a (mutated) prefill: the query is placed last."""
    def decode(q, kc, vc, rho, gate, seqlens, scale=None, streams=None):
        kc, vc = po._f64(kc), po._f64(vc)
        q, rho = po._f64(q), po._f64(rho)
        B, H, Lmax, dk = kc.shape
        out = np.zeros((B, H, vc.shape[-1]))
        for b in range(B):
            n = int(min(max(int(seqlens[b]), 0), Lmax))
            if n == 0:
                continue
            qq = np.zeros((1, H, n, dk))
            qq[0, :, n - 1] = q[b]
            rr = np.zeros((1, H, n, dk))
            rr[0, :, n - 1] = rho[b]
            o = prefill_impl(qq, kc[b: b + 1, :, :n], vc[b: b + 1, :, :n], rr, gate,
                             scale=scale)
            out[b] = o[0, :, n - 1]
        return out
    return decode


def _mutant_prefill_rows(kind):
    """prefill_rows with one plausible indexing mistake."""
    def prefill_rows(q, k, v, rho, gate, b, h, rows, scale=None):
        dk = q.shape[-1]
        sc = 1 / np.sqrt(dk) if scale is None else scale
        gf = po._f64(gate)
        g = float(gf[b] if kind == "rows_gate_by_b" else gf[h])
        res = []
        for i in rows:
            i = int(i)
            n = i if kind == "rows_diagonal_dropped" else i + 1
            if kind == "rows_key_window_shifted":
                K, V = k[b, h, 1: i + 2], v[b, h, 1: i + 2]
            else:
                K, V = k[b, h, : max(n, 1)], v[b, h, : max(n, 1)]
            qi = q[b, h, i]
            ri = rho[b, h, i - 1] if kind == "rows_rho_of_previous_row" else rho[b, h, i]
            res.append(po.explicit_row(qi, K, V, ri, g, sc)[0])
        return np.stack(res)
    return prefill_rows


MUTANTS = ["sign_flip", "dropped_mean_term", "scaled_r", "mask_off_by_one",
           "gate_on_output", "uncentred", "transposed", "rows_diagonal_dropped",
           "rows_gate_by_b", "rows_key_window_shifted", "rows_rho_of_previous_row"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind):
    impl = _real_impl()
    if kind.startswith("rows_"):
        impl.prefill_rows = _mutant_prefill_rows(kind)
    elif kind in ("uncentred", "transposed"):
        impl.explicit_row = _mutant_explicit_row(kind)
    else:
        impl.prefill = _mutant_prefill(kind)
        impl.decode = _mutant_decode(impl.prefill)
    failures = []
    for pin in PINS:
        try:
            pin(impl)
        except Exception as e:  # any assertion or shape error is a caught mistake
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake {kind!r}"
