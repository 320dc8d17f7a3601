"""Pins of the oracle's training statistics and backward pass.

The pages give no backward pass, so the oracle's gradients are the exact
derivative of Eq. 2 (page "Parallax - Parameterized Local Linear Attention for
Language Modeling", section "Core mechanism"), written out by hand.  They are
pinned here against things that do not come from that derivation:
  * torch autograd in fp64 through a forward written in this file from the
    explicit covariance definition (Sigma^(i) built as a matrix per row);
  * central differences of the oracle's forward pass (itself pinned in
    test_oracle_pins.py);
  * special cases that reduce to torch's scaled-dot-product attention: rho = 0
    or gate = 0 leave softmax attention, whose gradients autograd gives.
`test_planted_backward_mistakes_are_caught` plants plausible mistakes in copies
of the backward and checks that a pin fails for each.  CPU only, seconds.
"""
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import parallax_oracle as po


def _case(seed, B=1, H=2, L=20, d=6, rho_std=0.7):
    rng = np.random.default_rng(seed)
    r = lambda *s, std=1.0: rng.standard_normal(s) * std
    return dict(q=r(B, H, L, d), k=r(B, H, L, d), v=r(B, H, L, d), rho=r(B, H, L, d, std=rho_std),
                gate=rng.uniform(0.2, 1.2, H), dout=r(B, H, L, d))


def _t(a, grad=True):
    return torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=grad)


def _explicit_forward_torch(q, k, v, rho, gate, scale):
    """Eq. 2 with Sigma^(i) as an explicit d x d matrix per row (torch, fp64)."""
    B, H, L, d = q.shape
    rows = []
    for b in range(B):
        for h in range(H):
            out_h = []
            for i in range(L):
                K, V = k[b, h, : i + 1], v[b, h, : i + 1]
                w = torch.softmax(scale * (K @ q[b, h, i]), dim=0)
                o_sa = w @ V
                kbar = w @ K
                sigma = (V - o_sa).T @ (w[:, None] * (K - kbar))
                out_h.append(o_sa - gate[h] * (sigma @ rho[b, h, i]))
            rows.append(torch.stack(out_h))
    return torch.stack(rows).view(B, H, L, -1)


def _autograd(c, scale):
    ts = {n: _t(c[n]) for n in ("q", "k", "v", "rho", "gate")}
    out = _explicit_forward_torch(ts["q"], ts["k"], ts["v"], ts["rho"], ts["gate"], scale)
    (out * _t(c["dout"], False)).sum().backward()
    return {n: ts[n].grad.numpy() for n in ts}, out.detach().numpy()


def _sdpa_grads(c, scale):
    ts = {n: _t(c[n]) for n in ("q", "k", "v")}
    out = F.scaled_dot_product_attention(ts["q"], ts["k"], ts["v"], is_causal=True, scale=scale)
    (out * _t(c["dout"], False)).sum().backward()
    return {n: ts[n].grad.numpy() for n in ts}


def _real():
    return types.SimpleNamespace(backward=po.prefill_backward, train=po.prefill_train)


def _grads(impl, c, scale):
    g = impl.backward(c["q"], c["k"], c["v"], c["rho"], c["gate"], c["dout"], scale=scale)
    return dict(q=g["dq"], k=g["dk"], v=g["dv"], rho=g["drho"], gate=g["dgate"])


# --------------------------------------------------------------------- pins
def pin_backward_matches_autograd(impl):
    for seed, scale in ((1, 0.41), (2, None)):
        c = _case(seed)
        sc = 1 / np.sqrt(c["q"].shape[-1]) if scale is None else scale
        ref, _ = _autograd(c, sc)
        got = _grads(impl, c, scale)
        for n in ref:
            np.testing.assert_allclose(got[n], ref[n], rtol=0, atol=1e-11, err_msg=n)


def pin_backward_central_differences(impl):
    """d/dx of sum(out * dout) at random coordinates, by central differences of
    the oracle's forward pass with step 1e-5 (truncation error ~1e-10)."""
    c = _case(3, L=12, d=4)
    sc = 0.5
    got = _grads(impl, c, sc)
    rng = np.random.default_rng(4)
    f = lambda cc: float((po.prefill(cc["q"], cc["k"], cc["v"], cc["rho"], cc["gate"],
                                     scale=sc) * cc["dout"]).sum())
    eps = 1e-5
    for name in ("q", "k", "v", "rho", "gate"):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in c[name].shape)
            cp = {n: a.copy() for n, a in c.items()}
            cm = {n: a.copy() for n, a in c.items()}
            cp[name][idx] += eps
            cm[name][idx] -= eps
            fd = (f(cp) - f(cm)) / (2 * eps)
            assert abs(fd - got[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd,
                                                                          got[name][idx])


def pin_backward_rho_zero_is_softmax_attention(impl):
    """rho = 0 leaves softmax attention for any gate (section "Significance"):
    the q, k, v gradients are those of torch SDPA; the gate gradient is zero."""
    c = _case(5, d=5)
    c["rho"] = np.zeros_like(c["rho"])
    sc = 0.3
    ref = _sdpa_grads(c, sc)
    got = _grads(impl, c, sc)
    for n in ref:
        np.testing.assert_allclose(got[n], ref[n], rtol=0, atol=1e-12, err_msg=n)
    np.testing.assert_allclose(got["gate"], 0.0, atol=1e-12)


def pin_backward_gate_zero(impl):
    """gate = 0: q, k, v gradients are SDPA's and rho gets no gradient, while the
    gate gradient is minus the sum of dout . Sigma rho (built here with numpy's
    weighted covariance, row by row)."""
    c = _case(6, d=5)
    c["gate"] = np.zeros(2)
    sc = 0.45
    ref = _sdpa_grads(c, sc)
    got = _grads(impl, c, sc)
    for n in ref:
        np.testing.assert_allclose(got[n], ref[n], rtol=0, atol=1e-12, err_msg=n)
    np.testing.assert_allclose(got["rho"], 0.0, atol=1e-12)
    B, H, L, d = c["q"].shape
    want = np.zeros(H)
    for h in range(H):
        for i in range(L):
            K, V = c["k"][0, h, : i + 1], c["v"][0, h, : i + 1]
            s = sc * K @ c["q"][0, h, i]
            w = np.exp(s - s.max())
            w /= w.sum()
            if i == 0:
                sig = np.zeros((d, d))
            else:
                full = np.cov(np.concatenate([V, K], axis=1).T, aweights=w, bias=True)
                sig = full[:d, d:]
            want[h] -= c["dout"][0, h, i] @ (sig @ c["rho"][0, h, i])
    np.testing.assert_allclose(got["gate"], want, rtol=0, atol=1e-11)


def pin_train_statistics(impl):
    """The saved statistics: out is the oracle's forward output, lse is torch's
    logsumexp of the masked scores, corr equals Sigma^(i) rho_i from the
    explicit form, and out = o_sa - g corr with o_sa from torch SDPA."""
    c = _case(7)
    sc = 0.6
    st = impl.train(c["q"], c["k"], c["v"], c["rho"], c["gate"], scale=sc)
    fwd = po.prefill(c["q"], c["k"], c["v"], c["rho"], c["gate"], scale=sc)
    np.testing.assert_allclose(st["out"], fwd, rtol=0, atol=1e-12)
    S = sc * torch.from_numpy(c["q"]) @ torch.from_numpy(c["k"]).transpose(-1, -2)
    L = S.shape[-1]
    S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(st["lse"], torch.logsumexp(S, -1).numpy(), rtol=0, atol=1e-12)
    o_sa = F.scaled_dot_product_attention(*(torch.from_numpy(c[n]) for n in ("q", "k", "v")),
                                          is_causal=True, scale=sc).numpy()
    g = c["gate"][None, :, None, None]
    np.testing.assert_allclose(st["out"], o_sa - g * st["corr"], rtol=0, atol=1e-12)
    for h, i in ((0, 0), (1, 7), (0, 19)):
        _, _, sig = po.explicit_row(c["q"][0, h, i], c["k"][0, h, : i + 1], c["v"][0, h, : i + 1],
                                    c["rho"][0, h, i], 1.0, sc)
        np.testing.assert_allclose(st["corr"][0, h, i], sig @ c["rho"][0, h, i], rtol=0,
                                   atol=1e-12)
        w = po.softmax_weights(c["q"][0, h, i], c["k"][0, h, : i + 1], sc)
        np.testing.assert_allclose(st["rbar"][0, h, i], w @ (c["k"][0, h, : i + 1]
                                                             @ c["rho"][0, h, i]), atol=1e-12)


BACKWARD_PINS = [pin_backward_matches_autograd, pin_backward_central_differences,
                 pin_backward_rho_zero_is_softmax_attention, pin_backward_gate_zero,
                 pin_train_statistics]


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(_real())


def test_rows_in_blocks_match_one_block():
    """Row blocking is only for memory: blocks of 7 rows give the same result."""
    c = _case(8, L=30)
    a = po.prefill_head_backward(c["q"][0, 0], c["k"][0, 0], c["v"][0, 0], c["rho"][0, 0], 0.7,
                                 0.4, c["dout"][0, 0])
    b = po.prefill_head_backward(c["q"][0, 0], c["k"][0, 0], c["v"][0, 0], c["rho"][0, 0], 0.7,
                                 0.4, c["dout"][0, 0], block=7)
    for x, y in zip(a[:4], b[:4]):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
    assert abs(a[4] - b[4]) <= 1e-12


# ---------------------------------------------------------- planted mistakes
def _mutant_backward(kind):
    def head(q, k, v, rho, g, scale, dout):
        L = q.shape[0]
        r = np.arange(L)
        W, R, rbar, o_sa, corr, _ = po._head_forward_blocks(q, k, v, rho, g, scale, r, L)
        o = o_sa - g * corr
        Delta = dout @ v.T
        D = (dout * (o if kind == "D_from_output" else o_sa)).sum(1, keepdims=True)
        Fr = (dout * o).sum(1, keepdims=True)
        Rc = R - rbar
        dv = (W * (1.0 - g * Rc)).T @ dout if kind != "dv_without_tilt" else W.T @ dout
        dR = -g * W * (Delta - D)
        if kind == "dR_sign":
            dR = -dR
        tilt = g * Rc * D if kind != "dropped_D_term" else 0.0
        dS = W * (Delta * (1.0 - g * Rc) + tilt - Fr)
        dq = scale * (dS @ k) if kind != "dq_unscaled" else dS @ k
        dk = scale * (dS.T @ q) + (dR.T @ rho if kind != "dk_without_rho" else 0.0)
        drho = dR @ k if kind != "drho_transposed" else dR.T @ k
        dg = -float((dout * corr).sum()) if kind != "dg_sign" else float((dout * corr).sum())
        return dq, dk, dv, drho, dg

    def backward(q, k, v, rho, gate, dout, scale=None, heads=None):
        q, k, v, rho, gate, dout = map(po._f64, (q, k, v, rho, gate, dout))
        B, H, L, d = q.shape
        sc = 1 / np.sqrt(d) if scale is None else scale
        res = {n: np.zeros(q.shape) for n in ("dq", "dk", "dv", "drho")}
        res["dgate"] = np.zeros(H)
        for b in range(B):
            for h in range(H):
                g = head(q[b, h], k[b, h], v[b, h], rho[b, h], gate[h], sc, dout[b, h])
                res["dq"][b, h], res["dk"][b, h], res["dv"][b, h], res["drho"][b, h] = g[:4]
                res["dgate"][h] += g[4]
        return res
    return backward


MUTANTS = ["D_from_output", "dv_without_tilt", "dR_sign", "dropped_D_term", "dq_unscaled",
           "dk_without_rho", "drho_transposed", "dg_sign"]


def test_mutant_harness_is_faithful():
    """The unmutated copy used by the planted-mistake test passes every pin."""
    impl = _real()
    impl.backward = _mutant_backward("none")
    for pin in BACKWARD_PINS:
        pin(impl)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_backward_mistakes_are_caught(kind):
    impl = _real()
    impl.backward = _mutant_backward(kind)
    failures = []
    for pin in BACKWARD_PINS:
        try:
            pin(impl)
        except Exception as e:  # an assertion or a shape error is a caught mistake
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake {kind!r}"
