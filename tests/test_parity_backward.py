"""GPU parity of the training forward pass and the backward pass against the
fp64 CPU oracle (prefill_train, prefill_backward).

Tolerances.  Training statistics: out, rbar and corr within 2e-2 max-abs (the
bf16 forward's bound); lse within 1e-3 (the partition function sums fp16-rounded
numerators: relative error <= 2^-11 per term).  Gradients: max-abs error within
2e-2 x max(1, max|reference|) per tensor.  Gradients scale with the sequence
length and with dout, so the bound is relative to each tensor's magnitude;
dout and the softmax-weight gradients are rounded to bf16 for the matrix
products, which a precision emulation puts at 2e-3 to 4e-3 of that magnitude.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import parallax_oracle as po

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "drho")


def _plx():
    import parallax_local_linear_amd as plx
    return plx


def _np(x):
    return x.detach().cpu().double().numpy()


def _dout(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)


def _rel_err(got, ref):
    return float(np.max(np.abs(got - ref))) / max(1.0, float(np.max(np.abs(ref))))


def _run(inp, dout):
    plx = _plx()
    out, lse, rbar, corr = plx.prefill_train(inp["q"], inp["k"], inp["v"], inp["rho"],
                                             inp["gate"])
    grads = plx.prefill_backward(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"], out,
                                 corr, lse, rbar, dout)
    torch.cuda.synchronize()
    return (out, lse, rbar, corr), grads


SHAPES = [(1, 1, 1), (1, 2, 31), (1, 1, 33), (2, 1, 64), (1, 2, 65), (1, 1, 130), (2, 2, 200),
          (1, 1, 511)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,L", SHAPES)
def test_train_statistics(B, H, L, d):
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=900 + L + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    plx = _plx()
    out, lse, rbar, corr = plx.prefill_train(inp["q"], inp["k"], inp["v"], inp["rho"],
                                             inp["gate"])
    plain = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, plain)          # the same forward kernel, plus side outputs
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_train(h["q"], h["k"], h["v"], h["rho"], h["gate"])
    errs = {n: float(np.max(np.abs(_np(t) - ref[n])))
            for n, t in (("out", out), ("lse", lse), ("rbar", rbar), ("corr", corr))}
    print(f"train B{B} H{H} L{L} d{d}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    assert errs["out"] <= 2e-2 and errs["rbar"] <= 2e-2 and errs["corr"] <= 2e-2
    assert errs["lse"] <= 1e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,L", SHAPES)
def test_backward_shapes(B, H, L, d):
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=950 + L + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    dout = _dout((B, H, L, d), 960 + L)
    _, grads = _run(inp, dout)
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_backward(h["q"], h["k"], h["v"], h["rho"], h["gate"], dout.cpu())
    errs = {n: _rel_err(_np(t), ref[n]) for n, t in zip(GRADS, grads[:4])}
    errs["dgate"] = _rel_err(_np(grads[4]), ref["dgate"])
    print(f"backward B{B} H{H} L{L} d{d}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= 2e-2, n


def test_backward_gate_zero_and_rho_zero():
    """gate = 0 leaves softmax attention: drho is exactly zero; with rho = 0 the
    gate gets no gradient.  Both against the oracle as well."""
    inp = wl.prefill_inputs(1, 2, 150, 128, "bf16", seed=970, device="cuda", rho_std=0.5)
    dout = _dout((1, 2, 150, 128), 971)
    inp["gate"].zero_()
    _, grads = _run(inp, dout)
    assert float(grads[3].abs().max()) == 0.0
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_backward(h["q"], h["k"], h["v"], h["rho"], h["gate"], dout.cpu())
    for n, t in zip(GRADS, grads[:4]):
        assert _rel_err(_np(t), ref[n]) <= 2e-2, n
    inp["gate"].fill_(0.7)
    inp["rho"].zero_()
    _, grads = _run(inp, dout)
    assert float(grads[4].abs().max()) == 0.0


def test_backward_deterministic():
    inp = wl.prefill_inputs(2, 2, 300, 128, "bf16", seed=972, device="cuda", rho_std=0.5)
    dout = _dout((2, 2, 300, 128), 973)
    _, a = _run(inp, dout)
    a = [t.clone() for t in a]
    _, b = _run(inp, dout)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


_FULL = {}


def _full_backward(wid):
    """Gradients of a full-size bf16 workload in the benchmark's launch
    configuration, with fp64 host copies of the inputs, made once per session."""
    if wid not in _FULL:
        _FULL.clear()
        torch.cuda.empty_cache()
        w = wl.WORKLOADS[wid]
        inp = wl.make_workload(wid, device="cuda")
        dout = _dout((w.B, w.H, w.L, w.d), 980 + wid)
        _, grads = _run(inp, dout)
        for t in grads:
            assert bool(torch.isfinite(t).all())
        _FULL[wid] = dict(
            h={n: inp[n].double().cpu().numpy() for n in ("q", "k", "v", "rho", "gate")},
            dout=dout.double().cpu().numpy(),
            grads=[t.cpu().numpy() for t in grads])
        del inp, dout, grads
        torch.cuda.empty_cache()
    return _FULL[wid]


def _check_heads(wid, heads, check_dgate=()):
    """Every gradient element of the given (b, h) heads against the oracle, and
    dgate[h] (summed over the batch) for the heads h in check_dgate, whose every
    batch entry must be among `heads`."""
    w = wl.WORKLOADS[wid]
    st = _full_backward(wid)
    h, grads = st["h"], st["grads"]
    worst = {n: 0.0 for n in GRADS}
    dg = {hh: 0.0 for hh in check_dgate}
    for b, hh in heads:
        ref = po.prefill_head_backward(h["q"][b, hh], h["k"][b, hh], h["v"][b, hh],
                                       h["rho"][b, hh], float(h["gate"][hh]), w.scale,
                                       st["dout"][b, hh])
        errs = {n: _rel_err(t[b, hh], r) for n, t, r in zip(GRADS, grads[:4], ref[:4])}
        for n, e in errs.items():
            worst[n] = max(worst[n], e)
        if hh in dg:
            dg[hh] += ref[4]
        print(f"workload {wid} head ({b},{hh}): " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
              flush=True)
    for n, e in worst.items():
        assert e <= 2e-2, n
    for hh, ref in dg.items():
        e = abs(float(grads[4][hh]) - ref) / max(1.0, abs(ref))
        print(f"workload {wid} dgate[{hh}]: {float(grads[4][hh]):.6e} vs {ref:.6e} (rel {e:.2e})",
              flush=True)
        assert e <= 2e-2


@pytest.mark.parametrize("part", range(4))
def test_backward_workload2_every_head(part):
    """Workload 2 (B4 H16 L4096 d128): every gradient element of all 64 heads and
    dgate of every head, four heads (all batch entries) per test."""
    w = wl.WORKLOADS[2]
    hs = range(4 * part, 4 * part + 4)
    _check_heads(2, [(b, hh) for hh in hs for b in range(w.B)], check_dgate=hs)


@pytest.mark.parametrize("part", range(8))
def test_backward_workload5_every_head(part):
    """Workload 5 (B2 H32 L16384 d64, duplicated key runs): every gradient element
    of all 64 heads, eight per test (about 2 s of oracle time per head on 16
    cores), and dgate of the four heads whose both batch entries a test holds."""
    w = wl.WORKLOADS[5]
    hs = range(4 * part, 4 * part + 4)
    _check_heads(5, [(b, hh) for hh in hs for b in range(w.B)], check_dgate=hs)


def test_autograd_function_matches_the_oracle():
    """torch autograd through parallax_attention: a loss on the output flows to
    q, k, v, rho (bf16) and the gate (fp32), matching the oracle's gradients of
    the same loss.  The op after the attention is affine, so the upstream
    gradient (2 w) is known without the GPU's output."""
    plx = _plx()
    B, H, L, d = 1, 2, 97, 64
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=990, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    leaves = {n: inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "rho", "gate")}
    w = _dout((B, H, L, d), 991)
    out = plx.parallax_attention(leaves["q"], leaves["k"], leaves["v"], leaves["rho"],
                                 leaves["gate"])
    loss = ((2.0 * out + 3.0) * w).sum()
    loss.backward()
    torch.cuda.synchronize()
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_backward(h["q"], h["k"], h["v"], h["rho"], h["gate"], 2.0 * w.cpu())
    for n, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("rho", "drho"), ("gate", "dgate")):
        g = leaves[n].grad
        assert g is not None and g.dtype == leaves[n].dtype, n
        assert _rel_err(_np(g), ref[key]) <= 2e-2, n


@pytest.mark.parametrize("d", [64, 128])
def test_backward_partial_head_group(d):
    """The backward kernels run heads in groups (32 at d=128, 16 at d=64):
    B*H = 40 leaves a partial last group at both sizes."""
    B, H, L = 2, 20, 96
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=995 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    dout = _dout((B, H, L, d), 996 + d)
    _, grads = _run(inp, dout)
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_backward(h["q"], h["k"], h["v"], h["rho"], h["gate"], dout.cpu())
    errs = {n: _rel_err(_np(t), ref[n]) for n, t in zip(GRADS, grads[:4])}
    errs["dgate"] = _rel_err(_np(grads[4]), ref["dgate"])
    print(f"backward partial group d{d}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= 2e-2, n


@pytest.mark.parametrize("d", [64, 128])
def test_backward_many_heads(d):
    """The widest backward grids: 4096 heads (B64 H64) of 100 rows, every
    gradient element and dgate (summed over 64 batch entries) against the
    oracle."""
    B, H, L = 64, 64, 100
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=1700 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    dout = _dout((B, H, L, d), 1800 + d)
    _, grads = _run(inp, dout)
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_backward(h["q"], h["k"], h["v"], h["rho"], h["gate"], dout.cpu())
    errs = {n: _rel_err(_np(t), ref[n]) for n, t in zip(GRADS, grads[:4])}
    errs["dgate"] = _rel_err(_np(grads[4]), ref["dgate"])
    print(f"backward 4096 heads d{d}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= 2e-2, n


@pytest.mark.parametrize("d,L", [(128, 32768), (64, 65536)])
def test_backward_long_sequence(d, L):
    """One head of 32768 (d=128) or 65536 (d=64) rows: 256 or 1024 key blocks
    of the key-stationary grid and the longest query-stationary rows, every
    gradient element against the oracle."""
    inp = wl.prefill_inputs(1, 1, L, d, "bf16", seed=1900 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    dout = _dout((1, 1, L, d), 2000 + d)
    _, grads = _run(inp, dout)
    for t in grads:
        assert bool(torch.isfinite(t).all())
    h = {n: inp[n].double().cpu().numpy() for n in ("q", "k", "v", "rho", "gate")}
    ref = po.prefill_head_backward(h["q"][0, 0], h["k"][0, 0], h["v"][0, 0], h["rho"][0, 0],
                                   float(h["gate"][0]), d ** -0.5,
                                   dout[0, 0].double().cpu().numpy())
    errs = {n: _rel_err(_np(t[0, 0]), r) for n, t, r in zip(GRADS, grads[:4], ref[:4])}
    errs["dgate"] = abs(float(grads[4][0]) - ref[4]) / max(1.0, abs(ref[4]))
    print(f"backward L{L} d{d}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= 2e-2, n


@pytest.mark.parametrize("seed", range(6))
def test_backward_random_shapes(seed):
    """Seeded random shapes: B 1-2, H 1-36 (partial head groups), L 1-260, d 64
    or 128; every gradient against the oracle."""
    rng = np.random.default_rng(2300 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 37))
    L = int(rng.integers(1, 261))
    d = int(rng.choice([64, 128]))
    if B * H * L > 4000:
        L = max(1, 4000 // (B * H))
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=2400 + seed, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    dout = _dout((B, H, L, d), 2500 + seed)
    _, grads = _run(inp, dout)
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill_backward(h["q"], h["k"], h["v"], h["rho"], h["gate"], dout.cpu())
    errs = {n: _rel_err(_np(t), ref[n]) for n, t in zip(GRADS, grads[:4])}
    errs["dgate"] = _rel_err(_np(grads[4]), ref["dgate"])
    print(f"random {seed}: B{B} H{H} L{L} d{d}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= 2e-2, n
