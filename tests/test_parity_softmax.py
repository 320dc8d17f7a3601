"""GPU parity of the softmax-only entry points against the fp64 CPU oracle.

The softmax baseline is the Parallax forward pass with the correction branch
compiled out, so its exact result is the oracle with rho = 0 (page "Parallax -
Parameterized Local Linear Attention for Language Modeling", section
"Significance": a zero probe projection gives back ordinary softmax attention).
Beyond the oracle comparison, the baseline must agree bit for bit with the
Parallax kernels run on rho = 0: with a zero probe every correction term is an
exact zero, and both variants share the softmax arithmetic instruction for
instruction, so any difference would mean the switch changed more than it
should.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import parallax_oracle as po

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _plx():
    import parallax_local_linear_amd as plx
    return plx


def _host(x):
    return x.detach().cpu()


def _maxerr(a, b):
    return float(np.max(np.abs(a - b)))


def _oracle_prefill(inp):
    h = {k: _host(v) for k, v in inp.items()}
    return po.prefill(h["q"], h["k"], h["v"], torch.zeros_like(h["rho"]), h["gate"])


SHAPES = [(1, 1, 1), (1, 2, 63), (2, 1, 65), (1, 1, 128), (1, 2, 129), (2, 2, 1000)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,L", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_prefill_shapes(dtype, B, H, L, d):
    plx = _plx()
    inp = wl.prefill_inputs(B, H, L, d, dtype, seed=800 + L + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = plx.softmax_prefill(inp["q"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    err = _maxerr(_host(out).double().numpy(), _oracle_prefill(inp))
    print(f"softmax prefill {dtype} B{B} H{H} L{L} d{d}: max-abs {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    zero = torch.zeros_like(inp["rho"])
    same = plx.prefill(inp["q"], inp["k"], inp["v"], zero, inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, same)


def test_softmax_prefill_is_sdpa():
    """Against torch's causal scaled-dot-product attention in fp64 on the CPU."""
    inp = wl.prefill_inputs(2, 2, 300, 128, "bf16", seed=810, device="cuda")
    out = _plx().softmax_prefill(inp["q"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    h = {k: _host(inp[k]).double() for k in ("q", "k", "v")}
    ref = torch.nn.functional.scaled_dot_product_attention(h["q"], h["k"], h["v"],
                                                           is_causal=True).numpy()
    assert _maxerr(_host(out).double().numpy(), ref) <= TOL["bf16"]


def test_softmax_stages_match_single_call():
    plx = _plx()
    inp = wl.prefill_inputs(2, 3, 333, 64, "bf16", seed=811, device="cuda")
    a = plx.softmax_prefill(inp["q"], inp["k"], inp["v"])
    vt = plx.prefill_stage_v(inp["v"])
    b = plx.softmax_prefill_attend(inp["q"], inp["k"], vt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_softmax_prefill_workload2_sampled():
    """The benchmark's prefill workload (B4 H16 L4096 d128, bf16) through the
    softmax baseline: every row of two heads, and the bit-identity with the
    Parallax kernel on rho = 0 over the whole output."""
    w = wl.WORKLOADS[2]
    inp = wl.make_workload(2, device="cuda")
    plx = _plx()
    out = plx.softmax_prefill(inp["q"], inp["k"], inp["v"])
    same = plx.prefill(inp["q"], inp["k"], inp["v"], torch.zeros_like(inp["rho"]), inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, same)
    worst = 0.0
    for b, hh in [(0, 0), (w.B - 1, w.H - 1)]:
        hq = {k: _host(inp[k][b, hh]).double().numpy() for k in ("q", "k", "v")}
        ref = po.prefill_head(hq["q"], hq["k"], hq["v"], np.zeros_like(hq["q"]), 1.0, w.scale)
        worst = max(worst, _maxerr(_host(out[b, hh]).double().numpy(), ref))
    print(f"softmax prefill workload 2: worst max-abs {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]


DECODE_CASES = [  # B, H, Lmax, seqlens
    (1, 1, 1, [1]),
    (3, 2, 300, [300, 1, 0]),
    (2, 3, 1000, [999, 513]),
    (4, 1, 4100, [4100, 4096, 65, 2049]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}L{c[2]}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_decode_cases(dtype, case, d):
    plx = _plx()
    B, H, Lmax, sl = case
    inp = wl.decode_inputs(B, H, Lmax, d, dtype, seed=820 + Lmax + d, device="cuda",
                           rho_std=0.5, gate=("uniform", 0.2, 1.0), seqlens=sl)
    h = {k: _host(v) for k, v in inp.items()}
    ref = po.decode(h["q"], h["kcache"], h["vcache"], torch.zeros_like(h["rho"]), h["gate"],
                    h["seqlens"])
    zero = torch.zeros_like(inp["rho"])
    for split in (0, 64, 256):
        out = plx.softmax_decode(inp["q"], inp["kcache"], inp["vcache"], inp["seqlens"],
                                 split_keys=split)
        same = plx.decode(inp["q"], inp["kcache"], inp["vcache"], zero, inp["gate"],
                          inp["seqlens"], split_keys=split)
        torch.cuda.synchronize()
        got = _host(out).double().numpy()
        err = _maxerr(got, ref)
        print(f"softmax decode {dtype} {case} d{d} split {split}: max-abs {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        assert torch.equal(out, same)
        assert all(np.all(got[b] == 0.0) for b in range(B) if sl[b] == 0)


def test_softmax_decode_workload3_sampled():
    """The benchmark's decode workload (B64 H16, 8192 cached keys, d128, bf16):
    sampled streams against the oracle, all streams against the Parallax kernels
    on rho = 0."""
    w = wl.WORKLOADS[3]
    inp = wl.make_workload(3, device="cuda")
    plx = _plx()
    out = plx.softmax_decode(inp["q"], inp["kcache"], inp["vcache"], inp["seqlens"])
    same = plx.decode(inp["q"], inp["kcache"], inp["vcache"], torch.zeros_like(inp["rho"]),
                      inp["gate"], inp["seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(out, same)
    streams = [(0, 0), (17, 5), (w.B - 1, w.H - 1)]
    h = {k: _host(inp[k]) for k in ("q", "kcache", "vcache", "rho", "gate", "seqlens")}
    ref = po.decode(h["q"], h["kcache"], h["vcache"], torch.zeros_like(h["rho"]), h["gate"],
                    h["seqlens"], streams=streams)
    got = _host(out).double().numpy()
    err = max(_maxerr(got[b, hh], ref[b, hh]) for b, hh in streams)
    print(f"softmax decode workload 3: max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
