"""GPU parity of the split-KV decode path against the fp64 CPU oracle."""
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


def _run(inp, split_keys=0):
    out = _plx().decode(inp["q"], inp["kcache"], inp["vcache"], inp["rho"], inp["gate"],
                        inp["seqlens"], split_keys=split_keys)
    torch.cuda.synchronize()
    return out


def _oracle(inp, streams=None):
    h = {k: _host(v) for k, v in inp.items()}
    return po.decode(h["q"], h["kcache"], h["vcache"], h["rho"], h["gate"], h["seqlens"],
                     streams=streams)


def _maxerr(a, b):
    return float(np.max(np.abs(a - b)))


CASES = [  # B, H, Lmax, seqlens
    (1, 1, 1, [1]),
    (2, 2, 64, [64, 3]),
    (3, 2, 300, [300, 1, 0]),
    (2, 3, 1000, [999, 513]),
    (4, 1, 4100, [4100, 4096, 65, 2049]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}L{c[2]}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_cases(dtype, case, d):
    B, H, Lmax, sl = case
    inp = wl.decode_inputs(B, H, Lmax, d, dtype, seed=200 + Lmax + d, device="cuda",
                           rho_std=0.5, gate=("uniform", 0.2, 1.0), seqlens=sl)
    for split in (0, 64, 256):
        out = _host(_run(inp, split)).double().numpy()
        ref = _oracle(inp)
        err = _maxerr(out, ref)
        print(f"decode {dtype} {case} d{d} split {split}: max-abs {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        zero = [b for b in range(B) if sl[b] == 0]
        assert all(np.all(out[b] == 0.0) for b in zero)


def test_split_invariance():
    inp = wl.decode_inputs(2, 4, 5000, 128, "bf16", seed=21, device="cuda", rho_std=1.0,
                           seqlens=[5000, 3333])
    outs = [_run(inp, s) for s in (64, 192, 1024, 4096, 8192)]
    for o in outs[1:]:
        assert torch.allclose(o, outs[0], rtol=0, atol=2e-5)


def test_cache_past_length_is_never_read():
    inp = wl.decode_inputs(3, 2, 777, 128, "bf16", seed=22, device="cuda",
                           seqlens=[777, 500, 129])
    a = _run(inp).clone()
    for b, n in enumerate([777, 500, 129]):
        inp["kcache"][b, :, n:] = float("nan")
        inp["vcache"][b, :, n:] = float("nan")
    b_ = _run(inp)
    assert torch.isfinite(b_).all()
    assert torch.equal(a, b_)


def test_decode_matches_prefill_row():
    plx = _plx()
    pin = wl.prefill_inputs(1, 2, 257, 128, "bf16", seed=23, device="cuda", rho_std=0.5)
    pre = plx.prefill(pin["q"], pin["k"], pin["v"], pin["rho"], pin["gate"])
    for i in (0, 100, 256):
        sl = torch.tensor([i + 1], dtype=torch.int32, device="cuda")
        out = plx.decode(pin["q"][:, :, i].contiguous(), pin["k"], pin["v"],
                         pin["rho"][:, :, i].contiguous(), pin["gate"], sl)
        torch.cuda.synchronize()
        assert (out - pre[:, :, i]).abs().max().item() <= TOL["bf16"]


def test_stages_match_single_call():
    plx = _plx()
    inp = wl.decode_inputs(2, 2, 3000, 64, "bf16", seed=24, device="cuda",
                           seqlens=[3000, 1234])
    a = _run(inp, 512)
    part = plx.decode_partials(inp["q"], inp["kcache"], inp["vcache"], inp["rho"],
                               inp["seqlens"], 512)
    b = plx.decode_combine(part, inp["gate"], inp["seqlens"], 3000, 512)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_workload3_full():
    """64 x 16 streams of 8192 keys, in the benchmark's launch configuration;
    every stream is checked against the oracle."""
    inp = wl.make_workload(3, device="cuda")
    out = _host(_run(inp)).double().numpy()
    ref = _oracle(inp)
    err = _maxerr(out, ref)
    print(f"workload 3: max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_workload4_sampled():
    """Long ragged decode (65536..131072 keys): 24 sampled streams."""
    inp = wl.make_workload(4, device="cuda")
    out = _host(_run(inp)).double().numpy()
    rng = np.random.default_rng(4)
    streams = [(b, int(rng.integers(0, 16))) for b in range(8)]
    streams += [(int(rng.integers(0, 8)), int(rng.integers(0, 16))) for _ in range(16)]
    streams = sorted(set(streams))
    ref = _oracle(inp, streams=streams)
    err = max(_maxerr(out[b, h], ref[b, h]) for b, h in streams)
    print(f"workload 4 ({len(streams)} streams): max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert np.isfinite(out).all()


def test_widest_grid():
    """B*H = 65535 streams, the largest second grid dimension the decode launch
    uses; sampled streams against the oracle."""
    B, H, Lmax, d = 65535, 1, 64, 64
    rng = np.random.default_rng(36)
    sl = rng.integers(0, Lmax + 1, B).tolist()
    inp = wl.decode_inputs(B, H, Lmax, d, "bf16", seed=36, device="cuda", seqlens=sl)
    out = _host(_run(inp)).double().numpy()
    streams = [0, 1, 2, 32767, 65533, 65534]
    h = {k: _host(v) for k, v in inp.items()}
    ref = po.decode(h["q"], h["kcache"], h["vcache"], h["rho"], h["gate"], h["seqlens"],
                    streams=[(b, 0) for b in streams])
    err = max(_maxerr(out[b, 0], ref[b, 0]) for b in streams)
    print(f"decode B*H=65535: max-abs over sampled streams {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("seed", range(8))
def test_decode_random_shapes(seed):
    """Seeded random shapes: B 1-6, H 1-8, Lmax 1-5000 with ragged lengths
    (including 0 and Lmax), d 64 or 128, bf16 or fp32, the library's split or a
    random multiple of 64; every stream against the oracle."""
    rng = np.random.default_rng(2600 + seed)
    B, H = int(rng.integers(1, 7)), int(rng.integers(1, 9))
    Lmax = int(rng.integers(1, 5001))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if seed % 4 == 1 else "bf16"
    lens = [int(x) for x in rng.integers(0, Lmax + 1, B)]
    lens[0] = Lmax
    if B > 1:
        lens[-1] = 0
    split = 0 if seed % 2 == 0 else 64 * int(rng.integers(1, 33))
    inp = wl.decode_inputs(B, H, Lmax, d, dtype, seed=2700 + seed, device="cuda",
                           rho_std=0.5, seqlens=lens)
    out = _run(inp, split_keys=split)
    err = _maxerr(_host(out).double().numpy(), _oracle(inp))
    print(f"random {seed}: {dtype} B{B} H{H} Lmax{Lmax} d{d} lens{lens} split {split}: "
          f"max-abs {err:.3e}", flush=True)
    assert err <= TOL[dtype]
