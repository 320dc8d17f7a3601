"""GPU parity of the split-KV decode path against the fp64 CPU oracle."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import parallax_oracle as po

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
U = 2.0 ** -24          # fp32 unit roundoff


def _gamma(n):
    return n * U / (1.0 - n * U)


def decode_error_bound(q, K, V, rho, g, scale, C, ns, dtype):
    """First-order bound on the rounding error of one decode stream, computed in
    fp64 from its exact inputs.  The decode keeps P, R and every sum in fp32, so
    the error comes from fp32 rounding only:
      * sums: with n the longest chain of dependent fp32 additions (the keys a
        lane group accumulates, its rescales, the merge of the lane groups in a
        split, the split merge), the sums of p v, p r v, p, p r carry at most
        gamma_n times the sums of their absolute terms;
      * scores and probe products: a dot product of nd steps (per-lane dot2 /
        fma chain plus the DPP tree) is off by gamma_nd sum_f |q_f k_jf|, which
        with the fma and exp2 roundings perturbs each weight by a relative eps_j;
        the output moves by the weighted spread of those perturbations;
      * the output formula adds a few roundings of its terms.
    Returns the bound per feature [d_v]."""
    q, K, V, rho = (np.asarray(x, dtype=np.float64) for x in (q, K, V, rho))
    n = K.shape[0]
    d = K.shape[1]
    epl = 8 if dtype == "bf16" else 4        # elements per 16-byte lane load
    lpr = d // epl                           # lanes per key row
    kpw = 64 // lpr                          # rows per wave load
    ng = 4 * kpw                             # lane groups per split workgroup
    chunk = kpw * 16
    nsg = 256 // ((2 * d) // 4)              # split groups of the combine
    n_sum = (-(-C // ng) + -(-C // (4 * chunk)) + ng + -(-ns // nsg) + nsg + 8)
    n_dot = epl // (2 if dtype == "bf16" else 1) + int(np.log2(lpr)) + 2
    s = scale * (K @ q)
    r = K @ rho
    m = s.max()
    e = np.exp(s - m)
    w = e / e.sum()
    o_sa = w @ V
    rbar = float(w @ r)
    dv = np.abs(V - o_sa)
    u_ = (w * r) @ V
    corr = u_ - o_sa * rbar
    a1 = w @ np.abs(V)
    a2 = (w * np.abs(r)) @ np.abs(V)
    a3 = float(w @ np.abs(r))
    term_sum = 2.0 * _gamma(n_sum) * (a1 + g * a2 + g * np.abs(o_sa) * a3)
    ln2, l2e = np.log(2.0), 1.0 / np.log(2.0)
    eps = (ln2 * scale * l2e * _gamma(n_dot) * (np.abs(K) @ np.abs(q))
           + 2 * ln2 * U * np.abs((s - m) * l2e) + 14 * U)
    term_w = 2.0 * ((w * eps) @ dv + g * ((w * eps * np.abs(r - rbar)) @ dv
                                          + float(w @ eps) * np.abs(corr)))
    term_r = 2.0 * g * ((w * _gamma(n_dot) * (np.abs(K) @ np.abs(rho))) @ dv)
    term_out = 4 * U * (np.abs(o_sa) + g * np.abs(u_) + g * np.abs(o_sa) * abs(rbar))
    return term_sum + term_w + term_r + term_out + 1e-30


def _check_streams(out, inp, streams, C, dtype, label):
    """Every listed stream against the oracle, element by element: within the
    2e-2 (bf16) / 1e-4 (fp32) tolerance and within its own rounding bound.
    Returns (max error, max error / bound)."""
    H = inp["q"].shape[1]
    Lmax = inp["kcache"].shape[2]
    d = inp["q"].shape[2]
    scale = 1.0 / np.sqrt(d)
    sl = [int(x) for x in inp["seqlens"].tolist()]
    gate = inp["gate"].detach().cpu().double().numpy()
    worst, ratio = 0.0, 0.0
    for b, h in streams:
        n = min(max(sl[b], 0), Lmax)
        K = _host(inp["kcache"][b, h, :n]).double().numpy()
        V = _host(inp["vcache"][b, h, :n]).double().numpy()
        q = _host(inp["q"][b, h]).double().numpy()
        r = _host(inp["rho"][b, h]).double().numpy()
        ref = po.decode_stream(q, K, V, r, float(gate[h]), scale)
        err = np.abs(out[b, h] - ref)
        worst = max(worst, float(err.max()))
        if n > 0:
            bnd = decode_error_bound(q, K, V, r, float(gate[h]), scale, C, -(-n // C), dtype)
            ratio = max(ratio, float((err / bnd).max()))
            assert np.all(err <= bnd), (label, b, h, float(err.max()), float(bnd.min()))
        else:
            assert np.all(out[b, h] == 0.0)
    print(f"{label}: {len(streams)} streams, max-abs {worst:.3e}, max error/bound {ratio:.3f}",
          flush=True)
    assert worst <= TOL[dtype]
    return worst, ratio


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
        C = split if split else _plx().decode_default_split(B, H, Lmax, d)
        _check_streams(out, inp, [(b, h) for b in range(B) for h in range(H)], C, dtype,
                       f"decode {dtype} {case} d{d} split {split}")


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


def _bench_split(w):
    return _plx().decode_default_split(w.B, w.H, w.Lmax, w.d)


def test_workload3_full():
    """64 x 16 streams of 8192 keys, in the benchmark's launch configuration
    (the library's split); every element of every stream is checked against the
    oracle, within 2e-2 and within the stream's own fp32 rounding bound (about
    1e-5 here, so one key dropped or counted twice, about 1e-4, fails)."""
    w = wl.WORKLOADS[3]
    inp = wl.make_workload(3, device="cuda")
    out = _host(_run(inp)).double().numpy()
    _check_streams(out, inp, [(b, h) for b in range(w.B) for h in range(w.H)],
                   _bench_split(w), "bf16", "workload 3")


def test_workload4_full():
    """Long ragged decode (65536..131072 keys, up to 64 splits per stream) in the
    benchmark's launch configuration: all 128 streams, every element, within
    2e-2 and within each stream's rounding bound."""
    w = wl.WORKLOADS[4]
    inp = wl.make_workload(4, device="cuda")
    out = _host(_run(inp)).double().numpy()
    assert np.isfinite(out).all()
    _check_streams(out, inp, [(b, h) for b in range(w.B) for h in range(w.H)],
                   _bench_split(w), "bf16", "workload 4")


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
    C = split if split else _plx().decode_default_split(B, H, Lmax, d)
    _check_streams(_host(out).double().numpy(), inp,
                   [(b, h) for b in range(B) for h in range(H)], C, dtype, f"random {seed}")
