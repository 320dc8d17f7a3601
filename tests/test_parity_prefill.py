"""GPU parity of the prefill path against the fp64 CPU oracle.

Tolerances (max-abs over every compared element): 1e-4 for fp32 inputs and
2e-2 for bf16 inputs with fp32 accumulation; outputs are fp32.
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


def _run(inp):
    plx = _plx()
    out = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    return _host(out).double().numpy()


def _oracle_all(inp):
    h = {k: _host(v) for k, v in inp.items()}
    return po.prefill(h["q"], h["k"], h["v"], h["rho"], h["gate"])


def _maxerr(a, b):
    return float(np.max(np.abs(a - b)))


def test_native_library_is_loaded():
    plx = _plx()
    import parallax_local_linear_amd._native as nat
    assert plx.lib()._name == nat.LIB_PATH


def test_workload1_fp32_full():
    inp = wl.make_workload(1, device="cuda")
    out = _run(inp)
    ref = _oracle_all(inp)
    err = _maxerr(out, ref)
    print(f"workload 1 fp32 max-abs {err:.3e}", flush=True)
    assert err <= TOL["f32"]
    h = {k: _host(v) for k, v in inp.items()}
    ex = po.prefill_explicit(h["q"], h["k"], h["v"], h["rho"], h["gate"])
    assert _maxerr(out, ex) <= TOL["f32"]


SHAPES = [(1, 1, 1), (1, 1, 2), (1, 2, 63), (1, 1, 64), (2, 1, 65), (1, 1, 127),
          (1, 1, 128), (1, 2, 129), (1, 1, 255), (2, 2, 1000)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,L", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_shapes(dtype, B, H, L, d):
    inp = wl.prefill_inputs(B, H, L, d, dtype, seed=100 + L + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = _run(inp)
    ref = _oracle_all(inp)
    err = _maxerr(out, ref)
    print(f"prefill {dtype} B{B} H{H} L{L} d{d}: max-abs {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_first_row_is_v0_exactly(dtype):
    """A query that attends one key returns that key's value exactly."""
    inp = wl.prefill_inputs(2, 3, 130, 128, dtype, seed=7, device="cuda", rho_std=2.0)
    out = _plx().prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 0].cpu(), inp["v"][:, :, 0].float().cpu())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rho_zero_is_softmax_attention(dtype):
    inp = wl.prefill_inputs(1, 2, 300, 64, dtype, seed=8, device="cuda")
    inp["rho"].zero_()
    out = _run(inp)
    h = {k: _host(v).double() for k, v in inp.items()}
    ref = torch.nn.functional.scaled_dot_product_attention(h["q"], h["k"], h["v"],
                                                           is_causal=True).numpy()
    assert _maxerr(out, ref) <= TOL[dtype] / 4


def test_identical_keys_give_uniform_average():
    inp = wl.prefill_inputs(1, 1, 200, 128, "bf16", seed=9, device="cuda", rho_std=1.0)
    inp["k"].copy_(inp["k"][:, :, :1].expand_as(inp["k"]))
    out = _run(inp)
    v = _host(inp["v"]).double().numpy()
    ref = np.cumsum(v, axis=2) / np.arange(1, 201)[None, None, :, None]
    assert _maxerr(out, ref) <= TOL["bf16"]


def test_deterministic():
    inp = wl.prefill_inputs(1, 4, 700, 128, "bf16", seed=10, device="cuda")
    plx = _plx()
    a = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"]).clone()
    b = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_stages_match_single_call():
    plx = _plx()
    inp = wl.prefill_inputs(2, 2, 333, 64, "bf16", seed=11, device="cuda")
    a = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    vt = plx.prefill_stage_v(inp["v"])
    b = plx.prefill_attend(inp["q"], inp["k"], vt, inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _sample_rows(L, rng, n_rand=24):
    rows = {0, 1, 2, 3, L - 1}
    rows.update(int(x) for x in rng.integers(0, L, n_rand))
    return sorted(rows)


@pytest.mark.parametrize("wid", [2, 5])
def test_full_workload_sampled(wid):
    """The full-size bf16 workloads, in the launch configuration the benchmark
    times: every row of two heads by the expanded form, and sampled rows of
    further heads by the explicit covariance form."""
    w = wl.WORKLOADS[wid]
    inp = wl.make_workload(wid, device="cuda")
    plx = _plx()
    out = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(wid)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    worst = 0.0
    for b, h in heads:
        hq = {k: _host(inp[k][b, h]).double().numpy() for k in ("q", "k", "v", "rho")}
        g = float(inp["gate"][h])
        ref = po.prefill_head(hq["q"], hq["k"], hq["v"], hq["rho"], g, w.scale)
        err = _maxerr(_host(out[b, h]).double().numpy(), ref)
        worst = max(worst, err)
        print(f"workload {wid} head ({b},{h}) all rows: max-abs {err:.3e}", flush=True)
    hcpu = {k: _host(inp[k]) for k in ("q", "k", "v", "rho", "gate")}
    for _ in range(6):
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.H))
        rows = _sample_rows(w.L, rng)
        ref = po.prefill_rows(hcpu["q"], hcpu["k"], hcpu["v"], hcpu["rho"], hcpu["gate"], b, h,
                              rows, scale=w.scale)
        got = _host(out[b, h, rows]).double().numpy()
        err = _maxerr(got, ref)
        worst = max(worst, err)
    print(f"workload {wid}: worst max-abs {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]


def test_workload2_every_head():
    """The benchmark's prefill workload (B4 H16 L4096 d128, bf16) compared with the
    expanded-form oracle on every output element of all 64 heads."""
    w = wl.WORKLOADS[2]
    inp = wl.make_workload(2, device="cuda")
    out = _plx().prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    got = _host(out).double().numpy()
    h = {k: _host(inp[k]).double().numpy() for k in ("q", "k", "v", "rho", "gate")}
    worst = 0.0
    for b in range(w.B):
        for hh in range(w.H):
            ref = po.prefill_head(h["q"][b, hh], h["k"][b, hh], h["v"][b, hh], h["rho"][b, hh],
                                  float(h["gate"][hh]), w.scale)
            worst = max(worst, _maxerr(got[b, hh], ref))
        print(f"workload 2: {(b + 1) * w.H} of {w.B * w.H} heads, worst max-abs {worst:.3e}",
              flush=True)
    assert worst <= TOL["bf16"]


_W5 = {}


def _workload5():
    """Workload 5 (B2 H32 L16384 d64, duplicated key runs), its GPU output in the
    benchmark's launch configuration and fp64 host copies, made once per session."""
    if not _W5:
        inp = wl.make_workload(5, device="cuda")
        out = _plx().prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        _W5["out"] = _host(out).double().numpy()
        _W5["h"] = {k: _host(inp[k]).double().numpy() for k in ("q", "k", "v", "rho", "gate")}
        del inp, out
        torch.cuda.empty_cache()
    return _W5


@pytest.mark.parametrize("part", range(8))
def test_workload5_every_head(part):
    """Workload 5 compared with the expanded-form oracle on every output element
    of all 64 heads, eight heads per test (about 3 s of oracle time per head)."""
    w = wl.WORKLOADS[5]
    st = _workload5()
    h, got = st["h"], st["out"]
    worst = 0.0
    for idx in range(8 * part, 8 * part + 8):
        b, hh = divmod(idx, w.H)
        ref = po.prefill_head(h["q"][b, hh], h["k"][b, hh], h["v"][b, hh], h["rho"][b, hh],
                              float(h["gate"][hh]), w.scale)
        err = _maxerr(got[b, hh], ref)
        worst = max(worst, err)
        print(f"workload 5 head ({b},{hh}): max-abs {err:.3e}", flush=True)
    assert worst <= TOL["bf16"]


def _row_bound(q, k, v, rho, g, scale, base):
    """Rounding bound of each prefill row of one head when rho is large: the
    fp16 roundings of P, R (after the row's power-of-two scale) and T = P*R
    each carry a relative error of at most 2^-11 (four roundings with the
    weight normalisation), so the correction sum_j w_j r_j v_j - o_sa sum_j w_j r_j
    moves by at most 4 * 2^-11 * g * (sum_j w_j |r_j| |v_j| + sum_j w_j |r_j|
    sum_j w_j |v_j|), plus the bf16-path bound for the rest."""
    L = q.shape[0]
    S = scale * (q @ k.T)
    S = np.where(np.tril(np.ones((L, L), bool)), S, -np.inf)
    W = np.exp(S - S.max(1, keepdims=True))
    W /= W.sum(1, keepdims=True)
    R = np.abs(rho @ k.T)
    a = (W * R) @ np.abs(v) + (W * R).sum(1, keepdims=True) * (W @ np.abs(v))
    return base + 4 * 2.0 ** -11 * g * a


@pytest.mark.parametrize("d", [64, 128])
def test_large_rho_is_rescaled_exactly(d):
    """|<rho,k>| up to about 1e5 (far past what fp16 T = P*R holds unscaled):
    the kernel scales each such row by a power of two and unscales it in fp32.
    Every row must be finite and within its rounding bound of the oracle."""
    B, H, L = 1, 3, 300
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=760 + d, device="cuda", rho_std=1.0,
                            gate=("uniform", 0.2, 1.0))
    # heads 0, 1, 2: |r| up to about 1e5, 4e3 and 1e2
    for hh, std in enumerate((2.2e4 / d ** 0.5, 900.0 / d ** 0.5, 22.0 / d ** 0.5)):
        inp["rho"][:, hh] = (inp["rho"][:, hh].float() * std).to(torch.bfloat16)
    out = _run(inp)
    assert np.isfinite(out).all()
    h = {k: _host(x).double().numpy() for k, x in inp.items()}
    rmax = np.abs(np.einsum("bhid,bhjd->bhij", h["rho"], h["k"])).max(axis=(0, 2, 3))
    print(f"d{d}: max |<rho,k>| per head {rmax}", flush=True)
    assert rmax[0] > 5e4
    ref = po.prefill(h["q"], h["k"], h["v"], h["rho"], h["gate"])
    for hh in range(H):
        bnd = _row_bound(h["q"][0, hh], h["k"][0, hh], h["v"][0, hh], h["rho"][0, hh],
                         float(h["gate"][hh]), 1.0 / np.sqrt(d), TOL["bf16"])
        err = np.abs(out[0, hh] - ref[0, hh])
        rel = float((err / bnd).max())
        print(f"d{d} head {hh}: max-abs {err.max():.3e}, max |ref| {np.abs(ref[0, hh]).max():.3e},"
              f" max error/bound {rel:.3f}", flush=True)
        assert np.all(err <= bnd)
    # row 0 still reproduces v_0 exactly (one key: no correction at any scale)
    assert np.array_equal(out[:, :, 0], h["v"][:, :, 0])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("i0", [37, 299])
def test_one_large_rho_row_leaves_the_others_bit_identical(d, i0):
    """One row whose |<rho,k>| exceeds fp16's range among ordinary rows: its R
    overflows the fp16 products unless scaled, so the kernel takes the checked
    pass for its 16-row block, which scales that row only.  Every other row (those
    of the same block included) must come out bit-identical to a run without it,
    and the row itself within its rounding bound of the oracle."""
    B, H, L = 1, 2, 300
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=790 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    base = _run(inp)
    inp["rho"][0, 1, i0] = (inp["rho"][0, 1, i0].float() * (4e5 / d ** 0.5)).to(torch.bfloat16)
    out = _run(inp)
    keep = np.ones((B, H, L), bool)
    keep[0, 1, i0] = False
    assert np.array_equal(out[keep], base[keep])
    assert np.isfinite(out).all()
    h = {k: _host(x).double().numpy() for k, x in inp.items()}
    rmax = float(np.abs(h["k"][0, 1, : i0 + 1] @ h["rho"][0, 1, i0]).max())
    assert rmax > 65520                     # R itself overflows fp16 unscaled
    ref = po.prefill_rows(h["q"], h["k"], h["v"], h["rho"], h["gate"], 0, 1, [i0])
    bnd = _row_bound(h["q"][0, 1, : i0 + 1], h["k"][0, 1, : i0 + 1], h["v"][0, 1, : i0 + 1],
                     h["rho"][0, 1, : i0 + 1], float(h["gate"][1]), 1.0 / np.sqrt(d),
                     TOL["bf16"])[i0]
    err = np.abs(out[0, 1, i0] - ref[0])
    print(f"d{d} row {i0}: max |<rho,k>| {rmax:.3e}, max-abs {err.max():.3e}, "
          f"max error/bound {(err / bnd).max():.3f}", flush=True)
    assert np.all(err <= bnd)


@pytest.mark.parametrize("d", [64, 128])
def test_t_overflow_with_r_in_fp16_range(d):
    """R itself inside fp16's range (|r| about 2e4) while T = P*R is not: the
    scores grow along the keys by about 3 (log2 units) per 64-key tile, so the
    running max moves only every other tile and P reaches about 8 in between;
    8 * 2e4 overflows fp16, and only T does.  Every row must be finite and within
    its rounding bound of the oracle."""
    B, H, L = 1, 1, 256
    scale = 1.0 / np.sqrt(d)
    step = 3.0 / (8.0 * scale * np.log2(np.e))        # k[:, 0] slope per tile, q[:, 0] = 8
    q = torch.zeros((B, H, L, d))
    k = torch.zeros((B, H, L, d))
    rho = torch.zeros((B, H, L, d))
    g = torch.Generator().manual_seed(810 + d)
    q[..., 0] = 8.0
    q[..., 2:] = 0.1 * torch.randn((B, H, L, d - 2), generator=g)
    k[..., 0] = step * torch.arange(L, dtype=torch.float32) / 64
    k[..., 1] = 100.0 + 10.0 * torch.randn((B, H, L), generator=g)
    k[..., 2:] = torch.randn((B, H, L, d - 2), generator=g)
    rho[..., 1] = 200.0
    inp = {"q": q, "k": k, "v": torch.randn((B, H, L, d), generator=g), "rho": rho,
           "gate": torch.full((H,), 0.7)}
    inp = {n: (t.to(torch.bfloat16) if n != "gate" else t).cuda() for n, t in inp.items()}
    out = _run(inp)
    h = {n: _host(x).double().numpy() for n, x in inp.items()}
    R = h["rho"][0, 0] @ h["k"][0, 0].T
    assert np.abs(R).max() < 65504 and np.abs(R).max() > 4096
    assert np.isfinite(out).all()
    ref = po.prefill(h["q"], h["k"], h["v"], h["rho"], h["gate"])
    bnd = _row_bound(h["q"][0, 0], h["k"][0, 0], h["v"][0, 0], h["rho"][0, 0],
                     float(h["gate"][0]), scale, TOL["bf16"])
    err = np.abs(out[0, 0] - ref[0, 0])
    print(f"d{d}: max |r| {np.abs(R).max():.3e}, max-abs {err.max():.3e}, "
          f"max error/bound {(err / bnd).max():.3f}", flush=True)
    assert np.all(err <= bnd)


@pytest.mark.parametrize("d", [64, 128])
def test_large_rho_training_statistics(d):
    """The training forward with |<rho,k>| past fp16's range: the same output as
    the inference kernel (bit-identical), the log partition function within
    1e-3, and rbar and the correction vector within their rounding bounds (the
    bound of the output's correction without the gate)."""
    plx = _plx()
    B, H, L = 1, 2, 200
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=800 + d, device="cuda", rho_std=1.0,
                            gate=("uniform", 0.2, 1.0))
    inp["rho"][:, 0] = (inp["rho"][:, 0].float() * (6e4 / d ** 0.5)).to(torch.bfloat16)
    out, lse, rbar, corr = plx.prefill_train(inp["q"], inp["k"], inp["v"], inp["rho"],
                                             inp["gate"])
    plain = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    h = {k: _host(x).double().numpy() for k, x in inp.items()}
    assert np.abs(np.einsum("id,jd->ij", h["rho"][0, 0], h["k"][0, 0])).max() > 65520
    ref = po.prefill_train(h["q"], h["k"], h["v"], h["rho"], h["gate"])
    lse_h, rbar_h, corr_h = (t.cpu().double().numpy() for t in (lse, rbar, corr))
    assert np.isfinite(corr_h).all() and np.isfinite(rbar_h).all()
    assert float(np.abs(lse_h - ref["lse"]).max()) <= 1e-3
    scale = 1.0 / np.sqrt(d)
    for hh in range(H):
        q, k, v, rho = (h[n][0, hh] for n in ("q", "k", "v", "rho"))
        S = np.where(np.tril(np.ones((L, L), bool)), scale * (q @ k.T), -np.inf)
        W = np.exp(S - S.max(1, keepdims=True))
        W /= W.sum(1, keepdims=True)
        R = np.abs(rho @ k.T)
        # rbar = sum_j w_j r_j: each term within 4 roundings of 2^-11
        bnd_r = TOL["bf16"] + 4 * 2.0 ** -11 * (W * R).sum(1)
        bnd_c = _row_bound(q, k, v, rho, 1.0, scale, TOL["bf16"])
        er = np.abs(rbar_h[0, hh] - ref["rbar"][0, hh])
        ec = np.abs(corr_h[0, hh] - ref["corr"][0, hh])
        print(f"train large rho d{d} head {hh}: max |rbar| {np.abs(ref['rbar'][0, hh]).max():.3e}"
              f" err/bound {(er / bnd_r).max():.3f}; corr err/bound {(ec / bnd_c).max():.3f}",
              flush=True)
        assert np.all(er <= bnd_r)
        assert np.all(ec <= bnd_c)


@pytest.mark.parametrize("d", [64, 128])
def test_value_beyond_fp16_range_stays_in_its_rows(d):
    """A value past fp16's range at key j (clamped to +-65504 in the fp16 copy)
    must not change any row that does not attend it: rows i < j, including those
    in j's own 64-key tile where j is a masked key, stay bit-identical and
    finite."""
    B, H, L = 1, 2, 200
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=780 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    base = _run(inp)
    j = 150                                   # inside the tile of keys 128..191
    inp["v"][0, 1, j, 3] = 1.0e6
    inp["v"][0, 1, j, 4] = -float("inf")
    out = _run(inp)
    assert np.array_equal(out[0, 1, :j], base[0, 1, :j])
    assert np.array_equal(out[0, 0], base[0, 0])
    assert np.isfinite(out[0, 1, :j]).all()


@pytest.mark.parametrize("d", [64, 128])
def test_long_sequence_sampled(d):
    """A single long head (L = 65537, one past a power of two): sampled rows,
    including the last ones, against the explicit-form oracle."""
    L = 65537
    inp = wl.prefill_inputs(1, 1, L, d, "bf16", seed=700 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = _plx().prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    h = {k: _host(v) for k, v in inp.items()}
    rows = [0, 1, 4095, 4096, 32768, 65535, 65536]
    ref = po.prefill_rows(h["q"], h["k"], h["v"], h["rho"], h["gate"], 0, 0, rows)
    err = _maxerr(_host(out[0, 0, rows]).double().numpy(), ref)
    print(f"L={L} d={d}: max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_many_heads():
    """B*H = 4096 short heads: the grid's head index runs over thousands of heads."""
    B, H, L, d = 64, 64, 100, 64
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=710, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = _plx().prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    h = {k: _host(v) for k, v in inp.items()}
    worst = 0.0
    for b, hh in [(0, 0), (0, 63), (31, 17), (63, 63)]:
        ref = po.prefill_head(h["q"][b, hh].double().numpy(), h["k"][b, hh].double().numpy(),
                              h["v"][b, hh].double().numpy(), h["rho"][b, hh].double().numpy(),
                              float(h["gate"][hh]), 1.0 / 8.0)
        worst = max(worst, _maxerr(_host(out[b, hh]).double().numpy(), ref))
    print(f"prefill B*H=4096: max-abs {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("B,H", [(1, 20), (2, 17)])
def test_partial_head_group_d64(B, H):
    """d=64 runs heads in groups of 16: B*H = 20 and 34 leave a partial last
    group, whose query tiles must all be computed (every row against the
    oracle)."""
    import parallax_local_linear_amd as plx
    L, d = 200, 64
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=880 + B * H, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    h = {n: inp[n].cpu() for n in inp}
    ref = po.prefill(h["q"], h["k"], h["v"], h["rho"], h["gate"])
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    print(f"partial head group B{B} H{H}: max-abs {err:.3e}", flush=True)
    assert err <= 2e-2


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random_shapes(seed):
    """Seeded random shapes: B 1-3, H 1-20 (partial head groups at d=64), L
    1-700, d 64 or 128, bf16 or fp32; every element against the oracle."""
    rng = np.random.default_rng(2100 + seed)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 21))
    L = int(rng.integers(1, 701))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if seed % 4 == 3 else "bf16"
    if B * H * L > 6000:                      # keep the fp64 oracle to seconds
        L = max(1, 6000 // (B * H))
    inp = wl.prefill_inputs(B, H, L, d, dtype, seed=2200 + seed, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = _run(inp)
    err = _maxerr(out, _oracle_all(inp))
    print(f"random {seed}: {dtype} B{B} H{H} L{L} d{d}: max-abs {err:.3e}", flush=True)
    assert err <= TOL[dtype]
