"""GPU parity of the chunked prefill against a KV cache (parallax_prefill_chunk)
with the fp64 CPU oracle (prefill_chunk), whole-prefix and split-KV.
Tolerance: 2e-2 max-abs, the bf16 forward's bound."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import parallax_oracle as po

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _plx():
    import parallax_local_linear_amd as plx
    return plx


def _run(inp, out=None, split_keys=0):
    out = _plx().prefill_chunk(inp["q"], inp["kcache"], inp["vcache"], inp["rho"], inp["gate"],
                               inp["cu_q"], inp["ctx"], inp["max_q"], out=out,
                               split_keys=split_keys)
    torch.cuda.synchronize()
    return out


def _oracle(inp, rows=None):
    h = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp.items()}
    return po.prefill_chunk(h["q"], h["kcache"], h["vcache"], h["rho"], h["gate"], h["cu_q"],
                            h["ctx"], rows=rows)


CASES = [  # (ctx per sequence, chunk length per sequence)
    ([0], [1]),
    ([0], [65]),
    ([1], [1]),
    ([63, 64, 65], [1, 2, 3]),
    ([60, 4, 0, 130], [16, 17, 15, 64]),
    ([1000, 7], [65, 200]),
    ([100, 0, 33, 257, 5], [33, 1, 128, 9, 300]),
    ([60, 4, 0, 130], [16, 17, 15, 32]),               # 17-32 queries: two busy waves
    ([0, 191, 64], [32, 18, 29]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "ctx" + "-".join(map(str, c[0])) + "_n" +
                         "-".join(map(str, c[1])))
def test_chunk_cases(case, d):
    ctx, n = case
    inp = wl.chunk_inputs(3, d, ctx, n, seed=1200 + sum(ctx) + sum(n) + d, device="cuda",
                          rho_std=0.5)
    out = _run(inp).cpu().double().numpy()
    ref = _oracle(inp)
    err = float(np.max(np.abs(out - ref)))
    print(f"chunk d{d} ctx{ctx} n{n}: max-abs {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_empty_cache_chunk_is_the_prefill(d):
    """ctx = 0 and one sequence, not split: bit-identical to the whole-sequence
    prefill (the same kernel arithmetic over the same tiles)."""
    plx = _plx()
    L, H = 333, 2
    inp = wl.chunk_inputs(H, d, [0], [L], seed=1300 + d, device="cuda", rho_std=0.5)
    out = _run(inp, split_keys=384)
    q = inp["q"].transpose(0, 1).unsqueeze(0).contiguous()
    rho = inp["rho"].transpose(0, 1).unsqueeze(0).contiguous()
    ref = plx.prefill(q, inp["kcache"], inp["vcache"], rho, inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0].transpose(0, 1))


@pytest.mark.parametrize("n", [[20, 70, 100], [20, 7, 64]], ids=["staged", "fused"])
def test_cache_past_the_chunk_is_never_read_and_other_rows_untouched(n):
    """NaN in every cache row past each chunk changes no output bit.  Chunks of at
    most 64 queries at d = 128 read V straight from the cache (fused path)."""
    ctx = [50, 200, 3]
    inp = wl.chunk_inputs(2, 128, ctx, n, seed=1310, device="cuda", Lmax=400)
    a = _run(inp).clone()
    for b in range(3):
        inp["kcache"][b, :, ctx[b] + n[b]:] = float("nan")
        inp["vcache"][b, :, ctx[b] + n[b]:] = float("nan")
    # an out buffer with 5 extra rows past the packed chunks, filled with a sentinel
    T = sum(n)
    out = torch.full((T + 5, 2, 128), -7.0, dtype=torch.float32, device="cuda")
    _plx().prefill_chunk(inp["q"], inp["kcache"], inp["vcache"], inp["rho"], inp["gate"],
                         inp["cu_q"], inp["ctx"], inp["max_q"], out=out[:T])
    torch.cuda.synchronize()
    assert torch.equal(out[:T], a)
    assert bool((out[T:] == -7.0).all())


def test_bad_lengths_are_clamped_on_the_device():
    """ctx beyond the cache and cu_q beyond T are clamped, not followed: the
    call stays in bounds and the well-formed sequences are unaffected."""
    inp = wl.chunk_inputs(2, 64, [10, 20], [5, 6], seed=1320, device="cuda", Lmax=40)
    good = _run(inp).clone()
    bad = dict(inp)
    bad["ctx"] = torch.tensor([10, 10 ** 6], dtype=torch.int32, device="cuda")
    out = _run(bad)
    assert torch.equal(out[:5], good[:5])
    assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("name", sorted(wl.CHUNK_WORKLOADS))
def test_chunk_workload_sampled(name):
    """The benchmark's chunked workloads: sampled token rows of every sequence
    against the oracle."""
    inp = wl.make_chunk_workload(name, device="cuda")
    out = _run(inp)
    assert bool(torch.isfinite(out).all())
    cu = inp["cu_q"].tolist()
    rng = np.random.default_rng(7)
    rows = []
    for b in range(0, len(cu) - 1, max(1, (len(cu) - 1) // 4)):
        rows += [cu[b], cu[b + 1] - 1] + [int(x) for x in rng.integers(cu[b], cu[b + 1], 3)]
    ref = _oracle(inp, rows=rows)
    got = out.cpu().double().numpy()
    err = float(np.max(np.abs(got[rows] - ref[rows])))
    print(f"{name}: {len(rows)} sampled rows, max-abs {err:.3e}", flush=True)
    assert err <= TOL
    # the serving path the benchmark also times: V from a staged cache (for
    # one-tile chunks with non-temporal tile loads), the same bits
    plx = _plx()
    vt = plx.prefill_stage_v(inp["vcache"])
    staged = plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"], inp["gate"],
                               inp["cu_q"], inp["ctx"], inp["max_q"], vt_cache=vt)
    torch.cuda.synchronize()
    assert torch.equal(staged, out)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES[2:6], ids=lambda c: "ctx" + "-".join(map(str, c[0])))
def test_staged_cache_matches_per_call_staging(case, d):
    """V read from a caller-kept staged cache gives the same bits as the call
    that stages the rows it reads."""
    plx = _plx()
    ctx, n = case
    inp = wl.chunk_inputs(3, d, ctx, n, seed=1400 + sum(ctx) + d, device="cuda", rho_std=0.5)
    ref = _run(inp)
    vt = plx.prefill_stage_v(inp["vcache"])
    out = plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"], inp["gate"], inp["cu_q"],
                            inp["ctx"], inp["max_q"], vt_cache=vt)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("d", [64, 128])
def test_incremental_serving_with_a_staged_cache(d):
    """Four rounds of appended chunks: the new K/V rows are written into the
    caches (whose unwritten rows hold NaN), stage_v_rows re-stages only their
    tiles, and the chunk reads the staged cache.  Every round matches the
    oracle and the per-call-staging path bit for bit."""
    plx = _plx()
    H, Lmax, B = 2, 400, 3
    g = torch.Generator(device="cuda").manual_seed(1500 + d)
    kc = torch.full((B, H, Lmax, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    vt = plx.chunk_vt_cache(B, H, Lmax, d, "cuda")
    gate = torch.rand(H, generator=g, device="cuda") * 0.8 + 0.2
    ctx = [0, 37, 100]
    # rows already cached before the first round, staged like an append from 0
    for b in range(B):
        kc[b, :, :ctx[b]] = torch.randn((H, ctx[b], d), generator=g, device="cuda").to(torch.bfloat16)
        vc[b, :, :ctx[b]] = torch.randn((H, ctx[b], d), generator=g, device="cuda").to(torch.bfloat16)
    cu0 = torch.tensor([0] + list(np.cumsum(ctx)), dtype=torch.int32, device="cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    plx.stage_v_rows(vc, vt, cu0, zero, max(ctx), int(sum(ctx)))
    for n in ([5, 64, 17], [1, 1, 80], [70, 3, 0], [16, 1, 9]):
        for b in range(B):
            kc[b, :, ctx[b]:ctx[b] + n[b]] = torch.randn((H, n[b], d), generator=g,
                                                        device="cuda").to(torch.bfloat16)
            vc[b, :, ctx[b]:ctx[b] + n[b]] = torch.randn((H, n[b], d), generator=g,
                                                        device="cuda").to(torch.bfloat16)
        T = sum(n)
        q = torch.randn((T, H, d), generator=g, device="cuda").to(torch.bfloat16)
        rho = (0.5 * torch.randn((T, H, d), generator=g, device="cuda")).to(torch.bfloat16)
        cu = torch.tensor([0] + list(np.cumsum(n)), dtype=torch.int32, device="cuda")
        cx = torch.tensor(ctx, dtype=torch.int32, device="cuda")
        plx.stage_v_rows(vc, vt, cu, cx, max(n), T)
        out = plx.prefill_chunk(q, kc, None, rho, gate, cu, cx, max(n), vt_cache=vt)
        ref = plx.prefill_chunk(q, kc, vc, rho, gate, cu, cx, max(n))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        assert torch.equal(out, ref)
        want = po.prefill_chunk(q.cpu(), kc.cpu(), vc.cpu(), rho.cpu(), gate.cpu(), cu.cpu(),
                                cx.cpu())
        err = float(np.max(np.abs(out.cpu().double().numpy() - want)))
        print(f"serving d{d} ctx{ctx} n{n}: max-abs {err:.3e}", flush=True)
        assert err <= TOL
        ctx = [c + m for c, m in zip(ctx, n)]


SPLIT_CASES = [  # (ctx per sequence, chunk length per sequence, keys per split)
    ([0], [65], 64),                                   # a split boundary inside the chunk
    ([63, 64, 65], [1, 2, 3], 64),
    ([60, 4, 0, 130], [16, 17, 15, 64], 64),
    ([1000, 7], [65, 200], 128),
    ([100, 0, 33, 257, 5], [33, 1, 128, 9, 300], 192),
    ([3000], [16], 0),                                 # the library's split
    ([5000, 20], [1, 130], 0),
    ([60, 4, 0, 130], [16, 17, 15, 32], 64),
    ([2500, 1000], [32, 20], 0),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "ctx" + "-".join(map(str, c[0])) +
                         "_n" + "-".join(map(str, c[1])) + f"_s{c[2]}")
def test_chunk_split_kv(case, d):
    """Split-KV: every row against the oracle, the staged-cache call with the
    same split bit for bit, and the unsplit call within the tolerance."""
    plx = _plx()
    ctx, n, split = case
    H = 3
    inp = wl.chunk_inputs(H, d, ctx, n, seed=1600 + sum(ctx) + sum(n) + d, device="cuda",
                          rho_std=0.5)
    B, Lmax = len(ctx), inp["kcache"].shape[2]
    if split == 0:
        assert plx.chunk_default_split(B, H, Lmax, inp["max_q"], d) < Lmax   # it does split
    out = _run(inp, split_keys=split)
    err = float(np.max(np.abs(out.cpu().double().numpy() - _oracle(inp))))
    print(f"split d{d} ctx{ctx} n{n} split {split}: max-abs {err:.3e}", flush=True)
    assert err <= TOL
    vt = plx.prefill_stage_v(inp["vcache"])
    staged = plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"], inp["gate"],
                               inp["cu_q"], inp["ctx"], inp["max_q"], vt_cache=vt,
                               split_keys=split)
    whole = _run(inp, split_keys=(Lmax + 63) // 64 * 64)
    torch.cuda.synchronize()
    assert torch.equal(staged, out)
    assert float((whole - out).abs().max()) <= TOL


def test_split_kv_small_batch_long_cache_sampled():
    """Two sequences of 16-query chunks on 8192 cached keys (d=128, 16 heads):
    the default splits each prefix into 15 ranges of 576 keys; sampled rows
    against the oracle."""
    plx = _plx()
    B, H, d, ctx, n = 2, 16, 128, 8192, 16
    inp = wl.chunk_inputs(H, d, [ctx] * B, [n] * B, seed=1700, device="cuda")
    assert plx.chunk_default_split(B, H, ctx + n, n, d) == 576
    out = _run(inp)
    rows = [0, 7, 15, 16, 23, 31]
    ref = _oracle(inp, rows=rows)
    err = float(np.max(np.abs(out.cpu().double().numpy()[rows] - ref[rows])))
    print(f"split B{B} H{H} ctx{ctx}: max-abs {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("seed", range(12))
def test_chunk_random_shapes(seed):
    """Seeded random ragged batches: 1-6 sequences, 0-2000 cached keys, 1-150
    queries, d 64 or 128, the library's split, an explicit split or none, V
    staged per call or read from a staged cache.  Every row against the oracle;
    the staged-cache call with the same split gives the same bits."""
    plx = _plx()
    rng = np.random.default_rng(1900 + seed)
    B = int(rng.integers(1, 7))
    d = int(rng.choice([64, 128]))
    ctx = [int(x) for x in rng.integers(0, 2001, B)]
    n = [int(x) for x in rng.integers(1, 151, B)]
    H = int(rng.integers(1, 4))
    inp = wl.chunk_inputs(H, d, ctx, n, seed=2000 + seed, device="cuda", rho_std=0.5)
    Lmax = inp["kcache"].shape[2]
    split = [0, 64 * int(rng.integers(1, 9)), (Lmax + 63) // 64 * 64][seed % 3]
    out = _run(inp, split_keys=split)
    err = float(np.max(np.abs(out.cpu().double().numpy() - _oracle(inp))))
    vt = plx.prefill_stage_v(inp["vcache"])
    staged = plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"], inp["gate"],
                               inp["cu_q"], inp["ctx"], inp["max_q"], vt_cache=vt,
                               split_keys=split)
    torch.cuda.synchronize()
    print(f"random {seed}: B{B} H{H} d{d} ctx{ctx} n{n} split {split}: max-abs {err:.3e}",
          flush=True)
    assert err <= TOL
    assert torch.equal(staged, out)


@pytest.mark.parametrize("seed", range(8))
def test_chunk_random_short_chunks(seed):
    """Seeded random batches of short chunks at d = 128 (1-64 queries, the shapes
    whose per-call V tiles the kernel converts itself): 1-8 sequences, 0-3000
    cached keys, the library's split, an explicit split or none.  Every row
    against the oracle; the staged-cache call gives the same bits."""
    plx = _plx()
    rng = np.random.default_rng(2100 + seed)
    B = int(rng.integers(1, 9))
    ctx = [int(x) for x in rng.integers(0, 3001, B)]
    n = [int(x) for x in rng.integers(1, (17, 33, 65)[seed % 3], B)]
    H = int(rng.integers(1, 5))
    inp = wl.chunk_inputs(H, 128, ctx, n, seed=2200 + seed, device="cuda", rho_std=0.5)
    Lmax = inp["kcache"].shape[2]
    split = [0, 64 * int(rng.integers(1, 9)), (Lmax + 63) // 64 * 64][seed % 3]
    out = _run(inp, split_keys=split)
    err = float(np.max(np.abs(out.cpu().double().numpy() - _oracle(inp))))
    vt = plx.prefill_stage_v(inp["vcache"])
    staged = plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"], inp["gate"],
                               inp["cu_q"], inp["ctx"], inp["max_q"], vt_cache=vt,
                               split_keys=split)
    torch.cuda.synchronize()
    print(f"short {seed}: B{B} H{H} ctx{ctx} n{n} split {split}: max-abs {err:.3e}", flush=True)
    assert err <= TOL
    assert torch.equal(staged, out)


def _chunk_row_bounds(inp):
    """Per-row rounding bound for large rho (see the prefill test of the same
    name): 2e-2 plus 4 * 2^-11 * g * (sum_j w_j |r_j| |v_j| + sum_j w_j |r_j| sum_j w_j |v_j|)
    over the row's causal cache prefix."""
    h = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp.items()}
    q, rho = h["q"].double().numpy(), h["rho"].double().numpy()
    kc, vc = h["kcache"].double().numpy(), h["vcache"].double().numpy()
    gate = h["gate"].double().numpy()
    cu, ctx = h["cu_q"].tolist(), h["ctx"].tolist()
    T, H, d = q.shape
    bnd = np.full((T, H, d), np.nan)
    for b in range(len(ctx)):
        for j, t in enumerate(range(cu[b], cu[b + 1])):
            p = ctx[b] + j
            for hh in range(H):
                K, V = kc[b, hh, : p + 1], vc[b, hh, : p + 1]
                s = (K @ q[t, hh]) / np.sqrt(d)
                w = np.exp(s - s.max())
                w /= w.sum()
                r = np.abs(K @ rho[t, hh])
                a = (w * r) @ np.abs(V) + (w @ r) * (w @ np.abs(V))
                bnd[t, hh] = TOL + 4 * 2.0 ** -11 * gate[hh] * a
    return bnd


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [[40, 130], [40, 20]], ids=["long", "short"])
@pytest.mark.parametrize("split", [0, 128, 4096])
def test_chunk_large_rho(d, n, split):
    """|<rho,k>| up to about 1e5: the chunk kernels scale such rows by a power of
    two, split records carry the scale (slot 3) and the combine removes it.  Per
    call and with the staged V cache (bit-identical), split and not split;
    [40, 20] at d = 128 runs the in-kernel V conversion."""
    plx = _plx()
    ctx = [500, 37]
    inp = wl.chunk_inputs(2, d, ctx, n, seed=1400 + d + sum(n), device="cuda", rho_std=1.0)
    inp["rho"] = (inp["rho"].float() * (2.2e4 / d ** 0.5)).to(torch.bfloat16)
    out = _run(inp, split_keys=split)
    vt = plx.prefill_stage_v(inp["vcache"])
    out_vt = plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"], inp["gate"],
                               inp["cu_q"], inp["ctx"], inp["max_q"], vt_cache=vt,
                               split_keys=split)
    torch.cuda.synchronize()
    assert torch.equal(out, out_vt)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    ref = _oracle(inp)
    bnd = _chunk_row_bounds(inp)
    err = np.abs(got - ref)
    print(f"chunk large rho d{d} n{n} split {split}: max-abs {err.max():.3e}, "
          f"max |ref| {np.abs(ref).max():.3e}, max error/bound {(err / bnd).max():.3f}",
          flush=True)
    assert np.all(err <= bnd)
