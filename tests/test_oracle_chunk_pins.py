"""Pins of the oracle's chunked prefill (prefill_chunk) against the already
pinned prefill and decode forms (test_oracle_pins.py): a chunk appended to a
cache must reproduce the rows of a whole-sequence causal prefill over the
concatenation (page "Parallax - Parameterized Local Linear Attention for
Language Modeling", section "Core mechanism", Eq. 2: each row depends only on
the keys it attends), a one-token chunk is a decode step, and an empty cache is
a plain prefill.  CPU only."""
import numpy as np

from oracle import parallax_oracle as po


def _setup(seed, B=3, H=2, Lmax=40, d=6):
    rng = np.random.default_rng(seed)
    kc = rng.standard_normal((B, H, Lmax, d))
    vc = rng.standard_normal((B, H, Lmax, d))
    return rng, kc, vc


def test_chunk_equals_rows_of_whole_prefill():
    rng, kc, vc = _setup(1)
    ctx = [5, 0, 17]
    n = [7, 12, 1]
    cu = np.concatenate([[0], np.cumsum(n)])
    T = int(cu[-1])
    H, d = 2, 6
    q = rng.standard_normal((T, H, d))
    rho = rng.standard_normal((T, H, d)) * 0.7
    gate = np.array([0.4, 0.9])
    out = po.prefill_chunk(q, kc, vc, rho, gate, cu, ctx, scale=0.5)
    for b in range(3):
        Ltot = ctx[b] + n[b]
        # whole-sequence prefill whose last n[b] rows carry the chunk's queries
        qq = rng.standard_normal((1, H, Ltot, d))
        rr = rng.standard_normal((1, H, Ltot, d))
        qq[0, :, ctx[b]:] = np.transpose(q[cu[b]:cu[b + 1]], (1, 0, 2))
        rr[0, :, ctx[b]:] = np.transpose(rho[cu[b]:cu[b + 1]], (1, 0, 2))
        full = po.prefill(qq, kc[b:b + 1, :, :Ltot], vc[b:b + 1, :, :Ltot], rr, gate, scale=0.5)
        got = np.transpose(out[cu[b]:cu[b + 1]], (1, 0, 2))
        np.testing.assert_allclose(got, full[0, :, ctx[b]:], rtol=0, atol=1e-12)


def test_one_token_chunk_is_decode():
    rng, kc, vc = _setup(2)
    ctx = [9, 30, 0]
    cu = np.arange(4)
    q = rng.standard_normal((3, 2, 6))
    rho = rng.standard_normal((3, 2, 6))
    gate = np.array([1.0, 0.3])
    out = po.prefill_chunk(q, kc, vc, rho, gate, cu, ctx)
    dec = po.decode(q, kc, vc, rho, gate, [c + 1 for c in ctx])
    np.testing.assert_allclose(out, dec, rtol=0, atol=1e-12)


def test_empty_cache_is_prefill():
    rng, kc, vc = _setup(3, B=1, Lmax=25)
    q = rng.standard_normal((25, 2, 6))
    rho = rng.standard_normal((25, 2, 6))
    gate = np.array([0.6, 0.8])
    out = po.prefill_chunk(q, kc, vc, rho, gate, [0, 25], [0])
    ref = po.prefill(np.transpose(q, (1, 0, 2))[None], kc, vc,
                     np.transpose(rho, (1, 0, 2))[None], gate)
    np.testing.assert_allclose(np.transpose(out, (1, 0, 2)), ref[0], rtol=0, atol=1e-12)


def test_cache_past_the_chunk_is_never_read():
    rng, kc, vc = _setup(4)
    ctx, n = [4, 10, 2], [3, 5, 6]
    cu = np.concatenate([[0], np.cumsum(n)])
    for b in range(3):
        kc[b, :, ctx[b] + n[b]:] = np.nan
        vc[b, :, ctx[b] + n[b]:] = np.nan
    q = rng.standard_normal((int(cu[-1]), 2, 6))
    rho = rng.standard_normal((int(cu[-1]), 2, 6))
    out = po.prefill_chunk(q, kc, vc, rho, np.ones(2), cu, ctx)
    assert np.all(np.isfinite(out))
