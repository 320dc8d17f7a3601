"""Pins of the oracle's exact local-linear attention (lla_row, lla_prefill,
conjugate_gradient), the estimator Parallax approximates (page "Parallax -
Parameterized Local Linear Attention for Language Modeling", sections
"Problem" and "Core mechanism").  CPU only."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import parallax_oracle as po


def _case(seed, n=30, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(dk), rng.standard_normal((n, dk)), rng.standard_normal((n, dv))


def test_lambda_zero_is_the_weighted_least_squares_intercept():
    """lambda = 0: the intercept of the softmax-weighted least-squares fit of v
    on (k - q), by numpy lstsq."""
    q, K, V = _case(1)
    sc = 0.6
    o, _ = po.lla_row(q, K, V, sc, 0.0)
    s = sc * K @ q
    w = np.exp(s - s.max())
    w /= w.sum()
    X = np.hstack([np.ones((K.shape[0], 1)), K - q])
    sw = np.sqrt(w)[:, None]
    coef = np.linalg.lstsq(sw * X, sw * V, rcond=None)[0]
    np.testing.assert_allclose(o, coef[0], rtol=0, atol=1e-10)


def test_ridge_matches_a_ridge_fit_and_large_lambda_is_softmax_attention():
    """lambda > 0 equals the weighted ridge fit with an unpenalised intercept
    (normal equations built here with numpy), and a huge lambda leaves
    softmax attention (torch SDPA in fp64)."""
    q, K, V = _case(2)
    sc, lam = 0.4, 0.3
    o, rho = po.lla_row(q, K, V, sc, lam)
    s = sc * K @ q
    w = np.exp(s - s.max())
    w /= w.sum()
    X = np.hstack([np.ones((K.shape[0], 1)), K - q])
    P = np.diag([0.0] + [lam] * K.shape[1])      # ridge on the slopes only
    coef = np.linalg.solve(X.T @ (w[:, None] * X) + P, X.T @ (w[:, None] * V))
    np.testing.assert_allclose(o, coef[0], rtol=0, atol=1e-10)
    o_big, _ = po.lla_row(q, K, V, sc, 1e12)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    ref = F.scaled_dot_product_attention(t(q[None]), t(K), t(V), scale=sc)[0, 0, 0].numpy()
    np.testing.assert_allclose(o_big, ref, rtol=0, atol=1e-9)


def test_parallax_with_the_lla_probe_is_lla():
    """Eq. 2 with rho = rho*_i and gate 1 reproduces the exact LLA output."""
    q, K, V = _case(3, n=12)
    o, rho = po.lla_row(q, K, V, 0.5, 0.2)
    plx = po.explicit_row(q, K, V, rho, 1.0, 0.5)[0]
    np.testing.assert_allclose(o, plx, rtol=0, atol=1e-12)


def test_conjugate_gradient_solves_spd_systems():
    """d steps of CG solve a d x d SPD system (numpy solve); fewer steps reduce
    the energy-norm error monotonically."""
    rng = np.random.default_rng(4)
    M = rng.standard_normal((6, 6))
    A = M @ M.T + 0.5 * np.eye(6)
    b = rng.standard_normal(6)
    x = np.linalg.solve(A, b)
    np.testing.assert_allclose(po.conjugate_gradient(A, b), x, rtol=0, atol=1e-9)
    errs = [float((po.conjugate_gradient(A, b, k) - x) @ A @ (po.conjugate_gradient(A, b, k) - x))
            for k in range(7)]
    assert all(e1 <= e0 + 1e-12 for e0, e1 in zip(errs, errs[1:]))
    q, K, V = _case(5)
    a, _ = po.lla_row(q, K, V, 0.5, 0.1, solver="cg")
    b2, _ = po.lla_row(q, K, V, 0.5, 0.1)
    np.testing.assert_allclose(a, b2, rtol=0, atol=1e-9)


def test_lla_prefill_rows_are_lla_rows():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, 9, 4)) for _ in range(3))
    out = po.lla_prefill(q, k, v, 0.25)
    for h, i in ((0, 0), (1, 4), (0, 8)):
        o, _ = po.lla_row(q[0, h, i], k[0, h, : i + 1], v[0, h, : i + 1], 0.5, 0.25)
        np.testing.assert_allclose(out[0, h, i], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[0, :, 0], v[0, :, 0], rtol=0, atol=1e-12)
