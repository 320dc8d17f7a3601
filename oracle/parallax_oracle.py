"""CPU oracle for the Parallax attention forward pass and its gradients.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
shares no code with that path.

Source: the page "Parallax - Parameterized Local Linear Attention for Language
Modeling" (technical summary, Korean and German editions on gist.science):
  * section "Core mechanism", Eq. 2: the output is softmax attention minus the
    per-query KV covariance matrix applied to the probe, o_i = o^SA_i - Sigma_KV^(i) rho_i;
  * section "Core mechanism", Eq. 1: the probe rho_i = W_R x_i comes from the
    layer input; here it is an input array;
  * section "Core mechanism", design choices: the boundary-amplification factor
    eta_i is fixed to zero, and no per-token solver is used;
  * section "Problem": softmax attention is the local-constant (Nadaraya-Watson)
    estimator, whose weights are the softmax of the scaled scores;
  * section "Significance": W_R = 0 turns the layer back into ordinary softmax
    attention (the rho = 0 special case);
  * section "Results": a gate value scales the correction branch.

Readings taken where the pages are silent:
  * Sigma_KV^(i) is the cross-covariance of values and keys under the causal
    softmax weights w_ij of query i, centred at the weighted means, weights
    summing to one, no Bessel factor; it is d_v x d_k so that it acts on
    rho_i in R^{d_k}.
  * Scores are s_ij = scale <q_i, k_j> with scale = 1/sqrt(d_k) unless given;
    the probe products r_ij = <rho_i, k_j> are unscaled.
  * The gate g_h is a per-head scalar on the correction:
    o_i = o^SA_i - g_h Sigma_KV^(i) rho_i.
  * Prefill is causal with the diagonal included (j <= i); decode attends the
    first seqlens[b] cached keys, and a sequence of length zero gives zeros.

Everything is computed in float64 from the exact values of the inputs (an
up-cast of bf16 or fp32 to fp64 is exact).  There is no tie-break, argmax or
iteration, so every output element has exactly one correct value.

Two forms are provided:
  * the explicit form builds Sigma_KV^(i) as a d_v x d_k matrix per query
    (`explicit_row`, `prefill_explicit`, `decode_explicit`);
  * the expanded form uses the identity
      Sigma^(i) rho_i = sum_j w_ij r_ij v_j - o^SA_i sum_j w_ij r_ij
    with r_ij = <rho_i, k_j>, evaluated with whole-row matrix products
    (`prefill`, `decode`).
Both are pinned by the CPU tests against library routines, closed forms and
invariants; they are not only compared with each other.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact up-cast of an array-like (numpy or a CPU torch tensor) to fp64."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def softmax_weights(q_i, K, scale):
    """Nadaraya-Watson weights of one query over the keys K [n, d_k]:
    w_j = softmax_j(scale <q_i, k_j>) (page section "Problem")."""
    s = scale * (K @ q_i)
    e = np.exp(s - s.max())
    return e / e.sum()


def explicit_row(q_i, K, V, rho_i, g, scale):
    """One output row by the explicit covariance form of Eq. 2.

    K [n, d_k], V [n, d_v] are the keys and values the query attends.  Returns
    (o_plx, o_sa, Sigma) with Sigma the d_v x d_k weighted cross-covariance
    sum_j w_j (v_j - o_sa)(k_j - kbar)^T.
    """
    q_i, K, V, rho_i = _f64(q_i), _f64(K), _f64(V), _f64(rho_i)
    w = softmax_weights(q_i, K, scale)
    o_sa = w @ V
    kbar = w @ K
    sigma = (V - o_sa).T @ (w[:, None] * (K - kbar))
    return o_sa - g * (sigma @ rho_i), o_sa, sigma


def _default_scale(d_k, scale):
    return 1.0 / np.sqrt(d_k) if scale is None else float(scale)


def prefill_explicit(q, k, v, rho, gate, scale=None):
    """Causal prefill, every row by the explicit form.  q, k, rho [B,H,L,d_k],
    v [B,H,L,d_v], gate [H].  Cost O(L^2 d^2) per head: small inputs only."""
    q, k, v, rho, gate = map(_f64, (q, k, v, rho, gate))
    B, H, L, dk = q.shape
    sc = _default_scale(dk, scale)
    out = np.zeros(v.shape[:3] + (v.shape[3],), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(L):
                out[b, h, i] = explicit_row(q[b, h, i], k[b, h, : i + 1],
                                            v[b, h, : i + 1], rho[b, h, i],
                                            gate[h], sc)[0]
    return out


def prefill_head(q, k, v, rho, g, scale, rows=None, block=512):
    """Expanded form for one head: q, k, rho [L, d_k], v [L, d_v].

    Returns the output rows listed in `rows` (default: all), each attending
    keys 0..i.  Rows are processed a block at a time only to bound memory; each
    row is computed from its own scores exactly as in the definition.
    """
    L = q.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    for s0 in range(0, rows.size, block):
        r = rows[s0: s0 + block]
        n = int(r.max()) + 1
        S = scale * (q[r] @ k[:n].T)                      # [rows, n] scores
        causal = np.arange(n)[None, :] <= r[:, None]
        S = np.where(causal, S, -np.inf)
        W = np.exp(S - S.max(axis=1, keepdims=True))
        W /= W.sum(axis=1, keepdims=True)                 # softmax weights w_ij
        R = rho[r] @ k[:n].T                              # r_ij = <rho_i, k_j>
        WR = W * R
        o_sa = W @ v[:n]                                  # sum_j w_ij v_j
        u = WR @ v[:n]                                    # sum_j w_ij r_ij v_j
        rbar = WR.sum(axis=1, keepdims=True)              # sum_j w_ij r_ij
        out[s0: s0 + r.size] = o_sa - g * (u - o_sa * rbar)
    return out


def prefill(q, k, v, rho, gate, scale=None, heads=None):
    """Causal prefill by the expanded form.  Same layouts as prefill_explicit.
    `heads` optionally restricts the work to a list of (b, h) pairs; the other
    heads of the returned array are left as NaN."""
    q, k, v, rho, gate = map(_f64, (q, k, v, rho, gate))
    B, H, L, dk = q.shape
    sc = _default_scale(dk, scale)
    out = np.full(v.shape, np.nan, dtype=np.float64)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in todo:
        out[b, h] = prefill_head(q[b, h], k[b, h], v[b, h], rho[b, h], gate[h], sc)
    return out


def prefill_rows(q, k, v, rho, gate, b, h, rows, scale=None):
    """Selected causal output rows of head (b, h), by the explicit form."""
    dk = q.shape[-1]
    sc = _default_scale(dk, scale)
    g = float(_f64(gate)[h])
    res = []
    for i in rows:
        i = int(i)
        res.append(explicit_row(q[b, h, i], k[b, h, : i + 1], v[b, h, : i + 1],
                                rho[b, h, i], g, sc)[0])
    return np.stack(res)


def decode_stream(q, K, V, rho, g, scale):
    """Expanded form for one decode query over all keys K [n, d_k], V [n, d_v]
    (no mask: the cache holds exactly the keys the query attends).  n = 0
    gives a zero row."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    w /= w.sum()
    r = K @ rho
    o_sa = w @ V
    u = (w * r) @ V
    rbar = (w * r).sum()
    return o_sa - g * (u - o_sa * rbar)


def _lens(seqlens, Lmax):
    sl = _f64(seqlens).astype(np.int64)
    return np.clip(sl, 0, Lmax)


def decode(q, kcache, vcache, rho, gate, seqlens, scale=None, streams=None):
    """One decode step by the expanded form.  q, rho [B,H,d_k];
    kcache [B,H,Lmax,d_k]; vcache [B,H,Lmax,d_v]; seqlens [B]; gate [H].
    Sequence b attends cache positions 0..seqlens[b]-1 (clamped to
    [0, Lmax]).  `streams` optionally restricts the work to (b, h) pairs; the
    rest of the output is NaN.  Cache rows are up-cast per stream."""
    B, H, Lmax, dk = kcache.shape
    dv = vcache.shape[-1]
    sc = _default_scale(dk, scale)
    qf, rf, gf = _f64(q), _f64(rho), _f64(gate)
    lens = _lens(seqlens, Lmax)
    out = np.full((B, H, dv), np.nan, dtype=np.float64)
    todo = [(b, h) for b in range(B) for h in range(H)] if streams is None else streams
    for b, h in todo:
        n = int(lens[b])
        K = _f64(kcache[b, h, :n])
        V = _f64(vcache[b, h, :n])
        out[b, h] = decode_stream(qf[b, h], K, V, rf[b, h], gf[h], sc)
    return out


def decode_explicit(q, kcache, vcache, rho, gate, seqlens, scale=None, streams=None):
    """One decode step with Sigma_KV built explicitly per stream."""
    B, H, Lmax, dk = kcache.shape
    dv = vcache.shape[-1]
    sc = _default_scale(dk, scale)
    qf, rf, gf = _f64(q), _f64(rho), _f64(gate)
    lens = _lens(seqlens, Lmax)
    out = np.full((B, H, dv), np.nan, dtype=np.float64)
    todo = [(b, h) for b in range(B) for h in range(H)] if streams is None else streams
    for b, h in todo:
        n = int(lens[b])
        if n == 0:
            out[b, h] = 0.0
            continue
        out[b, h] = explicit_row(qf[b, h], _f64(kcache[b, h, :n]), _f64(vcache[b, h, :n]),
                                 rf[b, h], gf[h], sc)[0]
    return out


# ----------------------------------------------------------------- training
# The pages describe no backward pass; pretraining (section "Results") implies
# one.  What follows is the exact derivative of Eq. 2 (section "Core
# mechanism") with respect to q, k, v, rho and the per-head gate, written out
# by hand from the expanded form.  With S = scale Q K^T (causal), W its row
# softmax, R = rho K^T, rbar = rowsum(W*R), O_sa = W V, U = (W*R) V and the
# correction C = U - O_sa rbar (= Sigma^(i) rho_i row by row), the output is
# O = O_sa - g C.  Given dO:
#   Delta = dO V^T,  D = rowsum(dO * O_sa),  F = rowsum(dO * O)
#   dV   = (W * (1 - g (R - rbar)))^T dO
#   dR   = -g W * (Delta - D)
#   dS   = W * (Delta * (1 - g (R - rbar)) + g (R - rbar) D - F)
#   dQ   = scale dS K,  dK = scale dS^T Q + dR^T rho,  drho = dR K
#   dg   = -sum over rows of rowsum(dO * C)
# The forward statistics a backward pass needs besides O are the natural-log
# partition function lse_i = log sum_j exp(s_ij), rbar_i and the correction C_i
# (O alone does not determine O_sa when g != 0).  Pinned in the CPU tests
# against torch autograd in fp64 and central differences.

def _head_forward_blocks(q, k, v, rho, g, scale, r, n):
    """Forward quantities of the rows r (all < n) of one head, keys 0..n-1."""
    S = scale * (q[r] @ k[:n].T)
    causal = np.arange(n)[None, :] <= r[:, None]
    S = np.where(causal, S, -np.inf)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    Z = E.sum(axis=1, keepdims=True)
    W = E / Z
    lse = (mx + np.log(Z))[:, 0]
    R = rho[r] @ k[:n].T
    WR = W * R
    o_sa = W @ v[:n]
    u = WR @ v[:n]
    rbar = WR.sum(axis=1, keepdims=True)
    corr = u - o_sa * rbar
    return W, R, rbar, o_sa, corr, lse


def prefill_head_train(q, k, v, rho, g, scale, block=512):
    """Forward pass of one head that also returns the statistics a backward pass
    needs: (out [L,d_v], lse [L], rbar [L], corr [L,d_v])."""
    L = q.shape[0]
    out = np.empty((L, v.shape[1]))
    corr = np.empty((L, v.shape[1]))
    lse = np.empty(L)
    rbar = np.empty(L)
    for s0 in range(0, L, block):
        r = np.arange(s0, min(s0 + block, L))
        _, _, rb, o_sa, c, ls = _head_forward_blocks(q, k, v, rho, g, scale, r, int(r[-1]) + 1)
        out[r] = o_sa - g * c
        corr[r] = c
        lse[r] = ls
        rbar[r] = rb[:, 0]
    return out, lse, rbar, corr


def prefill_train(q, k, v, rho, gate, scale=None, heads=None):
    """Causal prefill with its saved statistics, all heads (or the listed (b, h)
    pairs; the rest stays NaN).  Returns dict(out, lse, rbar, corr)."""
    q, k, v, rho, gate = map(_f64, (q, k, v, rho, gate))
    B, H, L, dk = q.shape
    sc = _default_scale(dk, scale)
    res = dict(out=np.full(v.shape, np.nan), lse=np.full((B, H, L), np.nan),
               rbar=np.full((B, H, L), np.nan), corr=np.full(v.shape, np.nan))
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in todo:
        o, ls, rb, c = prefill_head_train(q[b, h], k[b, h], v[b, h], rho[b, h], gate[h], sc)
        res["out"][b, h], res["lse"][b, h], res["rbar"][b, h], res["corr"][b, h] = o, ls, rb, c
    return res


def prefill_head_backward(q, k, v, rho, g, scale, dout, block=512):
    """Gradients of one causal head: returns (dq, dk, dv, drho, dg) where dg is
    this head's contribution to the gate gradient.  Rows are processed a block
    at a time; the key-side gradients (dk, dv) are sums over all row blocks."""
    L = q.shape[0]
    dq = np.zeros_like(q)
    drho = np.zeros_like(rho)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dg = 0.0
    for s0 in range(0, L, block):
        r = np.arange(s0, min(s0 + block, L))
        n = int(r[-1]) + 1
        W, R, rbar, o_sa, corr, _ = _head_forward_blocks(q, k, v, rho, g, scale, r, n)
        do = dout[r]
        o = o_sa - g * corr
        Delta = do @ v[:n].T
        D = (do * o_sa).sum(axis=1, keepdims=True)
        F = (do * o).sum(axis=1, keepdims=True)
        Rc = R - rbar
        dv[:n] += (W * (1.0 - g * Rc)).T @ do
        dR = -g * W * (Delta - D)
        dS = W * (Delta * (1.0 - g * Rc) + g * Rc * D - F)
        dq[r] = scale * (dS @ k[:n])
        drho[r] = dR @ k[:n]
        dk[:n] += scale * (dS.T @ q[r]) + dR.T @ rho[r]
        dg -= float((do * corr).sum())
    return dq, dk, dv, drho, dg


def prefill_backward(q, k, v, rho, gate, dout, scale=None, heads=None):
    """Gradients of sum(out * dout) for the causal prefill.  Returns
    dict(dq, dk, dv, drho [B,H,L,d], dgate [H]).  With `heads`, only those
    (b, h) pairs are computed (their rows of the other arrays stay NaN) and
    dgate sums their contributions only."""
    q, k, v, rho, gate, dout = map(_f64, (q, k, v, rho, gate, dout))
    B, H, L, dk_ = q.shape
    sc = _default_scale(dk_, scale)
    res = {n: np.full(q.shape if n != "dv" else v.shape, np.nan)
           for n in ("dq", "dk", "dv", "drho")}
    res["dgate"] = np.zeros(H)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in todo:
        g = prefill_head_backward(q[b, h], k[b, h], v[b, h], rho[b, h], gate[h], sc,
                                  dout[b, h])
        res["dq"][b, h], res["dk"][b, h], res["dv"][b, h], res["drho"][b, h] = g[:4]
        res["dgate"][h] += g[4]
    return res


# ---------------------------------------------------------- chunked prefill
# The step between prefill and decode (section "Contributions": the kernels are
# meant for any batch size and context length): each sequence b already holds
# ctx[b] keys in its cache and appends a chunk of n_b new queries, whose keys and
# values have been written to cache positions ctx[b] .. ctx[b]+n_b-1.  Chunk
# query j sits at position p = ctx[b] + j and attends cache positions 0..p
# (causal), so every output row is one decode query (Eq. 2) over the cache
# prefix it sees.  Queries come packed and token-major: sequence b owns rows
# cu_q[b] .. cu_q[b+1]-1 of q, rho and out ([T, H, d]).

def prefill_chunk(q, kcache, vcache, rho, gate, cu_q, ctx, scale=None, rows=None):
    """Chunked causal prefill against a KV cache.  q, rho [T,H,d_k];
    kcache [B,H,Lmax,d_k]; vcache [B,H,Lmax,d_v]; cu_q [B+1]; ctx [B]; gate [H].
    Returns out [T,H,d_v].  `rows` optionally restricts the work to a list of
    token rows (the others stay NaN)."""
    B, H, Lmax, dk = kcache.shape
    dv = vcache.shape[-1]
    sc = _default_scale(dk, scale)
    qf, rf, gf = _f64(q), _f64(rho), _f64(gate)
    cu = [int(x) for x in _f64(cu_q)]
    cx = [int(x) for x in _f64(ctx)]
    T = qf.shape[0]
    out = np.full((T, H, dv), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(B):
        for j, t in enumerate(range(cu[b], cu[b + 1])):
            if want is not None and t not in want:
                continue
            p = cx[b] + j
            for h in range(H):
                K = _f64(kcache[b, h, : p + 1])
                V = _f64(vcache[b, h, : p + 1])
                out[t, h] = decode_stream(qf[t, h], K, V, rf[t, h], gf[h], sc)
    return out


# ------------------------------------------------------- exact LLA (reference)
# Section "Problem": exact local-linear attention fits, for every query, a
# softmax-weighted linear model of the values around q_i; its probe is the
# solution of a per-token linear system, solved in the original method by
# parallel conjugate gradients with a regulariser lambda that trades solver
# stability against collapse to softmax attention.  Section "Core mechanism":
# Parallax replaces that probe by a learned rho_i and drops the boundary
# factor eta_i.  Readings (the pages give neither the system nor eta or lambda):
#   * the system is the ridge-regularised normal equation of the weighted fit,
#     (Sigma_KK^(i) + lambda I) rho*_i = kbar_i - q_i, with Sigma_KK^(i) the
#     weighted key covariance (no Bessel factor) and kbar_i the weighted key mean;
#   * the output is Eq. 2 with that probe and gate 1: o_i = o^SA_i - Sigma_VK rho*_i
#     (lambda = 0 gives the intercept of the weighted least-squares fit of v on
#     k - q_i, the local-linear estimate at q_i; lambda -> infinity gives o^SA_i);
#   * eta_i = 0, as in Parallax.
# Oracle only: no kernel computes it.

def conjugate_gradient(A, b, iters=None, tol=0.0):
    """Hestenes-Stiefel conjugate gradients for a symmetric positive definite A,
    from x = 0, for `iters` steps (default: the dimension, which is exact in
    exact arithmetic) or until the residual norm is <= tol."""
    n = b.shape[0]
    iters = n if iters is None else iters
    x = np.zeros_like(b)
    r = b.copy()
    p = r.copy()
    rr = float(r @ r)
    for _ in range(iters):
        if rr <= tol * tol:
            break
        Ap = A @ p
        alpha = rr / float(p @ Ap)
        x = x + alpha * p
        r = r - alpha * Ap
        rr_new = float(r @ r)
        p = r + (rr_new / rr) * p
        rr = rr_new
    return x


def lla_row(q_i, K, V, scale, lam, solver="direct", cg_iters=None):
    """Exact LLA output for one query over keys K [n, d_k], values V [n, d_v].
    Returns (o, rho_star)."""
    q_i, K, V = _f64(q_i), _f64(K), _f64(V)
    w = softmax_weights(q_i, K, scale)
    o_sa = w @ V
    kbar = w @ K
    Kc = K - kbar
    s_kk = Kc.T @ (w[:, None] * Kc)
    s_vk = (V - o_sa).T @ (w[:, None] * Kc)
    A = s_kk + lam * np.eye(K.shape[1])
    rhs = kbar - q_i
    if solver == "cg":
        rho = conjugate_gradient(A, rhs, cg_iters)
    else:
        rho = np.linalg.solve(A, rhs)
    return o_sa - s_vk @ rho, rho


def lla_prefill(q, k, v, lam, scale=None, solver="direct", cg_iters=None):
    """Causal exact-LLA prefill: q, k [B,H,L,d_k], v [B,H,L,d_v].  lam > 0
    unless every prefix's key covariance is non-singular."""
    q, k, v = map(_f64, (q, k, v))
    B, H, L, dk = q.shape
    sc = _default_scale(dk, scale)
    out = np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            for i in range(L):
                out[b, h, i] = lla_row(q[b, h, i], k[b, h, : i + 1], v[b, h, : i + 1], sc, lam,
                                       solver, cg_iters)[0]
    return out
