"""Seeded synthetic inputs for the Parallax attention forward pass.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle are fed from it (the
tests pass the same tensors to each side), and nothing else is shared between
them.

Shapes and distributions follow the five workloads the library is measured
on.  The probe rho_i = W_R x_i of the page "Parallax - Parameterized Local
Linear Attention for Language Modeling" (section "Core mechanism", Eq. 1) is a
model-layer projection that sits above the attention operator; for the bf16
prefill workload it is drawn here, as an input, by that projection of random
x and W_R.

Tensor layouts (all contiguous):
  prefill: q, k, v, rho  [B, H, L, d]   gate [H] fp32
  decode : q, rho        [B, H, d]      kcache, vcache [B, H, Lmax, d]
           seqlens       [B] int32      gate [H] fp32
  chunk  : q, rho        [T, H, d]      (packed, token-major)
           kcache, vcache [B, H, Lmax, d]   cu_q [B+1], ctx [B] int32   gate [H] fp32
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One measured workload: its kind, sizes, storage dtype and seed."""
    wid: int
    kind: str            # "prefill" | "decode"
    name: str
    B: int
    H: int
    d: int
    dtype: str           # "f32" | "bf16"
    L: int = 0           # prefill sequence length
    Lmax: int = 0        # decode cache length (allocated)
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    1: Workload(1, "prefill", "prefill_f32_B1_H2_L256_d64", B=1, H=2, L=256, d=64,
                dtype="f32", seed=1001),
    2: Workload(2, "prefill", "prefill_bf16_B4_H16_L4096_d128", B=4, H=16, L=4096,
                d=128, dtype="bf16", seed=1002),
    3: Workload(3, "decode", "decode_bf16_B64_H16_L8192_d128", B=64, H=16, Lmax=8192,
                d=128, dtype="bf16", seed=1003),
    4: Workload(4, "decode", "decode_bf16_B8_H16_L65536-131072_d128", B=8, H=16,
                Lmax=131072, d=128, dtype="bf16", seed=1004),
    5: Workload(5, "prefill", "prefill_bf16_B2_H32_L16384_d64_dupkeys", B=2, H=32,
                L=16384, d=64, dtype="bf16", seed=1005),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def duplicate_key_runs(k: torch.Tensor, g: torch.Generator, frac: float = 0.05,
                       run: int = 64) -> torch.Tensor:
    """Make about `frac` of the keys of every (b, h) copies of another key.

    The sequence is cut into aligned runs of `run` keys; round(frac * L / run)
    distinct runs are chosen per (b, h), and inside each chosen run every key is
    set equal to the run's first key.  Such runs have one distinct key and so a
    vanishing key covariance.  Works in place and returns k.
    """
    B, H, L, d = k.shape
    n_runs = L // run
    n_dup = int(round(frac * L / run))
    if n_dup == 0 or n_runs == 0:
        return k
    order = torch.rand((B, H, n_runs), generator=g, device=k.device).argsort(dim=-1)
    chosen = order[..., :n_dup]                                   # [B, H, n_dup]
    kr = k[:, :, : n_runs * run].view(B, H, n_runs, run, d)
    idx = chosen[..., None, None].expand(B, H, n_dup, run, d)
    first = torch.gather(kr, 2, idx)[:, :, :, :1, :].expand(B, H, n_dup, run, d)
    kr.scatter_(2, idx, first.contiguous())
    return k


def prefill_inputs(B, H, L, d, dtype="bf16", seed=0, device="cpu", rho_std=0.1,
                   gate="ones", rho_proj_width=0, dup_keys=0.0):
    """Draw q, k, v, rho and gate for a causal prefill.

    q, k, v ~ N(0, 1).  rho ~ N(0, rho_std^2) per element, or, when
    rho_proj_width > 0, rho = x W_R^T with x ~ N(0, 1) of that width and
    W_R ~ N(0, 0.02^2) of shape [H*d, width], split head-major into [H, d].
    gate is "ones", a float constant, or ("uniform", lo, hi) drawn per head.
    All draws come from one generator seeded with `seed`, in a fixed order.
    """
    g = _gen(device, seed)
    q = _randn((B, H, L, d), g, device)
    k = _randn((B, H, L, d), g, device)
    v = _randn((B, H, L, d), g, device)
    if rho_proj_width:
        x = _randn((B, L, rho_proj_width), g, device)
        w_r = _randn((H * d, rho_proj_width), g, device, std=0.02)
        rho = torch.matmul(x, w_r.t()).view(B, L, H, d).permute(0, 2, 1, 3)
        del x, w_r
    else:
        rho = _randn((B, H, L, d), g, device, std=rho_std)
    if dup_keys:
        duplicate_key_runs(k, g, frac=dup_keys)
    gt = _gate(H, gate, g, device)
    t = DTYPES[dtype]
    return dict(q=q.to(t).contiguous(), k=k.to(t).contiguous(), v=v.to(t).contiguous(),
                rho=rho.to(t).contiguous(), gate=gt)


def decode_inputs(B, H, Lmax, d, dtype="bf16", seed=0, device="cpu", rho_std=0.1,
                  gate="ones", seqlens=None, len_range=None):
    """Draw q, rho, the K/V cache, seqlens and gate for one decode step.

    q, rho [B, H, d] and the cache [B, H, Lmax, d] are N(0, 1); rho is then
    scaled by rho_std.  seqlens is `seqlens` if given, else integers drawn
    uniformly from len_range=(lo, hi) inclusive, else Lmax for every sequence.
    The whole cache is filled, so positions past a sequence's length hold
    ordinary values that a correct kernel never reads.
    """
    g = _gen(device, seed)
    q = _randn((B, H, d), g, device)
    rho = _randn((B, H, d), g, device, std=rho_std)
    t = DTYPES[dtype]
    kc = torch.empty((B, H, Lmax, d), dtype=t, device=device)
    vc = torch.empty((B, H, Lmax, d), dtype=t, device=device)
    # fill per batch row to bound the fp32 staging memory
    for b in range(B):
        kc[b].copy_(_randn((H, Lmax, d), g, device))
    for b in range(B):
        vc[b].copy_(_randn((H, Lmax, d), g, device))
    if seqlens is not None:
        sl = torch.as_tensor(seqlens, dtype=torch.int32).to(device)
    elif len_range is not None:
        lo, hi = len_range
        sl = torch.randint(lo, hi + 1, (B,), generator=g, device=device,
                           dtype=torch.int64).to(torch.int32)
    else:
        sl = torch.full((B,), Lmax, dtype=torch.int32, device=device)
    gt = _gate(H, gate, g, device)
    return dict(q=q.to(t).contiguous(), rho=rho.to(t).contiguous(), kcache=kc,
                vcache=vc, seqlens=sl, gate=gt)


def _gate(H, gate, g, device):
    if isinstance(gate, str) and gate == "ones":
        return torch.ones(H, dtype=torch.float32, device=device)
    if isinstance(gate, (int, float)):
        return torch.full((H,), float(gate), dtype=torch.float32, device=device)
    kind, lo, hi = gate
    assert kind == "uniform"
    u = torch.rand((H,), generator=g, device=device, dtype=torch.float32)
    return (lo + (hi - lo) * u).contiguous()


def make_workload(wid: int, device="cpu", seed=None):
    """Inputs of one of the five measured workloads, by number."""
    w = WORKLOADS[wid]
    s = w.seed if seed is None else seed
    if wid == 1:
        return prefill_inputs(w.B, w.H, w.L, w.d, "f32", s, device, rho_std=0.1,
                              gate="ones")
    if wid == 2:
        return prefill_inputs(w.B, w.H, w.L, w.d, "bf16", s, device,
                              rho_proj_width=2048, gate=("uniform", 0.2, 1.0))
    if wid == 3:
        return decode_inputs(w.B, w.H, w.Lmax, w.d, "bf16", s, device, rho_std=0.1,
                             gate="ones")
    if wid == 4:
        return decode_inputs(w.B, w.H, w.Lmax, w.d, "bf16", s, device, rho_std=0.1,
                             gate="ones", len_range=(65536, 131072))
    if wid == 5:
        return prefill_inputs(w.B, w.H, w.L, w.d, "bf16", s, device, rho_std=0.1,
                              gate=("uniform", 0.0, 1.0), dup_keys=0.05)
    raise KeyError(wid)


def prefill_flops(B, H, L, d) -> float:
    """Algorithmic flops of one causal prefill: QK^T, rho K^T, PV and TV at
    2d flops each per causal (query, key) pair, L(L+1)/2 pairs per head."""
    return 8.0 * d * B * H * L * (L + 1) / 2.0


def decode_bytes(seqlens, H, d, elem=2) -> float:
    """Algorithmic HBM bytes of one decode step: K and V over the valid
    lengths, q and rho in, fp32 out, the fp32 gate and int32 seqlens."""
    sl = [int(x) for x in seqlens]
    B = len(sl)
    return (sum(sl) * H * 2 * d * elem + 2 * B * H * d * elem + B * H * d * 4
            + 4 * H + 4 * B)


# Chunked prefill against a cache (not among the five numbered workloads):
# sequences with ctx cached keys each append a chunk of queries.
CHUNK_WORKLOADS = {
    "chunk_bf16_B8_H16_ctx4096_q512_d128": dict(B=8, H=16, d=128, ctx=4096, n=512, seed=1101),
    "chunk_bf16_B32_H16_ctx8192_q16_d128": dict(B=32, H=16, d=128, ctx=8192, n=16, seed=1102),
    "chunk_bf16_B2_H16_ctx8192_q16_d128": dict(B=2, H=16, d=128, ctx=8192, n=16, seed=1103),
}


def chunk_inputs(H, d, ctx, n, dtype="bf16", seed=0, device="cpu", rho_std=0.1,
                 gate=("uniform", 0.2, 1.0), Lmax=None):
    """Draw a packed chunked-prefill batch.  ctx[b] cached keys and n[b] new
    queries per sequence; the cache [B, H, Lmax, d] is filled everywhere (rows
    past ctx[b] + n[b] hold ordinary values a correct kernel never reads),
    q and rho are N(0,1) and N(0, rho_std^2), token-major [T, H, d].  Returns
    the tensors plus cu_q, ctx (int32) and max_q."""
    B = len(ctx)
    assert len(n) == B
    Lmax = max(c + m for c, m in zip(ctx, n)) if Lmax is None else Lmax
    T = sum(n)
    g = _gen(device, seed)
    t = DTYPES[dtype]
    q = _randn((max(T, 1), H, d), g, device)[:T]
    rho = _randn((max(T, 1), H, d), g, device, std=rho_std)[:T]
    kc = torch.empty((B, H, Lmax, d), dtype=t, device=device)
    vc = torch.empty((B, H, Lmax, d), dtype=t, device=device)
    for b in range(B):
        kc[b].copy_(_randn((H, Lmax, d), g, device))
    for b in range(B):
        vc[b].copy_(_randn((H, Lmax, d), g, device))
    cu = [0]
    for m in n:
        cu.append(cu[-1] + m)
    gt = _gate(H, gate, g, device)
    return dict(q=q.to(t).contiguous(), rho=rho.to(t).contiguous(), kcache=kc, vcache=vc,
                gate=gt, cu_q=torch.tensor(cu, dtype=torch.int32, device=device),
                ctx=torch.tensor(list(ctx), dtype=torch.int32, device=device),
                max_q=max(max(n), 1), T=T)


def make_chunk_workload(name, device="cpu"):
    w = CHUNK_WORKLOADS[name]
    return chunk_inputs(w["H"], w["d"], [w["ctx"]] * w["B"], [w["n"]] * w["B"], "bf16",
                        w["seed"], device)


def chunk_flops(ctx, n, H, d) -> float:
    """Algorithmic flops of a chunked prefill: 8d per (query, attended key)
    pair; chunk query j of a sequence attends ctx + j + 1 keys."""
    pairs = sum(m * c + m * (m + 1) // 2 for c, m in zip(ctx, n))
    return 8.0 * d * H * pairs


def chunk_bytes(ctx, n, H, d, elem=2) -> float:
    """Algorithmic HBM bytes of a chunked prefill: the cache K and V rows the
    chunks attend, q and rho in, fp32 out, gate and the two index arrays."""
    keys = sum(c + m for c, m in zip(ctx, n))
    T = sum(n)
    B = len(n)
    return (keys * H * 2 * d * elem + T * H * d * (2 * elem + 4) + 4 * H + 4 * (2 * B + 1))
