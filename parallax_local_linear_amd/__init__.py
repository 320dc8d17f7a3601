"""Parallax attention forward pass on AMD MI355X (gfx950).

The operation (page "Parallax - Parameterized Local Linear Attention for
Language Modeling", section "Core mechanism", Eq. 2) is

    o_i = o^SA_i - g_h * Sigma_KV^(i) rho_i

softmax attention minus a gated correction: the softmax-weighted covariance of
values and keys applied to the probe rho_i.  `prefill` runs the causal forward
pass over whole sequences; `decode` runs one query per sequence against a KV
cache.  `prefill_train` and `prefill_backward` give the exact gradients of
the causal prefill (bf16).  The `softmax_*` functions run the same kernels with the correction
branch compiled out (plain causal softmax attention), the like-for-like
baseline for the cost of the correction.  All are thin wrappers over the C ABI
of libparallax.so: they check shapes, allocate outputs and workspaces with torch
on the inputs' device, and enqueue the HIP kernels on torch's current stream.
"""
from __future__ import annotations

import math

import torch

from ._native import PLX_BF16, PLX_F32, ParallaxError, call, lib  # noqa: F401

__all__ = ["prefill", "decode", "prefill_stage_v", "prefill_attend", "decode_partials",
           "decode_combine", "prefill_workspace_bytes", "decode_workspace_bytes",
           "decode_default_split", "softmax_prefill", "softmax_prefill_attend",
           "softmax_decode", "prefill_train", "prefill_backward",
           "prefill_backward_workspace_bytes", "prefill_chunk", "stage_v_rows",
           "chunk_vt_cache", "chunk_default_split", "parallax_attention",
           "ParallaxAttentionFunction",
           "ParallaxError"]

_DT = {torch.bfloat16: PLX_BF16, torch.float32: PLX_F32}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _launch(dev, name, *args):
    """Call the library with `dev` as the current device: the kernels run on that
    device's current torch stream (the last argument of every launching call)."""
    with torch.cuda.device(dev):
        return call(name, *args, _stream(dev))


def _split(split_keys):
    c = int(split_keys)
    if c <= 0 or c % 64:
        raise ValueError(f"split_keys must be a positive multiple of 64, got {split_keys}")
    return c


def _check(name, t, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _scale(scale, d):
    return float(scale) if scale is not None else 1.0 / math.sqrt(d)


def prefill_workspace_bytes(B, H, L, d, dtype=torch.bfloat16) -> int:
    return int(lib().parallax_prefill_workspace_bytes(B, H, L, d, _DT[dtype]))


def decode_workspace_bytes(B, H, Lmax, d, split_keys=0) -> int:
    return int(lib().parallax_decode_workspace_bytes(B, H, Lmax, d, split_keys))


def decode_default_split(B, H, Lmax, d) -> int:
    return int(lib().parallax_decode_default_split(B, H, Lmax, d))


def _prefill_checks(q, others):
    _check("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    dt = q.dtype
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    for n, t in others:
        _check(n, t, dt, q.shape, q.device)
    return (*q.shape, dt)


def _prefill_out_ws(q, out, workspace):
    B, H, L, d = q.shape
    dt = q.dtype
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (B, H, L, d), q.device)
    wsb = 0
    if workspace is None and dt == torch.bfloat16:
        wsb = prefill_workspace_bytes(B, H, L, d, dt)
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    elif workspace is not None:
        _check("workspace", workspace, device=q.device)
        wsb = workspace.numel() * workspace.element_size()
    return out, workspace, wsb


def prefill(q, k, v, rho, gate, scale=None, out=None, workspace=None):
    """Causal Parallax prefill.  q, k, v, rho: [B, H, L, d] bf16 or fp32 on one
    GPU; gate: [H] fp32.  Returns out [B, H, L, d] fp32."""
    B, H, L, d, dt = _prefill_checks(q, (("k", k), ("v", v), ("rho", rho)))
    _check("gate", gate, torch.float32, (H,), q.device)
    out, workspace, wsb = _prefill_out_ws(q, out, workspace)
    _launch(q.device, "parallax_prefill", _ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(gate),
            _ptr(out), B, H, L, d, _scale(scale, d), _DT[dt], _ptr(workspace), wsb)
    return out


def softmax_prefill(q, k, v, scale=None, out=None, workspace=None):
    """Causal softmax attention through the prefill kernels with the correction
    branch compiled out.  q, k, v: [B, H, L, d] bf16 or fp32.  Returns out
    [B, H, L, d] fp32."""
    B, H, L, d, dt = _prefill_checks(q, (("k", k), ("v", v)))
    out, workspace, wsb = _prefill_out_ws(q, out, workspace)
    _launch(q.device, "parallax_softmax_prefill", _ptr(q), _ptr(k), _ptr(v), _ptr(out),
            B, H, L, d, _scale(scale, d), _DT[dt], _ptr(workspace), wsb)
    return out


def prefill_backward_workspace_bytes(B, H, L, d) -> int:
    return int(lib().parallax_prefill_backward_workspace_bytes(B, H, L, d))


def prefill_train(q, k, v, rho, gate, scale=None, workspace=None):
    """Training forward pass (bf16): returns (out, lse, rbar, corr), the output
    and the statistics prefill_backward needs: lse [B,H,L] natural-log
    partition function, rbar [B,H,L], corr [B,H,L,d] = Sigma rho."""
    B, H, L, d, dt = _prefill_checks(q, (("k", k), ("v", v), ("rho", rho)))
    if dt != torch.bfloat16:
        raise TypeError("prefill_train supports bfloat16 inputs only")
    _check("gate", gate, torch.float32, (H,), q.device)
    out, workspace, wsb = _prefill_out_ws(q, None, workspace)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    rbar = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    corr = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    _launch(q.device, "parallax_prefill_train", _ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(gate),
            _ptr(out), _ptr(lse), _ptr(rbar), _ptr(corr), B, H, L, d, _scale(scale, d),
            PLX_BF16, _ptr(workspace), wsb)
    return out, lse, rbar, corr


def prefill_backward(q, k, v, rho, gate, out, corr, lse, rbar, dout, scale=None, grads=None,
                     workspace=None):
    """Gradients of sum(out * dout) for the causal prefill (bf16 inputs).  out,
    corr, lse and rbar come from prefill_train on the same inputs; dout is fp32
    [B,H,L,d].  Returns (dq, dk, dv, drho [B,H,L,d] fp32, dgate [H] fp32)."""
    B, H, L, d, dt = _prefill_checks(q, (("k", k), ("v", v), ("rho", rho)))
    if dt != torch.bfloat16:
        raise TypeError("prefill_backward supports bfloat16 inputs only")
    _check("gate", gate, torch.float32, (H,), q.device)
    for n, t in (("out", out), ("corr", corr), ("dout", dout)):
        _check(n, t, torch.float32, (B, H, L, d), q.device)
    for n, t in (("lse", lse), ("rbar", rbar)):
        _check(n, t, torch.float32, (B, H, L), q.device)
    if grads is None:
        grads = tuple(torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
                      for _ in range(4)) + (torch.empty(H, dtype=torch.float32, device=q.device),)
    for n, t in zip(("dq", "dk", "dv", "drho"), grads[:4]):
        _check(n, t, torch.float32, (B, H, L, d), q.device)
    _check("dgate", grads[4], torch.float32, (H,), q.device)
    wsb = prefill_backward_workspace_bytes(B, H, L, d)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    _launch(q.device, "parallax_prefill_backward", _ptr(q), _ptr(k), _ptr(v), _ptr(rho),
            _ptr(gate), _ptr(out), _ptr(corr), _ptr(lse), _ptr(rbar), _ptr(dout),
            *(_ptr(t) for t in grads), B, H, L, d, _scale(scale, d), PLX_BF16,
            _ptr(workspace), wsb)
    return grads


def _chunk_checks(q, kcache, rho, gate, cu_q, ctx):
    _check("q", q, torch.bfloat16)
    _check("kcache", kcache, torch.bfloat16)
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [T, H, d] and kcache [B, H, Lmax, d]")
    T, H, d = q.shape
    B, _, Lmax, _ = kcache.shape
    _check("kcache", kcache, torch.bfloat16, (B, H, Lmax, d), q.device)
    _check("rho", rho, torch.bfloat16, (T, H, d), q.device)
    _check("gate", gate, torch.float32, (H,), q.device)
    _check("cu_q", cu_q, torch.int32, (B + 1,), q.device)
    _check("ctx", ctx, torch.int32, (B,), q.device)
    return T, H, d, B, Lmax


def _vt_cache_bytes(B, H, Lmax, d):
    return int(lib().parallax_prefill_workspace_bytes(B, H, Lmax, d, PLX_BF16))


def chunk_vt_cache(B, H, Lmax, d, device):
    """An empty staged V^T cache for prefill_chunk(..., vt_cache=...)."""
    return torch.empty(_vt_cache_bytes(B, H, Lmax, d), dtype=torch.uint8, device=device)


def stage_v_rows(vcache, vt_cache, cu_q, ctx, max_q, T):
    """Re-stage into vt_cache the V^T tiles holding rows ctx[b] .. ctx[b]+n_b-1
    of vcache [B, H, Lmax, d] (after those rows were written)."""
    _check("vcache", vcache, torch.bfloat16)
    if vcache.dim() != 4:
        raise ValueError("vcache must be [B, H, Lmax, d]")
    B, H, Lmax, d = vcache.shape
    _check("vt_cache", vt_cache, device=vcache.device)
    if vt_cache.numel() * vt_cache.element_size() < _vt_cache_bytes(B, H, Lmax, d):
        raise ValueError("vt_cache is too small")
    _check("cu_q", cu_q, torch.int32, (B + 1,), vcache.device)
    _check("ctx", ctx, torch.int32, (B,), vcache.device)
    _launch(vcache.device, "parallax_stage_v_rows", _ptr(vcache), _ptr(vt_cache), _ptr(cu_q),
            _ptr(ctx), B, H, int(T), Lmax, int(max_q), d)
    return vt_cache


def chunk_default_split(B, H, Lmax, max_q, d):
    """Keys per split prefill_chunk uses with split_keys=0 (>= Lmax: no split)."""
    return int(lib().parallax_prefill_chunk_default_split(B, H, Lmax, int(max_q), d))


def prefill_chunk(q, kcache, vcache, rho, gate, cu_q, ctx, max_q, scale=None, out=None,
                  workspace=None, vt_cache=None, split_keys=0):
    """Chunked causal prefill against a KV cache (bf16).  q, rho: [T, H, d]
    packed token-major; kcache, vcache: [B, H, Lmax, d] holding each chunk's
    own keys at positions ctx[b] .. ctx[b]+n_b-1; cu_q [B+1] and ctx [B] int32 on
    the GPU; max_q >= the largest chunk.  With vt_cache (kept up to date by
    stage_v_rows) V is read from the staged cache and vcache may be None.
    split_keys: keys per split-KV range (0: the library's choice; a multiple of
    64, >= Lmax for none).  Returns out [T, H, d] fp32."""
    T, H, d, B, Lmax = _chunk_checks(q, kcache, rho, gate, cu_q, ctx)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (T, H, d), q.device)
    sk, mq = int(split_keys), int(max_q)
    if vt_cache is not None:
        _check("vt_cache", vt_cache, device=q.device)
        if vt_cache.numel() * vt_cache.element_size() < _vt_cache_bytes(B, H, Lmax, d):
            raise ValueError("vt_cache is too small")
        wsb = int(lib().parallax_prefill_chunk_vt_workspace_bytes(B, H, T, Lmax, mq, d, sk))
        if workspace is None and wsb > 0:
            workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            _check("workspace", workspace, device=q.device)
            wsb = workspace.numel() * workspace.element_size()
        _launch(q.device, "parallax_prefill_chunk_vt", _ptr(q), _ptr(kcache), _ptr(vt_cache),
                _ptr(rho), _ptr(gate), _ptr(out), _ptr(cu_q), _ptr(ctx), B, H, T, Lmax, mq, d,
                _scale(scale, d), PLX_BF16, sk,
                _ptr(workspace), wsb)
        return out
    _check("vcache", vcache, torch.bfloat16, (B, H, Lmax, d), q.device)
    wsb = int(lib().parallax_prefill_chunk_workspace_bytes(B, H, T, Lmax, mq, d, sk))
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check("workspace", workspace, device=q.device)
        wsb = workspace.numel() * workspace.element_size()
    _launch(q.device, "parallax_prefill_chunk", _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(rho),
            _ptr(gate), _ptr(out), _ptr(cu_q), _ptr(ctx), B, H, T, Lmax, mq, d,
            _scale(scale, d), PLX_BF16, sk, _ptr(workspace), wsb)
    return out


def prefill_stage_v(v, vt=None):
    """First stage of a bf16 prefill: V -> fp16 V^T tiles (a uint8 buffer)."""
    _check("v", v, torch.bfloat16)
    if v.dim() != 4:
        raise ValueError("v must be [B, H, L, d]")
    B, H, L, d = v.shape
    n = prefill_workspace_bytes(B, H, L, d, torch.bfloat16)
    if vt is None:
        vt = torch.empty(n, dtype=torch.uint8, device=v.device)
    _check("vt", vt, device=v.device)
    if vt.numel() * vt.element_size() < n:
        raise ValueError(f"vt must hold {n} bytes")
    _launch(v.device, "parallax_prefill_stage_v", _ptr(v), _ptr(vt), B, H, L, d)
    return vt


def prefill_attend(q, k, vt, rho, gate, scale=None, out=None):
    """Second stage of a bf16 prefill, reading V from prefill_stage_v's buffer."""
    _check("q", q, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    for n, t in (("k", k), ("rho", rho)):
        _check(n, t, torch.bfloat16, q.shape, q.device)
    _check("gate", gate, torch.float32, (H,), q.device)
    _check("vt", vt, device=q.device)
    if vt.numel() * vt.element_size() < prefill_workspace_bytes(B, H, L, d):
        raise ValueError("vt is too small")
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (B, H, L, d), q.device)
    _launch(q.device, "parallax_prefill_attend", _ptr(q), _ptr(k), _ptr(vt), _ptr(rho),
            _ptr(gate), _ptr(out), B, H, L, d, _scale(scale, d))
    return out


def softmax_prefill_attend(q, k, vt, scale=None, out=None):
    """Softmax-only second stage of a bf16 prefill, reading V from
    prefill_stage_v's buffer."""
    _check("q", q, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    _check("k", k, torch.bfloat16, q.shape, q.device)
    _check("vt", vt, device=q.device)
    if vt.numel() * vt.element_size() < prefill_workspace_bytes(B, H, L, d):
        raise ValueError("vt is too small")
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (B, H, L, d), q.device)
    _launch(q.device, "parallax_softmax_prefill_attend", _ptr(q), _ptr(k), _ptr(vt), _ptr(out),
            B, H, L, d, _scale(scale, d))
    return out


def _decode_checks(q, kcache, vcache, rho, seqlens):
    _check("q", q)
    _check("kcache", kcache)
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, H, d] and kcache [B, H, Lmax, d]")
    B, H, d = q.shape
    Lmax = kcache.shape[2]
    dt = q.dtype
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    if rho is not None:
        _check("rho", rho, dt, (B, H, d), q.device)
    _check("kcache", kcache, dt, (B, H, Lmax, d), q.device)
    _check("vcache", vcache, dt, (B, H, Lmax, d), q.device)
    _check("seqlens", seqlens, torch.int32, (B,), q.device)
    return B, H, Lmax, d, dt


def decode(q, kcache, vcache, rho, gate, seqlens, scale=None, split_keys=0, out=None,
           workspace=None):
    """One Parallax decode step.  q, rho: [B, H, d]; kcache, vcache:
    [B, H, Lmax, d] (bf16 or fp32); gate [H] fp32; seqlens [B] int32 on the
    GPU.  Returns out [B, H, d] fp32."""
    B, H, Lmax, d, dt = _decode_checks(q, kcache, vcache, rho, seqlens)
    _check("gate", gate, torch.float32, (H,), q.device)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (B, H, d), q.device)
    if workspace is None:
        wsb = decode_workspace_bytes(B, H, Lmax, d, split_keys)
        workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    _launch(q.device, "parallax_decode", _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(rho),
            _ptr(gate), _ptr(out), _ptr(seqlens), B, H, Lmax, d, _scale(scale, d), _DT[dt],
            int(split_keys), _ptr(workspace), wsb)
    return out


def decode_noalloc(q, kcache, vcache, rho, gate, seqlens, scale=None, split_keys=0, out=None):
    """decode through parallax_decode_noalloc: no workspace, the split records
    go to the library's fixed per-device scratch.  `out` must be given by a
    caller that allocates nothing per call."""
    B, H, Lmax, d, dt = _decode_checks(q, kcache, vcache, rho, seqlens)
    _check("gate", gate, torch.float32, (H,), q.device)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (B, H, d), q.device)
    _launch(q.device, "parallax_decode_noalloc", _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(rho),
            _ptr(gate), _ptr(out), _ptr(seqlens), B, H, Lmax, d, _scale(scale, d), _DT[dt],
            int(split_keys))
    return out


def decode_noalloc_max_bytes():
    """Bytes of split records parallax_decode_noalloc can hold."""
    return int(lib().parallax_decode_noalloc_max_bytes())


def softmax_decode(q, kcache, vcache, seqlens, scale=None, split_keys=0, out=None,
                   workspace=None):
    """One softmax-attention decode step through the decode kernels with the
    correction branch compiled out.  Arguments as for decode, without rho and
    gate.  Returns out [B, H, d] fp32."""
    B, H, Lmax, d, dt = _decode_checks(q, kcache, vcache, None, seqlens)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    _check("out", out, torch.float32, (B, H, d), q.device)
    if workspace is None:
        wsb = decode_workspace_bytes(B, H, Lmax, d, split_keys)
        workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    _launch(q.device, "parallax_softmax_decode", _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(out),
            _ptr(seqlens), B, H, Lmax, d, _scale(scale, d), _DT[dt], int(split_keys),
            _ptr(workspace), wsb)
    return out


def decode_partials(q, kcache, vcache, rho, seqlens, split_keys, scale=None, partials=None):
    """First stage of decode: per-split partial records [B, H, S, 2d+4] fp32."""
    B, H, Lmax, d, dt = _decode_checks(q, kcache, vcache, rho, seqlens)
    split_keys = _split(split_keys)
    S = -(-Lmax // split_keys)
    if partials is None:
        partials = torch.empty((B, H, S, 2 * d + 4), dtype=torch.float32, device=q.device)
    _check("partials", partials, torch.float32, (B, H, S, 2 * d + 4), q.device)
    _launch(q.device, "parallax_decode_partials", _ptr(q), _ptr(kcache), _ptr(vcache),
            _ptr(rho), _ptr(seqlens), _ptr(partials), B, H, Lmax, d, _scale(scale, d),
            _DT[dt], split_keys)
    return partials


def decode_combine(partials, gate, seqlens, Lmax, split_keys, out=None):
    """Second stage of decode: merge the partial records into out [B, H, d]."""
    _check("partials", partials, torch.float32)
    if partials.dim() != 4:
        raise ValueError("partials must be [B, H, S, 2d+4]")
    split_keys = _split(split_keys)
    B, H, S, w = partials.shape
    d = (w - 4) // 2
    _check("gate", gate, torch.float32, (H,), partials.device)
    _check("seqlens", seqlens, torch.int32, (B,), partials.device)
    if S != -(-Lmax // split_keys):
        raise ValueError("partials do not match Lmax / split_keys")
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=partials.device)
    _check("out", out, torch.float32, (B, H, d), partials.device)
    _launch(partials.device, "parallax_decode_combine", _ptr(partials), _ptr(gate),
            _ptr(seqlens), _ptr(out), B, H, Lmax, d, split_keys)
    return out


class ParallaxAttentionFunction(torch.autograd.Function):
    """Autograd wrapper of the causal bf16 prefill: the forward pass runs
    prefill_train (saving lse, rbar and the correction vector), the backward
    pass runs prefill_backward.  Gradients come back in the inputs' dtypes."""

    @staticmethod
    def forward(ctx, q, k, v, rho, gate, scale):
        out, lse, rbar, corr = prefill_train(q, k, v, rho, gate, scale=scale)
        ctx.save_for_backward(q, k, v, rho, gate, out, corr, lse, rbar)
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, rho, gate, out, corr, lse, rbar = ctx.saved_tensors
        dq, dk, dv, drho, dgate = prefill_backward(q, k, v, rho, gate, out, corr, lse, rbar,
                                                   dout.contiguous(), scale=ctx.scale)
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), drho.to(rho.dtype),
                dgate.to(gate.dtype), None)


def parallax_attention(q, k, v, rho, gate, scale=None):
    """Differentiable causal Parallax attention (bf16 q, k, v, rho [B,H,L,d];
    fp32 gate [H]).  Returns out [B,H,L,d] fp32."""
    return ParallaxAttentionFunction.apply(q, k, v, rho, gate, scale)
