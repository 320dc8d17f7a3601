"""parallax_decode_noalloc (no workspace, the library's fixed per-device
scratch) against parallax_decode with a workspace, through the raw C ABI.

Two calls in a row, the second with a smaller input: each must match
parallax_decode bit for bit at the same split (the same kernels read the same
records), and both against the fp64 oracle within the decode bound.  A call
whose records exceed the scratch is rejected before anything is enqueued
(checked on the host, in test_abi_host.py).
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import parallax_oracle as po
from parallax_local_linear_amd import _native

pytestmark = pytest.mark.gpu


def _call(fn, *args):
    lib = _native.lib()
    st = getattr(lib, fn)(*args)
    return st, lib.parallax_last_error().decode()


def _args(inp, out, split):
    B, H, Lmax, d = inp["kcache"].shape
    return (inp["q"].data_ptr(), inp["kcache"].data_ptr(), inp["vcache"].data_ptr(),
            inp["rho"].data_ptr(), inp["gate"].data_ptr(), out.data_ptr(),
            inp["seqlens"].data_ptr(), B, H, Lmax, d, ctypes.c_float(0.0), _native.PLX_BF16,
            split)


def _reference(inp, split):
    """parallax_decode with a caller workspace at the same split."""
    lib = _native.lib()
    B, H, Lmax, d = inp["kcache"].shape
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    nb = lib.parallax_decode_workspace_bytes(B, H, Lmax, d, split)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    st, msg = _call("parallax_decode", *_args(inp, out, split)[:-1], split, ws.data_ptr(), nb,
                    None)
    assert st == 0, msg
    return out


@pytest.mark.parametrize("dtype", ["bf16"])
def test_noalloc_matches_decode_twice(dtype):
    lib = _native.lib()
    cases = [  # (B, H, Lmax, d, seqlens, split): the second is smaller
        (8, 16, 20000, 128, [20000, 1, 0, 19999, 7000, 64, 65, 12345], 0),
        (3, 4, 700, 64, [700, 333, 0], 128),
    ]
    for i, (B, H, Lmax, d, sl, split) in enumerate(cases):
        print(f"noalloc call {i}: B{B} H{H} Lmax{Lmax} d{d} split {split}", flush=True)
        inp = wl.decode_inputs(B, H, Lmax, d, dtype, seed=900 + i, device="cuda", rho_std=0.5,
                               gate=("uniform", 0.2, 1.0), seqlens=sl)
        C = split if split else lib.parallax_decode_default_split(B, H, Lmax, d)
        assert lib.parallax_decode_workspace_bytes(B, H, Lmax, d, C) <= \
            lib.parallax_decode_noalloc_max_bytes()
        out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device="cuda")
        st, msg = _call("parallax_decode_noalloc", *_args(inp, out, split), None)
        assert st == 0, msg
        ref = _reference(inp, C)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i}: differs from parallax_decode"
        h = {k: v.cpu() for k, v in inp.items()}
        orc = po.decode(h["q"], h["kcache"], h["vcache"], h["rho"], h["gate"], h["seqlens"])
        err = float(np.max(np.abs(out.cpu().double().numpy() - orc)))
        print(f"noalloc call {i}: max-abs vs oracle {err:.3e}", flush=True)
        assert err <= 2e-2
        assert all(bool((out[b] == 0).all()) for b in range(B) if sl[b] == 0)
