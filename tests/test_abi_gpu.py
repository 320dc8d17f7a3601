"""GPU checks through the raw C ABI (ctypes, no binding helpers).

Covers the paths the Python binding does not take: a NULL workspace (the
library allocates and frees its scratch on the stream), a non-default scale,
the default stream, and a launch-time status of PLX_OK with an empty error
string.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import parallax_oracle as po
from parallax_local_linear_amd import _native

pytestmark = pytest.mark.gpu


def _lib():
    return _native.lib()


def test_prefill_null_workspace_and_scale():
    lib = _lib()
    inp = wl.prefill_inputs(2, 3, 200, 128, "bf16", seed=31, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    out = torch.full(inp["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    scale = 0.05
    st = lib.parallax_prefill(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                              inp["rho"].data_ptr(), inp["gate"].data_ptr(), out.data_ptr(),
                              2, 3, 200, 128, scale, _native.PLX_BF16, None, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert st == 0 and lib.parallax_last_error() == b""
    torch.cuda.synchronize()
    h = {k: v.cpu() for k, v in inp.items()}
    ref = po.prefill(h["q"], h["k"], h["v"], h["rho"], h["gate"], scale=scale)
    assert float(np.max(np.abs(out.cpu().double().numpy() - ref))) <= 2e-2


def test_decode_null_workspace_default_stream():
    lib = _lib()
    inp = wl.decode_inputs(3, 2, 700, 64, "bf16", seed=32, device="cuda",
                           seqlens=[700, 65, 1])
    out = torch.full((3, 2, 64), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    st = lib.parallax_decode(inp["q"].data_ptr(), inp["kcache"].data_ptr(),
                             inp["vcache"].data_ptr(), inp["rho"].data_ptr(),
                             inp["gate"].data_ptr(), out.data_ptr(), inp["seqlens"].data_ptr(),
                             3, 2, 700, 64, 0.0, _native.PLX_BF16, 0, None, 0, None)
    assert st == 0
    torch.cuda.synchronize()
    h = {k: v.cpu() for k, v in inp.items()}
    ref = po.decode(h["q"], h["kcache"], h["vcache"], h["rho"], h["gate"], h["seqlens"])
    assert float(np.max(np.abs(out.cpu().double().numpy() - ref))) <= 2e-2


def test_decode_seqlens_clamped_on_device():
    """seqlens beyond Lmax are clamped to Lmax and negative ones to 0."""
    import parallax_local_linear_amd as plx
    inp = wl.decode_inputs(3, 1, 130, 128, "bf16", seed=33, device="cuda",
                           seqlens=[500, -4, 130])
    out = plx.decode(inp["q"], inp["kcache"], inp["vcache"], inp["rho"], inp["gate"],
                     inp["seqlens"])
    torch.cuda.synchronize()
    h = {k: v.cpu() for k, v in inp.items()}
    ref = po.decode(h["q"], h["kcache"], h["vcache"], h["rho"], h["gate"], [130, 0, 130])
    got = out.cpu().double().numpy()
    assert np.all(got[1] == 0.0)
    assert float(np.max(np.abs(got - ref))) <= 2e-2


def test_binding_rejects_bad_arguments():
    """The torch binding refuses mismatched tensors before calling the library."""
    import parallax_local_linear_amd as plx
    inp = wl.prefill_inputs(1, 2, 64, 64, "bf16", seed=34, device="cuda")
    with pytest.raises(ValueError):
        plx.prefill(inp["q"], inp["k"][:, :, :32].contiguous(), inp["v"], inp["rho"], inp["gate"])
    with pytest.raises(TypeError):
        plx.prefill(inp["q"], inp["k"].float(), inp["v"], inp["rho"], inp["gate"])
    with pytest.raises(ValueError):
        plx.prefill(inp["q"], inp["k"].transpose(2, 3), inp["v"], inp["rho"], inp["gate"])
    with pytest.raises(ValueError):
        plx.prefill_stage_v(inp["v"][0])
    dec = wl.decode_inputs(2, 2, 128, 64, "bf16", seed=35, device="cuda")
    for bad in (0, 100, -64):
        with pytest.raises(ValueError):
            plx.decode_partials(dec["q"], dec["kcache"], dec["vcache"], dec["rho"],
                                dec["seqlens"], bad)
    with pytest.raises(plx.ParallaxError):
        plx.decode(dec["q"], dec["kcache"], dec["vcache"], dec["rho"], dec["gate"],
                   dec["seqlens"], split_keys=100)
    torch.cuda.synchronize()
