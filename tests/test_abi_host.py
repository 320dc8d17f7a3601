"""Host-side checks of the C ABI: no GPU needed.

The library must load, export every function include/parallax.h declares, and
reject bad arguments with the documented status before touching the GPU (the
validation runs before any HIP call, so these calls are safe without a device).
"""
import ctypes
import os
import re

import pytest

from parallax_local_linear_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "parallax.h")
PLX_OK, PLX_EINVAL, PLX_EUNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(parallax_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        pytest.fail("libparallax.so is not built: run python -m parallax_local_linear_amd.build")
    return _native.lib()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_native.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(_native.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_abi_version(lib):
    text = open(HEADER).read()
    ver = int(re.search(r"#define PARALLAX_ABI_VERSION (\d+)", text).group(1))
    assert lib.parallax_abi_version() == ver


def test_workspace_sizes(lib):
    # bf16 prefill stages V as fp16 in 64-key tiles: B*H*ceil(L/64)*64*d*2 bytes
    assert lib.parallax_prefill_workspace_bytes(4, 16, 4096, 128, 1) == 4 * 16 * 4096 * 128 * 2
    assert lib.parallax_prefill_workspace_bytes(1, 1, 65, 64, 1) == 128 * 64 * 2
    assert lib.parallax_prefill_workspace_bytes(1, 1, 65, 64, 0) == 0      # fp32 needs none
    assert lib.parallax_prefill_workspace_bytes(1, 1, 65, 96, 1) == 0
    # decode: one (2d+4)-float record per split
    assert lib.parallax_decode_workspace_bytes(2, 3, 1000, 128, 256) == 2 * 3 * 4 * 260 * 4
    assert lib.parallax_decode_workspace_bytes(2, 3, 1000, 128, 100) == 0
    c = lib.parallax_decode_default_split(64, 16, 8192, 128)
    assert c > 0 and c % 64 == 0


NULL = None


def _prefill(lib, q=1, d=128, L=16, dtype=1, ws=NULL, wsb=0, B=1, H=1):
    p = ctypes.c_void_p(0x1000) if q else NULL
    x = ctypes.c_void_p(0x1000)
    return lib.parallax_prefill(p, x, x, x, x, x, B, H, L, d, 0.0, dtype, ws, wsb, NULL)


def test_prefill_rejects_bad_arguments(lib):
    assert _prefill(lib, q=0) == PLX_EINVAL
    assert b"null" in lib.parallax_last_error()
    assert _prefill(lib, d=96) == PLX_EUNSUPPORTED
    assert _prefill(lib, L=0) == PLX_EINVAL
    assert _prefill(lib, B=-1) == PLX_EINVAL
    assert _prefill(lib, dtype=7) == PLX_EUNSUPPORTED
    # a workspace that is too small is refused before any launch
    assert _prefill(lib, ws=ctypes.c_void_p(0x2000), wsb=10) == PLX_EINVAL
    assert b"workspace" in lib.parallax_last_error()


def test_decode_rejects_bad_arguments(lib):
    x = ctypes.c_void_p(0x1000)
    f = lib.parallax_decode
    assert f(x, x, x, x, x, x, NULL, 1, 1, 64, 128, 0.0, 1, 0, NULL, 0, NULL) == PLX_EINVAL
    assert f(x, x, x, x, x, x, x, 1, 1, 64, 80, 0.0, 1, 0, NULL, 0, NULL) == PLX_EUNSUPPORTED
    assert f(x, x, x, x, x, x, x, 1, 1, 64, 128, 0.0, 1, 100, NULL, 0, NULL) == PLX_EINVAL
    assert f(x, x, x, x, x, x, x, 1, 1, 64, 128, 0.0, 1, -64, NULL, 0, NULL) == PLX_EINVAL
    assert f(x, x, x, x, x, x, x, 1, 1, 0, 128, 0.0, 1, 0, NULL, 0, NULL) == PLX_EINVAL
    assert f(x, x, x, x, x, x, x, 1, 1, 640, 128, 0.0, 1, 64, x, 16, NULL) == PLX_EINVAL
    g = lib.parallax_decode_partials
    assert g(x, x, x, x, x, x, 1, 1, 64, 128, 0.0, 1, 0, NULL) == PLX_EINVAL
    h = lib.parallax_decode_combine
    assert h(x, x, x, NULL, 1, 1, 64, 128, 64, NULL) == PLX_EINVAL


def test_decode_noalloc_rejects_bad_arguments(lib):
    x = ctypes.c_void_p(0x1000)
    f = lib.parallax_decode_noalloc
    assert lib.parallax_decode_noalloc_max_bytes() == 32 << 20
    assert f(x, x, x, x, x, x, NULL, 1, 1, 64, 128, 0.0, 1, 0, NULL) == PLX_EINVAL
    assert f(x, x, x, x, x, x, x, 1, 1, 64, 80, 0.0, 1, 0, NULL) == PLX_EUNSUPPORTED
    assert f(x, x, x, x, x, x, x, 1, 1, 64, 128, 0.0, 1, 100, NULL) == PLX_EINVAL
    assert f(x, x, x, x, x, x, x, 1, 1, 64, 128, 0.0, 3, 0, NULL) == PLX_EUNSUPPORTED
    # records beyond the fixed scratch are refused in validation, before any HIP call
    B, H, Lmax, d = 64, 16, 131072, 128
    assert lib.parallax_decode_workspace_bytes(B, H, Lmax, d, 64) > \
        lib.parallax_decode_noalloc_max_bytes()
    assert f(x, x, x, x, x, x, x, B, H, Lmax, d, 0.0, 1, 64, NULL) == PLX_EINVAL
    assert b"scratch" in lib.parallax_last_error()


def test_softmax_calls_reject_bad_arguments(lib):
    x = ctypes.c_void_p(0x1000)
    f = lib.parallax_softmax_prefill
    assert f(NULL, x, x, x, 1, 1, 64, 128, 0.0, 1, NULL, 0, NULL) == PLX_EINVAL
    assert b"parallax_softmax_prefill" in lib.parallax_last_error()
    assert f(x, x, x, x, 1, 1, 64, 48, 0.0, 1, NULL, 0, NULL) == PLX_EUNSUPPORTED
    assert f(x, x, x, x, 1, 1, 64, 128, 0.0, 1, x, 100, NULL) == PLX_EINVAL
    g = lib.parallax_softmax_prefill_attend
    assert g(x, x, x, NULL, 1, 1, 64, 128, 0.0, NULL) == PLX_EINVAL
    h = lib.parallax_softmax_decode
    assert h(x, x, x, x, NULL, 1, 1, 64, 128, 0.0, 1, 0, NULL, 0, NULL) == PLX_EINVAL
    assert h(x, x, x, x, x, 1, 1, 64, 128, 0.0, 9, 0, NULL, 0, NULL) == PLX_EUNSUPPORTED
    assert h(x, x, x, x, x, 1, 1, 64, 128, 0.0, 1, 32, NULL, 0, NULL) == PLX_EINVAL


def test_training_and_chunk_calls_reject_bad_arguments(lib):
    x = ctypes.c_void_p(0x1000)
    t = lib.parallax_prefill_train
    assert t(x, x, x, x, x, x, x, x, x, 1, 1, 64, 128, 0.0, 0, NULL, 0, NULL) == PLX_EUNSUPPORTED
    assert t(x, x, x, x, x, x, NULL, x, x, 1, 1, 64, 128, 0.0, 1, NULL, 0, NULL) == PLX_EINVAL
    b = lib.parallax_prefill_backward
    args = [x] * 14 + [NULL]
    assert b(*args, 1, 1, 64, 128, 0.0, 1, NULL, 0, NULL) == PLX_EINVAL
    assert b(*([x] * 15), 1, 1, 64, 128, 0.0, 0, NULL, 0, NULL) == PLX_EUNSUPPORTED
    assert lib.parallax_prefill_backward_workspace_bytes(1, 1, 64, 128) > 0
    c = lib.parallax_prefill_chunk
    assert c(*([x] * 8), 1, 1, 0, 64, 8, 128, 0.0, 1, 0, NULL, 0, NULL) == PLX_EINVAL
    assert c(*([x] * 8), 1, 1, 8, 64, 8, 48, 0.0, 1, 0, NULL, 0, NULL) == PLX_EUNSUPPORTED
    assert c(*([x] * 6), NULL, x, 1, 1, 8, 64, 8, 128, 0.0, 1, 0, NULL, 0, NULL) == PLX_EINVAL
    assert c(*([x] * 8), 1, 1, 8, 64, 8, 128, 0.0, 1, 32, NULL, 0, NULL) == PLX_EINVAL
    assert lib.parallax_prefill_chunk_default_split(1, 4, 4096, 16, 128) == 256
    assert lib.parallax_prefill_chunk_vt_workspace_bytes(1, 4, 8, 4096, 16, 128, 0) == \
        8 * 4 * 16 * (2 * 128 + 4) * 4
    sr = lib.parallax_stage_v_rows
    assert sr(x, NULL, x, x, 1, 1, 8, 64, 8, 128, NULL) == PLX_EINVAL
    assert sr(x, x, x, x, 1, 1, 8, 64, 8, 96, NULL) == PLX_EUNSUPPORTED
    cv = lib.parallax_prefill_chunk_vt
    assert cv(*([x] * 8), 1, 1, 8, 64, 0, 128, 0.0, 1, 0, NULL, 0, NULL) == PLX_EINVAL
    assert cv(*([x] * 8), 1, 1, 8, 64, 8, 128, 0.0, 0, 0, NULL, 0, NULL) == PLX_EUNSUPPORTED


def test_binding_raises_without_library(monkeypatch, tmp_path):
    """The product path has no fallback: a missing library is an error."""
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        _native.lib()


def test_binding_requires_gpu_tensors():
    """Host tensors are refused by the binding before the library is touched."""
    import torch
    import parallax_local_linear_amd as plx
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        plx.prefill(x, x, x, x, torch.ones(1))
    with pytest.raises(ValueError, match="GPU"):
        plx.decode(x[:, :, 0], x, x, x[:, :, 0], torch.ones(1), torch.ones(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        plx.softmax_prefill(x, x, x)
    with pytest.raises(ValueError, match="GPU"):
        plx.softmax_decode(x[:, :, 0], x, x, torch.ones(1, dtype=torch.int32))
