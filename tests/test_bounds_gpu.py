"""No kernel writes outside its outputs, and no kernel writes its inputs.

Every output and workspace is placed inside a larger buffer whose guard bands
(4 KiB on each side) hold a sentinel pattern; after the call the guard bands
must be unchanged, every element of an output must have been written, and the
inputs must be bit-identical to their copies taken before the call.  Calls go
through the raw C ABI with pointers into the guarded buffers.
"""
import pytest
import torch

import workloads as wl
from parallax_local_linear_amd import _native

pytestmark = pytest.mark.gpu

PAD = 4096                      # guard band, bytes (keeps 16-byte alignment)
SENT = 0xA5                     # sentinel byte; as fp32 it reads -2.9e-16, never an output


def _guarded(nbytes):
    buf = torch.full((PAD + nbytes + PAD,), SENT, dtype=torch.uint8, device="cuda")
    return buf, buf.data_ptr() + PAD


def _check_guards(buf, nbytes, what, fully_written=True):
    head, body, tail = buf[:PAD], buf[PAD:PAD + nbytes], buf[PAD + nbytes:]
    assert bool((head == SENT).all()), f"{what}: write before the buffer"
    assert bool((tail == SENT).all()), f"{what}: write past the end of the buffer"
    if fully_written:
        words = body.view(torch.int32)
        assert not bool((words == int.from_bytes(bytes([SENT]) * 4, "little", signed=True)).any()), \
            f"{what}: some elements were never written"


def _snapshot(inp):
    return {k: v.clone() for k, v in inp.items() if torch.is_tensor(v)}


def _unchanged(inp, snap):
    for k, v in snap.items():
        assert torch.equal(inp[k].view(torch.uint8), v.view(torch.uint8)), f"input {k} was modified"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 65, 200])
def test_prefill_writes_stay_in_bounds(dtype, d, L):
    lib = _native.lib()
    B, H = 2, 3
    inp = wl.prefill_inputs(B, H, L, d, dtype, seed=600 + L + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    snap = _snapshot(inp)
    out_bytes = B * H * L * d * 4
    out_buf, out_ptr = _guarded(out_bytes)
    code = _native.PLX_BF16 if dtype == "bf16" else _native.PLX_F32
    ws_bytes = lib.parallax_prefill_workspace_bytes(B, H, L, d, code)
    ws_buf, ws_ptr = _guarded(ws_bytes) if ws_bytes else (None, None)
    st = lib.parallax_prefill(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                              inp["rho"].data_ptr(), inp["gate"].data_ptr(), out_ptr,
                              B, H, L, d, 0.0, code, ws_ptr, ws_bytes,
                              torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(out_buf, out_bytes, "prefill out")
    if ws_buf is not None:
        # the staged V^T covers whole 64-key tiles, zero past L: every byte written
        _check_guards(ws_buf, ws_bytes, "prefill workspace")
    _unchanged(inp, snap)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_writes_stay_in_bounds(dtype, d):
    lib = _native.lib()
    B, H, Lmax, split = 3, 2, 700, 128
    inp = wl.decode_inputs(B, H, Lmax, d, dtype, seed=610 + d, device="cuda",
                           seqlens=[700, 129, 0])
    snap = _snapshot(inp)
    code = _native.PLX_BF16 if dtype == "bf16" else _native.PLX_F32
    out_bytes = B * H * d * 4
    stream = torch.cuda.current_stream().cuda_stream
    # one call with a library-sized workspace
    out_buf, out_ptr = _guarded(out_bytes)
    ws_bytes = lib.parallax_decode_workspace_bytes(B, H, Lmax, d, split)
    ws_buf, ws_ptr = _guarded(ws_bytes)
    st = lib.parallax_decode(inp["q"].data_ptr(), inp["kcache"].data_ptr(),
                             inp["vcache"].data_ptr(), inp["rho"].data_ptr(),
                             inp["gate"].data_ptr(), out_ptr, inp["seqlens"].data_ptr(),
                             B, H, Lmax, d, 0.0, code, split, ws_ptr, ws_bytes, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(out_buf, out_bytes, "decode out")
    # split records exist only for splits that hold keys: the rest may stay unwritten
    _check_guards(ws_buf, ws_bytes, "decode workspace", fully_written=False)
    _unchanged(inp, snap)
    # the two stages separately, into guarded partials
    part_buf, part_ptr = _guarded(ws_bytes)
    out2_buf, out2_ptr = _guarded(out_bytes)
    st = lib.parallax_decode_partials(inp["q"].data_ptr(), inp["kcache"].data_ptr(),
                                      inp["vcache"].data_ptr(), inp["rho"].data_ptr(),
                                      inp["seqlens"].data_ptr(), part_ptr, B, H, Lmax, d, 0.0,
                                      code, split, stream)
    assert st == 0, lib.parallax_last_error()
    st = lib.parallax_decode_combine(part_ptr, inp["gate"].data_ptr(), inp["seqlens"].data_ptr(),
                                     out2_ptr, B, H, Lmax, d, split, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(part_buf, ws_bytes, "decode partials", fully_written=False)
    _check_guards(out2_buf, out_bytes, "decode combine out")
    assert torch.equal(out_buf[PAD:PAD + out_bytes], out2_buf[PAD:PAD + out_bytes])
    _unchanged(inp, snap)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_softmax_writes_stay_in_bounds(dtype, d):
    """The softmax-only entry points: same guard bands; rho and gate are not
    passed at all."""
    lib = _native.lib()
    code = _native.PLX_BF16 if dtype == "bf16" else _native.PLX_F32
    stream = torch.cuda.current_stream().cuda_stream
    B, H, L = 2, 3, 130
    inp = wl.prefill_inputs(B, H, L, d, dtype, seed=630 + d, device="cuda")
    snap = _snapshot(inp)
    out_bytes = B * H * L * d * 4
    out_buf, out_ptr = _guarded(out_bytes)
    ws_bytes = lib.parallax_prefill_workspace_bytes(B, H, L, d, code)
    ws_buf, ws_ptr = _guarded(ws_bytes) if ws_bytes else (None, None)
    st = lib.parallax_softmax_prefill(inp["q"].data_ptr(), inp["k"].data_ptr(),
                                      inp["v"].data_ptr(), out_ptr, B, H, L, d, 0.0, code,
                                      ws_ptr, ws_bytes, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(out_buf, out_bytes, "softmax prefill out")
    if ws_buf is not None:
        _check_guards(ws_buf, ws_bytes, "softmax prefill workspace")
    _unchanged(inp, snap)
    B, H, Lmax, split = 3, 2, 700, 128
    inp = wl.decode_inputs(B, H, Lmax, d, dtype, seed=640 + d, device="cuda",
                           seqlens=[700, 129, 0])
    snap = _snapshot(inp)
    out_bytes = B * H * d * 4
    out_buf, out_ptr = _guarded(out_bytes)
    ws_bytes = lib.parallax_decode_workspace_bytes(B, H, Lmax, d, split)
    ws_buf, ws_ptr = _guarded(ws_bytes)
    st = lib.parallax_softmax_decode(inp["q"].data_ptr(), inp["kcache"].data_ptr(),
                                     inp["vcache"].data_ptr(), out_ptr, inp["seqlens"].data_ptr(),
                                     B, H, Lmax, d, 0.0, code, split, ws_ptr, ws_bytes, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(out_buf, out_bytes, "softmax decode out")
    _check_guards(ws_buf, ws_bytes, "softmax decode workspace", fully_written=False)
    _unchanged(inp, snap)


@pytest.mark.parametrize("d", [64, 128])
def test_training_writes_stay_in_bounds(d):
    """Training forward and backward: guard bands around every output and
    workspace, every element written, inputs unmodified."""
    lib = _native.lib()
    stream = torch.cuda.current_stream().cuda_stream
    B, H, L = 2, 3, 130
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=650 + d, device="cuda", rho_std=0.5,
                            gate=("uniform", 0.2, 1.0))
    snap = _snapshot(inp)
    nf, nr = B * H * L * d * 4, B * H * L * 4
    bufs = {n: _guarded(nb) for n, nb in (("out", nf), ("lse", nr), ("rbar", nr), ("corr", nf))}
    fws = lib.parallax_prefill_workspace_bytes(B, H, L, d, _native.PLX_BF16)
    fbuf, fptr = _guarded(fws)
    st = lib.parallax_prefill_train(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                                    inp["rho"].data_ptr(), inp["gate"].data_ptr(),
                                    *(bufs[n][1] for n in ("out", "lse", "rbar", "corr")),
                                    B, H, L, d, 0.0, _native.PLX_BF16, fptr, fws, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    for n, nb in (("out", nf), ("lse", nr), ("rbar", nr), ("corr", nf)):
        _check_guards(bufs[n][0], nb, "train " + n)
    _check_guards(fbuf, fws, "train workspace")
    _unchanged(inp, snap)
    dout = torch.randn((B, H, L, d), device="cuda")
    grads = {n: _guarded(nb) for n, nb in (("dq", nf), ("dk", nf), ("dv", nf), ("drho", nf),
                                          ("dgate", H * 4))}
    bws = lib.parallax_prefill_backward_workspace_bytes(B, H, L, d)
    bbuf, bptr = _guarded(bws)
    saved = [bufs[n][1] for n in ("out", "corr", "lse", "rbar")]
    st = lib.parallax_prefill_backward(inp["q"].data_ptr(), inp["k"].data_ptr(),
                                       inp["v"].data_ptr(), inp["rho"].data_ptr(),
                                       inp["gate"].data_ptr(), *saved, dout.data_ptr(),
                                       *(grads[n][1] for n in ("dq", "dk", "dv", "drho", "dgate")),
                                       B, H, L, d, 0.0, _native.PLX_BF16, bptr, bws, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    for n, nb in (("dq", nf), ("dk", nf), ("dv", nf), ("drho", nf), ("dgate", H * 4)):
        _check_guards(grads[n][0], nb, "backward " + n)
    # the workspace holds padded tiles and alignment gaps: only its bounds are checked
    _check_guards(bbuf, bws, "backward workspace", fully_written=False)
    _unchanged(inp, snap)


@pytest.mark.parametrize("ctx,n", [([70, 0, 5], [20, 90, 1]), ([70, 0, 130], [16, 9, 1]),
                                   ([70, 0, 130], [16, 9, 30]), ([70, 0, 130], [40, 9, 64])],
                         ids=["staged", "fused1", "fused2", "fused4"])
@pytest.mark.parametrize("split", [0, 64])
def test_chunk_writes_stay_in_bounds(split, ctx, n):
    """Per-call call and the staged-cache call, whole-prefix (split 0 is no
    split at this size) and split-KV (4 splits of 64 keys).  Chunks of up to 90
    queries stage V^T per call; chunks of at most 64 queries at d = 128 convert
    the V tiles in the kernel (no V^T workspace), with one, two or four busy
    waves."""
    lib = _native.lib()
    stream = torch.cuda.current_stream().cuda_stream
    H, d = 2, 128
    inp = wl.chunk_inputs(H, d, ctx, n, seed=660, device="cuda", Lmax=200)
    snap = _snapshot(inp)
    T = inp["T"]
    ob, op = _guarded(T * H * d * 4)
    ws = lib.parallax_prefill_chunk_workspace_bytes(3, H, T, 200, inp["max_q"], d, split)
    assert (ws == 0) == (inp["max_q"] <= 64 and split == 0)
    ws = max(ws, 256)
    wb, wp = _guarded(ws)
    st = lib.parallax_prefill_chunk(inp["q"].data_ptr(), inp["kcache"].data_ptr(),
                                    inp["vcache"].data_ptr(), inp["rho"].data_ptr(),
                                    inp["gate"].data_ptr(), op, inp["cu_q"].data_ptr(),
                                    inp["ctx"].data_ptr(), 3, H, T, 200, inp["max_q"], d, 0.0,
                                    _native.PLX_BF16, split, wp, ws, stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(ob, T * H * d * 4, "chunk out")
    # only the V^T tiles of cache rows the chunks read are staged, and a split
    # writes only the records of splits that reach a row
    _check_guards(wb, ws, "chunk workspace", fully_written=False)
    import parallax_local_linear_amd as plx
    vt = plx.prefill_stage_v(inp["vcache"])
    ob2, op2 = _guarded(T * H * d * 4)
    rws = lib.parallax_prefill_chunk_vt_workspace_bytes(3, H, T, 200, inp["max_q"], d, split)
    assert (rws > 0) == (split == 64)
    rb, rp = _guarded(max(rws, 256))
    st = lib.parallax_prefill_chunk_vt(inp["q"].data_ptr(), inp["kcache"].data_ptr(),
                                       vt.data_ptr(), inp["rho"].data_ptr(),
                                       inp["gate"].data_ptr(), op2, inp["cu_q"].data_ptr(),
                                       inp["ctx"].data_ptr(), 3, H, T, 200, inp["max_q"], d, 0.0,
                                       _native.PLX_BF16, split, rp, max(rws, 256), stream)
    assert st == 0, lib.parallax_last_error()
    torch.cuda.synchronize()
    _check_guards(ob2, T * H * d * 4, "chunk_vt out")
    _check_guards(rb, max(rws, 256), "chunk_vt records", fully_written=False)
    _unchanged(inp, snap)


def test_nan_in_a_query_row_stays_in_that_row():
    """A NaN in one query row turns that output row into NaN.  Rows outside its
    16-row block (one wave) are bit-identical to a clean run; rows inside it
    agree within the parity tolerance (the wave's shared rescale schedule may
    differ, which moves the fp16 rounding of P)."""
    import parallax_local_linear_amd as plx
    inp = wl.prefill_inputs(1, 2, 130, 128, "bf16", seed=620, device="cuda", rho_std=0.5)
    clean = plx.prefill(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"])
    q = inp["q"].clone()
    q[0, 1, 70, 5] = float("nan")
    out = plx.prefill(q, inp["k"], inp["v"], inp["rho"], inp["gate"])
    torch.cuda.synchronize()
    assert bool(torch.isnan(out[0, 1, 70]).all())
    block = torch.zeros(out.shape[:3], dtype=torch.bool, device="cuda")
    block[0, 1, 64:80] = True
    block[0, 1, 70] = False
    other = torch.ones_like(block)
    other[0, 1, 64:80] = False
    assert torch.equal(out[other], clean[other])
    assert bool(torch.isfinite(out[block]).all())
    assert float((out[block] - clean[block]).abs().max()) <= 2e-2


def test_nan_in_a_cache_row_stays_in_its_stream():
    """A NaN key inside one stream's valid range poisons that stream only; the
    other streams are bit-identical to a clean run."""
    import parallax_local_linear_amd as plx
    inp = wl.decode_inputs(2, 2, 300, 128, "bf16", seed=621, device="cuda", seqlens=[300, 200])
    clean = plx.decode(inp["q"], inp["kcache"], inp["vcache"], inp["rho"], inp["gate"],
                       inp["seqlens"], split_keys=128)
    kc = inp["kcache"].clone()
    kc[1, 0, 150, 3] = float("nan")
    out = plx.decode(inp["q"], kc, inp["vcache"], inp["rho"], inp["gate"], inp["seqlens"],
                     split_keys=128)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out[1, 0]).all())
    for b, h in [(0, 0), (0, 1), (1, 1)]:
        assert torch.equal(out[b, h], clean[b, h])
