"""The prefill, a chunked-prefill serving step and a training step (forward and
backward) captured in HIP graphs (torch.cuda.CUDAGraph over the library's
launches on the capture stream).  With
the caller's workspace every call is kernel launches only (no allocation, no
memset), so a step can be captured once and replayed with new inputs written
into the same buffers.  Each replay must equal, bit for bit, the same calls run
eagerly on the same inputs, with eager work and synchronisations between the
replays."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def _plx():
    import parallax_local_linear_amd as plx
    return plx


def _capture(step):
    """Warm the step up on a side stream, then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _fill(t, gen, std=1.0):
    t.copy_((std * torch.randn(t.shape, generator=gen, device="cuda")).to(t.dtype))


def test_prefill_graph_replays_match_eager():
    """V staging and the fused kernel of a ragged bf16 prefill (L = 1000, not a
    multiple of the 64-key tile) in one graph."""
    plx = _plx()
    B, H, L, d = 1, 4, 1000, 128
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=1600, device="cuda",
                            gate=("uniform", 0.2, 1.0))
    vt = torch.empty(plx.prefill_workspace_bytes(B, H, L, d), dtype=torch.uint8, device="cuda")
    out_g = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")

    def step(out=out_g):
        plx.prefill_stage_v(inp["v"], vt)
        plx.prefill_attend(inp["q"], inp["k"], vt, inp["rho"], inp["gate"], out=out)

    g = _capture(step)
    gen = torch.Generator(device="cuda").manual_seed(1601)
    prev = None
    for r in range(4):
        for name in ("q", "k", "v"):
            _fill(inp[name], gen)
        _fill(inp["rho"], gen, 0.1)
        g.replay()
        torch.cuda.synchronize()
        got = out_g.clone()
        ref = torch.empty_like(out_g)
        step(ref)
        torch.cuda.synchronize()
        print(f"prefill replay {r}: max |out| {float(got.abs().max()):.3f}", flush=True)
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"replay {r} differs from the eager calls"
        if prev is not None:
            assert not torch.equal(got, prev)
        prev = got


@pytest.mark.parametrize("split", [0, 512], ids=["unsplit", "split512"])
def test_chunk_serving_step_graph_replays_match_eager(split):
    """One serving step against a caller-kept staged V cache: re-stage the tiles of
    the appended rows, then the chunked prefill (split-KV with split = 512), in one
    graph.  Between replays the test writes new appended K/V rows, queries and
    probes into the captured buffers, as a serving loop would."""
    plx = _plx()
    H, d = 8, 128
    ctx, n = [700, 1500], [20, 45]
    inp = wl.chunk_inputs(H, d, ctx, n, "bf16", seed=1610, device="cuda")
    B, Lmax, T, max_q = len(ctx), inp["kcache"].shape[2], inp["T"], inp["max_q"]
    kc, vc = inp["kcache"], inp["vcache"]
    vt = plx.chunk_vt_cache(B, H, Lmax, d, "cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    full = torch.tensor([0, ctx[0] + n[0], sum(ctx) + sum(n)], dtype=torch.int32, device="cuda")
    plx.stage_v_rows(vc, vt, full, zero, max(c + m for c, m in zip(ctx, n)), int(full[-1]))
    sk = split if split else (Lmax + 63) // 64 * 64
    wsb = int(plx.lib().parallax_prefill_chunk_vt_workspace_bytes(B, H, T, Lmax, max_q, d, sk))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    out_g = torch.empty((T, H, d), dtype=torch.float32, device="cuda")

    def step(out=out_g):
        plx.stage_v_rows(vc, vt, inp["cu_q"], inp["ctx"], max_q, T)
        plx.prefill_chunk(inp["q"], kc, None, inp["rho"], inp["gate"], inp["cu_q"], inp["ctx"],
                          max_q, out=out, workspace=ws, vt_cache=vt, split_keys=sk)

    g = _capture(step)
    gen = torch.Generator(device="cuda").manual_seed(1611)
    prev = None
    for r in range(4):
        for b in range(B):
            rows = slice(ctx[b], ctx[b] + n[b])
            _fill(kc[b, :, rows], gen)
            _fill(vc[b, :, rows], gen)
        _fill(inp["q"], gen)
        _fill(inp["rho"], gen, 0.1)
        g.replay()
        torch.cuda.synchronize()
        got = out_g.clone()
        ref = torch.empty_like(out_g)
        step(ref)
        torch.cuda.synchronize()
        print(f"chunk ({split}) replay {r}: max |out| {float(got.abs().max()):.3f}", flush=True)
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"replay {r} differs from the eager calls"
        if prev is not None:
            assert not torch.equal(got, prev)
        prev = got


def test_training_step_graph_replays_match_eager():
    """The training forward (which saves the statistics) and the backward pass of a
    ragged bf16 prefill in one graph; the captured forward's outputs are the
    graph's own buffers.  Each replay's output and five gradients must equal the
    eager calls' bit for bit."""
    plx = _plx()
    B, H, L, d = 1, 2, 300, 128
    inp = wl.prefill_inputs(B, H, L, d, "bf16", seed=1620, device="cuda",
                            gate=("uniform", 0.2, 1.0))
    dout = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    fws = torch.empty(plx.prefill_workspace_bytes(B, H, L, d), dtype=torch.uint8, device="cuda")
    bws = torch.empty(plx.prefill_backward_workspace_bytes(B, H, L, d), dtype=torch.uint8,
                      device="cuda")

    def new_grads():
        return tuple(torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
                     for _ in range(4)) + (torch.empty(H, dtype=torch.float32, device="cuda"),)

    grads_g = new_grads()
    saved = {}

    def step(grads=grads_g):
        fwd = plx.prefill_train(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"],
                                workspace=fws)
        out, lse, rbar, corr = fwd
        plx.prefill_backward(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"], out, corr,
                             lse, rbar, dout, grads=grads, workspace=bws)
        return fwd

    gen = torch.Generator(device="cuda").manual_seed(1621)
    _fill(dout, gen)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        saved["fwd"] = step()
    torch.cuda.synchronize()

    prev = None
    for r in range(3):
        for name in ("q", "k", "v"):
            _fill(inp[name], gen)
        _fill(inp["rho"], gen, 0.1)
        _fill(dout, gen)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in saved["fwd"]] + [t.clone() for t in grads_g]
        ref_grads = new_grads()
        ref = list(step(ref_grads)) + list(ref_grads)
        torch.cuda.synchronize()
        print(f"training replay {r}: max |dq| {float(got[4].abs().max()):.3f}", flush=True)
        for i, (x, y) in enumerate(zip(got, ref)):
            assert torch.isfinite(x).all(), i
            assert torch.equal(x, y), f"replay {r}: tensor {i} differs from the eager calls"
        if prev is not None:
            assert not torch.equal(got[4], prev)
        prev = got[4]
