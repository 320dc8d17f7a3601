"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream), for callers that run under graph
capture.  With the caller's workspace the step is two kernel launches and
nothing else (no allocation, no memset), so it can be captured once and
replayed with new queries written into the same buffers.  Every replay must
equal, bit for bit, the same step run eagerly on the same inputs, with eager
work and synchronisations between the replays."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def _plx():
    import parallax_local_linear_amd as plx
    return plx


@pytest.mark.parametrize("corr", [True, False], ids=["parallax", "softmax"])
def test_decode_graph_replays_match_eager(corr):
    plx = _plx()
    B, H, Lmax, d = 2, 16, 3000, 128
    inp = wl.decode_inputs(B, H, Lmax, d, "bf16", seed=1500, device="cuda",
                           len_range=(1000, 3000))
    ws = torch.empty(plx.decode_workspace_bytes(B, H, Lmax, d), dtype=torch.uint8,
                     device="cuda")

    def step(out):
        if corr:
            return plx.decode(inp["q"], inp["kcache"], inp["vcache"], inp["rho"], inp["gate"],
                              inp["seqlens"], out=out, workspace=ws)
        return plx.softmax_decode(inp["q"], inp["kcache"], inp["vcache"], inp["seqlens"],
                                  out=out, workspace=ws)

    out_g = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out_g)                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda").manual_seed(1501)
    prev = None
    for r in range(5):
        # the next step's query (and probe) written into the captured buffers
        inp["q"].copy_(torch.randn(inp["q"].shape, generator=gen, device="cuda"))
        if corr:
            inp["rho"].copy_(0.1 * torch.randn(inp["rho"].shape, generator=gen, device="cuda"))
        g.replay()
        torch.cuda.synchronize()
        got = out_g.clone()
        ref = step(torch.empty_like(out_g))           # eager, same inputs and workspace
        torch.cuda.synchronize()
        print(f"replay {r}: max |out| {float(got.abs().max()):.3f}", flush=True)
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"replay {r} differs from the eager step"
        if prev is not None:
            assert not torch.equal(got, prev)         # the replay read the new query
        prev = got
