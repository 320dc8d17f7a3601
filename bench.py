"""Benchmark of the Parallax forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
                    [--no-softmax] [--no-backward] [--no-chunk] [--no-sweep]
                    [--no-gemm-ref]

One step is one pass of the whole hot path over resident synthetic inputs:
  1. bf16 causal prefill, B=4 H=16 L=4096 d=128 (V staging + fused kernel);
  2. bf16 decode, B=64 H=16 d=128, 8192 cached keys per sequence
     (split-KV partials + combine).
Every launch is bracketed by HIP events on the stream it runs on (torch's
current stream, which the library is handed).  Per kernel the line reports the
median, mean, min and max over the timed steps and the spread (max - min) /
median.  `value` is the prefill throughput in TFLOP/s: algorithmic flops
8*d*B*H*L(L+1)/2 over the median per-step time of both prefill kernels.  The
decode throughput in GB/s (algorithmic bytes: K and V over the valid lengths
plus q, rho, out, gate, seqlens) is reported beside it.

`roofline` describes the kernel that `value` measures, the fused prefill
kernel, against the bf16 MFMA peak.  The step's longest kernel is the decode
split pass (HBM-bound); its roofline is `decode.roofline`.  `rooflines` lists
every timed hot-path kernel on every full-size workload, each with the HBM
bytes its rocprofv3 counters read (`traffic`, null when no counter
measurement matches the current kernel source).

Unless --no-extra is given, the two other full-size workloads (long ragged
decode and the d=64 prefill) are timed too and reported under "extra".
"backward" times the training forward pass (which also saves the statistics
the gradient needs) and the backward pass on the prefill workloads; its
TFLOP/s count 16*d flops per causal pair (S and R recomputed, dO V^T, and the
dV, dK (two), dQ and drho products), twice the forward's 8*d.
"chunk" times the chunked prefill against a KV cache on three shapes: long
chunks on a 4096-key context (TFLOP/s), and 16-query chunks on an 8192-key
context for 32 and for 2 sequences (HBM GB/s of the cache rows read; the
2-sequence case runs split-KV, "split_keys" per range); "staged_cache" is the
serving loop that keeps the staged V cache and re-stages only the appended
rows' tiles.
"softmax_relative" times the same kernels with the correction branch compiled
out (plain causal softmax attention) against the Parallax kernels on each
workload, alternating the two launch by launch, and reports the time ratio;
"softmax_sweep" does the same over batch sizes and context lengths (prefill
L 1k-64k at d 64 and 128, decode B 1-64 x L 8k-128k).
"mfma_reference" times the vendor bf16 GEMM (torch.matmul, 8192^3) alternately
with the fused prefill kernel: on this power-limited chip it shows what share of
the published MFMA peak bf16 matrix work reaches at all on the same box.
The CPU baseline times the fp64 oracle on a bounded sample on the host.
"checksums" holds the fp64 sum of every input tensor of the step.
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("Parallax decode HBM GB/s (% of peak) + prefill TFLOP/s (% bf16 MFMA peak)")
PEAK_MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, published
PEAK_HBM_GBS = 8000.0               # MI355X HBM3E, published
SWEEP_AHEAD = 200000                # spin cycles queued before each timed sweep call
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {   # the files whose text determines each kernel's code
    "prefill_bf16_kernel": ["parallax_local_linear_amd/csrc/prefill_bf16.hip",
                            "parallax_local_linear_amd/csrc/plx_common.h"],
    "stage_v_kernel": ["parallax_local_linear_amd/csrc/prefill_bf16.hip",
                       "parallax_local_linear_amd/csrc/plx_common.h"],
    "decode_split_kernel": ["parallax_local_linear_amd/csrc/decode.hip",
                            "parallax_local_linear_amd/csrc/plx_common.h"],
    "decode_combine_kernel": ["parallax_local_linear_amd/csrc/decode.hip",
                              "parallax_local_linear_amd/csrc/plx_common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_sha(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` measured with rocprofv3
    counters for this exact kernel source, or None when no measurement matches
    the current source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not t or t.get("src_sha") != src_sha(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def roofline(kernel, template, workload, bound, work, ms):
    """Roofline object of one kernel: algorithmic work per launch over its
    median launch time, against the MI355X peak of its bound."""
    if bound == "mfma":
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, PEAK_MFMA_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"kernel": template, "workload": workload, "bound": bound,
            "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "ms": round(ms, 4),
            "traffic": traffic(kernel, workload)}


def _median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


class Timer:
    """Per-label lists of HIP-event pairs recorded on the current stream.

    With `ahead` > 0 every timed call is queued behind a spin kernel of that many
    GPU clock cycles, so that the host has submitted the call and its closing
    event before the GPU reaches the opening one: the pair then brackets GPU
    time only, not the host's submission of a call of a few microseconds."""

    def __init__(self, torch, ahead=0):
        self.torch = torch
        self.ev = {}
        self.ahead = ahead

    def run(self, label, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        if self.ahead:
            t.cuda._sleep(self.ahead)
        a.record()
        fn()
        b.record()
        self.ev.setdefault(label, []).append((a, b))

    def times(self, label, skip=0):
        return [a.elapsed_time(b) for a, b in self.ev[label][skip:]]

    def ms(self, label, skip=0):
        """Median launch time in ms."""
        return _median(self.times(label, skip))

    def stats(self, label, skip=0):
        return stats(self.times(label, skip))

    def reset(self):
        self.ev = {}


def stats(xs):
    med = _median(xs)
    return {"median": round(med, 4), "mean": round(sum(xs) / len(xs), 4),
            "min": round(min(xs), 4), "max": round(max(xs), 4),
            "spread": round((max(xs) - min(xs)) / med, 4) if med > 0 else None, "n": len(xs)}


def checksums(inp):
    """fp64 sum of every tensor input (computed on the device, outside timing)."""
    return {k: float(v.double().sum()) for k, v in inp.items() if hasattr(v, "double")}


def cpu_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api')} {p.get('version')} ({p.get('architecture')})"
                threads = p.get("num_threads", threads)
                break
    except Exception:
        pass
    import numpy as np
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": blas,
            "numpy": np.__version__}, threads


def cpu_baseline_prefill(inp, w, budget_s=12.0):
    """fp64 oracle (expanded form) on whole heads of the prefill workload until
    the time budget is spent; TFLOP/s over the same algorithmic count.  The
    device-to-host copy and the bf16 -> fp64 conversion are timed separately."""
    from oracle import parallax_oracle as po
    import workloads as wl
    heads = 0
    t_tot = t_d2h = t_conv = 0.0
    info, threads = cpu_info()
    for idx in range(w.B * w.H):
        b, h = divmod(idx, w.H)
        t0 = time.perf_counter()
        host = {k: inp[k][b, h].cpu() for k in ("q", "k", "v", "rho")}
        t1 = time.perf_counter()
        arrs = {k: x.float().double().numpy() for k, x in host.items()}
        t2 = time.perf_counter()
        g = float(inp["gate"][h])
        t3 = time.perf_counter()
        po.prefill_head(arrs["q"], arrs["k"], arrs["v"], arrs["rho"], g, w.scale)
        t_tot += time.perf_counter() - t3
        t_d2h += t1 - t0
        t_conv += t2 - t1
        heads += 1
        if t_tot >= budget_s:
            break
    flops = wl.prefill_flops(1, heads, w.L, w.d)
    return {"value": flops / t_tot / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of the B{w.B} H{w.H} L{w.L} d{w.d} "
                      f"prefill, fp64 expanded form, {t_tot:.1f}s",
            "oracle_s": round(t_tot, 3), "d2h_s": round(t_d2h, 3),
            "bf16_to_fp64_s": round(t_conv, 3), **info}


def cpu_baseline_decode(inp, w, budget_s=6.0):
    """fp64 oracle on whole decode streams until the time budget is spent."""
    from oracle import parallax_oracle as po
    H, d = w.H, w.d
    n_streams, nbytes = 0, 0
    t_tot = t_d2h = t_conv = 0.0
    info, threads = cpu_info()
    sl = inp["seqlens"].cpu().tolist()
    for idx in range(w.B * H):
        b, h = divmod(idx, H)
        n = sl[b]
        t0 = time.perf_counter()
        host = {"K": inp["kcache"][b, h, :n].cpu(), "V": inp["vcache"][b, h, :n].cpu(),
                "q": inp["q"][b, h].cpu(), "r": inp["rho"][b, h].cpu()}
        t1 = time.perf_counter()
        a = {k: x.float().double().numpy() for k, x in host.items()}
        t2 = time.perf_counter()
        po.decode_stream(a["q"], a["K"], a["V"], a["r"], float(inp["gate"][h]), w.scale)
        t_tot += time.perf_counter() - t2
        t_d2h += t1 - t0
        t_conv += t2 - t1
        n_streams += 1
        nbytes += n * 2 * d * 2 + 2 * d * 2 + d * 4
        if t_tot >= budget_s:
            break
    return {"value": nbytes / t_tot / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_streams} of {w.B * H} streams of the decode workload, fp64, "
                      f"bytes counted as bf16, {t_tot:.1f}s",
            "oracle_s": round(t_tot, 3), "d2h_s": round(t_d2h, 3),
            "bf16_to_fp64_s": round(t_conv, 3), **info}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip workloads 4 and 5")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-softmax", action="store_true",
                    help="skip the timing against the softmax-only kernels")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training forward and backward timing")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked prefill timing")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the softmax-relative sweep over batch sizes and lengths")
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the vendor bf16 GEMM timed beside the prefill kernel")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a "
                         "known-size kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import parallax_local_linear_amd as plx
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wp, wd = wl.WORKLOADS[2], wl.WORKLOADS[3]
    log("generating inputs")
    pin = wl.make_workload(2, device=dev)
    din = wl.make_workload(3, device=dev)
    sums = {wp.name: checksums(pin), wd.name: checksums(din)}
    B, H, L, d = wp.B, wp.H, wp.L, wp.d
    vt = torch.empty(plx.prefill_workspace_bytes(B, H, L, d), dtype=torch.uint8, device=dev)
    pout = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
    C = plx.decode_default_split(wd.B, wd.H, wd.Lmax, wd.d)
    S = -(-wd.Lmax // C)
    part = torch.empty((wd.B, wd.H, S, 2 * wd.d + 4), dtype=torch.float32, device=dev)
    dout = torch.empty((wd.B, wd.H, wd.d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    tm = Timer(torch)

    def step():
        tm.run("stage_v", lambda: plx.prefill_stage_v(pin["v"], vt))
        tm.run("attend", lambda: plx.prefill_attend(pin["q"], pin["k"], vt, pin["rho"],
                                                    pin["gate"], out=pout))
        tm.run("partials", lambda: plx.decode_partials(din["q"], din["kcache"], din["vcache"],
                                                       din["rho"], din["seqlens"], C,
                                                       partials=part))
        tm.run("combine", lambda: plx.decode_combine(part, din["gate"], din["seqlens"],
                                                     wd.Lmax, C, out=dout))

    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tm.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    st = {k: tm.stats(k) for k in ("stage_v", "attend", "partials", "combine")}
    ms = {k: v["median"] for k, v in st.items()}
    pre_steps = [a + b for a, b in zip(tm.times("stage_v"), tm.times("attend"))]
    dec_steps = [a + b for a, b in zip(tm.times("partials"), tm.times("combine"))]
    ms_step = wall * 1e3 / args.steps
    flops = wl.prefill_flops(B, H, L, d)
    pre_ms = _median(pre_steps)
    value = flops / (pre_ms * 1e-3) / 1e12
    dbytes = wl.decode_bytes(din["seqlens"].tolist(), wd.H, wd.d)
    dec_ms = _median(dec_steps)
    rl_att = roofline("prefill_bf16_kernel", "prefill_bf16_kernel<128>", wp.name, "mfma", flops,
                      ms["attend"])
    rl_dec = roofline("decode_split_kernel", "decode_split_kernel<bf16,128>", wd.name, "hbm",
                      dbytes, ms["partials"])
    # staging moves V once in and its fp16 copy once out; the combine reads the
    # split records and writes the output
    vt_bytes = 2 * B * H * L * d * 2
    comb_bytes = wd.B * wd.H * S * (2 * wd.d + 4) * 4 + wd.B * wd.H * wd.d * 4
    rooflines = [
        rl_att,
        roofline("stage_v_kernel", "stage_v_kernel<128>", wp.name, "hbm", vt_bytes,
                 ms["stage_v"]),
        rl_dec,
        roofline("decode_combine_kernel", "decode_combine_kernel<128>", wd.name, "hbm",
                 comb_bytes, ms["combine"]),
    ]

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wp.name, "B": B, "H": H, "L": L, "d": d, "causal": True,
                   "step": "prefill(B4 H16 L4096 d128) + decode(B64 H16 Lkv8192 d128)"},
        "prefill": {"ms": round(pre_ms, 4), "tflops": round(value, 2),
                    "frac_of_peak": round(value / PEAK_MFMA_BF16_TFLOPS, 4),
                    "step_ms": stats(pre_steps),
                    "kernels_ms": {"stage_v": st["stage_v"], "attend": st["attend"]},
                    "flops": flops},
        "roofline": {k: v for k, v in rl_att.items() if k != "workload"},
        "decode": {"workload": wd.name, "ms": round(dec_ms, 4),
                   "value": round(dbytes / (dec_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                   "frac_of_peak": round(dbytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "split_keys": C, "bytes": dbytes, "step_ms": stats(dec_steps),
                   "kernels_ms": {"partials": st["partials"], "combine": st["combine"]},
                   "roofline": {k: v for k, v in rl_dec.items() if k != "workload"}},
        "rooflines": rooflines,
        "checksums": sums,
    }

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = {"read": n * 4, "write": n * 4}
        del src, dst

    if not args.no_gemm_ref:
        log("vendor GEMM reference")
        res["mfma_reference"] = mfma_reference(torch, plx, wl, pin, wp, vt, pout)
    if not args.no_chunk:
        res["chunk"] = [chunk_block(torch, plx, wl, name, dev) for name in sorted(wl.CHUNK_WORKLOADS)]
    if not args.no_backward:
        log("backward: workload 2")
        res["backward"] = [backward_block(torch, plx, wl, pin, wp)]
    rel = []
    if not args.no_softmax:
        log("softmax-relative timing: workloads 2 and 3")
        rel.append(softmax_relative_prefill(torch, plx, wl, pin, wp, vt, pout))
        rel.append(softmax_relative_decode(torch, plx, wl, din, wd))
    cpu = None
    if not args.no_cpu:
        log("cpu baseline")
        cpu = cpu_baseline_prefill(pin, wp)
        res["decode"]["cpu_baseline"] = cpu_baseline_decode(din, wd)
    del pin, din, vt, pout, part, dout
    torch.cuda.empty_cache()
    if not args.no_extra:
        res["extra"], rel_extra, bwd_extra, rl_extra, sums_extra = extra_workloads(
            torch, plx, wl, dev, softmax=not args.no_softmax, backward=not args.no_backward)
        if bwd_extra:
            res.setdefault("backward", []).append(bwd_extra)
        rel += rel_extra
        res["rooflines"] += rl_extra
        res["checksums"].update(sums_extra)
    if rel:
        res["softmax_relative"] = rel
    if not args.no_sweep and not args.no_softmax:
        res["softmax_sweep"] = softmax_sweep(torch, plx, wl, dev)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def chunk_block(torch, plx, wl, name, dev, steps=10):
    """Chunked prefill (V^T staging of the rows read + fused kernel) on one
    chunk workload, workspace allocated before timing."""
    log(f"chunk: {name}")
    cw = wl.CHUNK_WORKLOADS[name]
    inp = wl.make_chunk_workload(name, device=dev)
    B, H, d = cw["B"], cw["H"], cw["d"]
    Lmax = inp["kcache"].shape[2]
    T, mq = inp["T"], inp["max_q"]
    ws = torch.empty(int(plx.lib().parallax_prefill_chunk_workspace_bytes(B, H, T, Lmax, mq, d, 0)),
                     dtype=torch.uint8, device=dev)
    rn = int(plx.lib().parallax_prefill_chunk_vt_workspace_bytes(B, H, T, Lmax, mq, d, 0))
    rws = torch.empty(rn, dtype=torch.uint8, device=dev) if rn else None
    out = torch.empty((inp["T"], H, d), dtype=torch.float32, device=dev)
    tm = Timer(torch)
    for _ in range(steps + 2):
        tm.run("chunk", lambda: plx.prefill_chunk(inp["q"], inp["kcache"], inp["vcache"],
                                                  inp["rho"], inp["gate"], inp["cu_q"],
                                                  inp["ctx"], inp["max_q"], out=out,
                                                  workspace=ws))
    torch.cuda.synchronize()
    ms = tm.ms("chunk", 2)
    # serving loop with a staged V cache kept by the caller: per step, re-stage
    # the tiles of the appended rows and run the chunk on the staged cache
    vt = plx.prefill_stage_v(inp["vcache"])
    for _ in range(steps + 2):
        tm.run("staged", lambda: (plx.stage_v_rows(inp["vcache"], vt, inp["cu_q"], inp["ctx"],
                                                   inp["max_q"], inp["T"]),
                                  plx.prefill_chunk(inp["q"], inp["kcache"], None, inp["rho"],
                                                    inp["gate"], inp["cu_q"], inp["ctx"],
                                                    inp["max_q"], out=out, vt_cache=vt,
                                                    workspace=rws)))
    torch.cuda.synchronize()
    ms_st = tm.ms("staged", 2)
    ctx, n = [cw["ctx"]] * B, [cw["n"]] * B
    fl = wl.chunk_flops(ctx, n, H, d)
    nb = wl.chunk_bytes(ctx, n, H, d)
    split = plx.chunk_default_split(B, H, Lmax, mq, d)
    res = {"workload": name, "split_keys": split if split < Lmax else None,
           "ms": round(ms, 4), "ms_stats": tm.stats("chunk", 2),
           "TFLOP/s": round(fl / ms / 1e9, 2), "GB/s": round(nb / ms / 1e6, 1),
           "staged_cache": {"ms": round(ms_st, 4), "TFLOP/s": round(fl / ms_st / 1e9, 2),
                            "GB/s": round(nb / ms_st / 1e6, 1)},
           "flops": fl, "bytes": nb}
    del inp, ws, out, vt, rws
    torch.cuda.empty_cache()
    return res


def backward_block(torch, plx, wl, inp, w, steps=10):
    """Training forward pass and backward pass on one prefill workload, with a
    seeded N(0,1) dout; all buffers allocated before timing."""
    B, H, L, d = w.B, w.H, w.L, w.d
    dev = inp["q"].device
    g = torch.Generator(device=dev).manual_seed(1234)
    dout = torch.randn((B, H, L, d), generator=g, device=dev, dtype=torch.float32)
    fws = torch.empty(plx.prefill_workspace_bytes(B, H, L, d), dtype=torch.uint8, device=dev)
    bws = torch.empty(plx.prefill_backward_workspace_bytes(B, H, L, d), dtype=torch.uint8,
                      device=dev)
    grads = tuple(torch.empty((B, H, L, d), dtype=torch.float32, device=dev) for _ in range(4)) \
        + (torch.empty(H, dtype=torch.float32, device=dev),)
    saved = {}

    def fwd():
        saved["t"] = plx.prefill_train(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"],
                                       workspace=fws)

    def bwd():
        out, lse, rbar, corr = saved["t"]
        plx.prefill_backward(inp["q"], inp["k"], inp["v"], inp["rho"], inp["gate"], out, corr,
                             lse, rbar, dout, grads=grads, workspace=bws)

    tm = Timer(torch)
    for _ in range(steps + 2):
        tm.run("fwd", fwd)
        tm.run("bwd", bwd)
    torch.cuda.synchronize()
    f_ms, b_ms = tm.ms("fwd", 2), tm.ms("bwd", 2)
    fl = wl.prefill_flops(B, H, L, d)
    return {"workload": w.name, "train_forward_ms": round(f_ms, 4),
            "backward_ms": round(b_ms, 4), "backward_ms_stats": tm.stats("bwd", 2),
            "step_ms": round(f_ms + b_ms, 4),
            "train_forward_TFLOP/s": round(fl / f_ms / 1e9, 2),
            "backward_TFLOP/s": round(2 * fl / b_ms / 1e9, 2),
            "backward_frac_of_mfma_peak": round(2 * fl / b_ms / 1e9 / PEAK_MFMA_BF16_TFLOPS, 4),
            "flops": {"forward": fl, "backward": 2 * fl}}


def mfma_reference(torch, plx, wl, inp, w, vt, pout, steps=20, n=8192):
    """What the device's bf16 matrix cores deliver to the vendor GEMM (torch.matmul
    on two resident n x n bf16 matrices, which runs hipBLASLt) on this machine, beside
    the fused prefill kernel: each back to back on its own, then alternating
    launch by launch.  The chip is power-limited under MFMA load, so this
    measures how much of the published 2.5 PF any bf16 MFMA work reaches here;
    it is context for `roofline.frac`, not a replacement for its peak.  (The
    GEMM's 384 MB of operands also evict the prefill's inputs from the last-level
    cache, which the alternating figures include.)"""
    dev = inp["q"].device
    g = torch.Generator(device=dev).manual_seed(4321)
    a = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)

    def gemm():
        torch.matmul(a, b, out=c)

    def attend():
        plx.prefill_attend(inp["q"], inp["k"], vt, inp["rho"], inp["gate"], out=pout)

    tm = Timer(torch)
    for _ in range(steps + 2):
        tm.run("gemm_alone", gemm)
    for _ in range(steps + 2):
        tm.run("attend_alone", attend)
    for _ in range(steps + 2):
        tm.run("gemm_alt", gemm)
        tm.run("attend_alt", attend)
    torch.cuda.synchronize()
    gfl = 2.0 * n ** 3
    afl = wl.prefill_flops(w.B, w.H, w.L, w.d)
    out = {"gemm": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), fp32 accumulate, bf16 out",
           "attend_workload": w.name}
    for mode in ("alone", "alt"):
        g_ms, a_ms = tm.ms("gemm_" + mode, 2), tm.ms("attend_" + mode, 2)
        out[mode] = {"gemm_ms": round(g_ms, 4), "gemm_TFLOP/s": round(gfl / g_ms / 1e9, 1),
                     "gemm_frac_of_peak": round(gfl / g_ms / 1e9 / PEAK_MFMA_BF16_TFLOPS, 4),
                     "attend_ms": round(a_ms, 4), "attend_TFLOP/s": round(afl / a_ms / 1e9, 1),
                     "attend_over_gemm": round(afl / a_ms / (gfl / g_ms), 4)}
    del a, b, c
    return out


def softmax_relative_prefill(torch, plx, wl, inp, w, vt, pout, steps=10):
    """Parallax prefill against the same kernels with the correction compiled out,
    on one workload.  The V staging pass is the same for both and is timed once
    per step; the attend kernels alternate launch by launch."""
    tm = Timer(torch)
    for _ in range(steps + 2):
        tm.run("stage_v", lambda: plx.prefill_stage_v(inp["v"], vt))
        tm.run("parallax", lambda: plx.prefill_attend(inp["q"], inp["k"], vt, inp["rho"],
                                                      inp["gate"], out=pout))
        tm.run("softmax", lambda: plx.softmax_prefill_attend(inp["q"], inp["k"], vt, out=pout))
    torch.cuda.synchronize()
    st, pa, sm = tm.ms("stage_v", 2), tm.ms("parallax", 2), tm.ms("softmax", 2)
    fl = wl.prefill_flops(w.B, w.H, w.L, w.d)
    return {"workload": w.name, "kind": "prefill",
            "parallax_attend_ms": round(pa, 4), "softmax_attend_ms": round(sm, 4),
            "attend_time_ratio": round(pa / sm, 4),
            "stage_v_ms": round(st, 4), "path_time_ratio": round((st + pa) / (st + sm), 4),
            "parallax_attend_TFLOP/s": round(fl / pa / 1e9, 2),
            "softmax_attend_TFLOP/s": round(fl / 2 / sm / 1e9, 2),
            "flops": {"parallax": fl, "softmax": fl / 2}}


def softmax_relative_decode(torch, plx, wl, inp, w, steps=10, ahead=0):
    """Parallax decode step against the softmax-only decode step (split pass and
    combine each, same split size and workspace), alternating launch by launch
    (`ahead`: see Timer)."""
    B, H, Lmax, d = inp["kcache"].shape
    C = plx.decode_default_split(B, H, Lmax, d)
    ws = torch.empty(plx.decode_workspace_bytes(B, H, Lmax, d, C), dtype=torch.uint8,
                     device=inp["q"].device)
    out = torch.empty((B, H, d), dtype=torch.float32, device=inp["q"].device)
    tm = Timer(torch, ahead)
    for _ in range(steps + 2):
        tm.run("parallax", lambda: plx.decode(inp["q"], inp["kcache"], inp["vcache"], inp["rho"],
                                              inp["gate"], inp["seqlens"], split_keys=C,
                                              out=out, workspace=ws))
        tm.run("softmax", lambda: plx.softmax_decode(inp["q"], inp["kcache"], inp["vcache"],
                                                     inp["seqlens"], split_keys=C, out=out,
                                                     workspace=ws))
    torch.cuda.synchronize()
    pa, sm = tm.ms("parallax", 2), tm.ms("softmax", 2)
    nb = wl.decode_bytes(inp["seqlens"].tolist(), H, d)
    nb_sm = nb - B * H * d * 2 - 4 * H          # no rho, no gate
    return {"workload": w.name if w is not None else f"decode_bf16_B{B}_H{H}_L{Lmax}_d{d}",
            "kind": "decode", "split_keys": C,
            "parallax_ms": round(pa, 4), "softmax_ms": round(sm, 4),
            "time_ratio": round(pa / sm, 4),
            "parallax_GB/s": round(nb / pa / 1e6, 1), "softmax_GB/s": round(nb_sm / sm / 1e6, 1),
            "bytes": {"parallax": nb, "softmax": nb_sm}}


def softmax_sweep(torch, plx, wl, dev, steps=3):
    """The pages' comparison with softmax attention across batch sizes and
    context lengths: the Parallax kernels and their softmax-only twins on a grid
    of shapes, alternating launch by launch (median of `steps` launches each
    after one warm-up), each call queued behind a 200k-cycle spin kernel so that
    the events bracket GPU time (the smallest calls take 20 us).  Prefill: H 16, L 1k-64k with B = max(1, 16k / L), at
    d 64 and 128 (attend kernels; V staged once).  Decode: H 16, d 128,
    B 1 / 8 / 64 x L 8k / 32k / 128k (split pass + combine)."""
    pts = []
    for d in (64, 128):
        for L in (1024, 4096, 16384, 65536):
            B = max(1, 16384 // L)
            log(f"sweep: prefill B{B} H16 L{L} d{d}")
            inp = wl.prefill_inputs(B, 16, L, d, "bf16", seed=3000 + L + d, device=dev,
                                    rho_std=0.1, gate=("uniform", 0.2, 1.0))
            vt = plx.prefill_stage_v(inp["v"])
            out = torch.empty((B, 16, L, d), dtype=torch.float32, device=dev)
            tm = Timer(torch, SWEEP_AHEAD)
            for _ in range(steps + 1):
                tm.run("parallax", lambda: plx.prefill_attend(inp["q"], inp["k"], vt, inp["rho"],
                                                              inp["gate"], out=out))
                tm.run("softmax", lambda: plx.softmax_prefill_attend(inp["q"], inp["k"], vt,
                                                                     out=out))
            torch.cuda.synchronize()
            pa, sm = tm.ms("parallax", 1), tm.ms("softmax", 1)
            fl = wl.prefill_flops(B, 16, L, d)
            pts.append({"kind": "prefill", "B": B, "H": 16, "L": L, "d": d,
                        "parallax_ms": round(pa, 4), "softmax_ms": round(sm, 4),
                        "time_ratio": round(pa / sm, 4),
                        "parallax_TFLOP/s": round(fl / pa / 1e9, 1),
                        "softmax_TFLOP/s": round(fl / 2 / sm / 1e9, 1)})
            del inp, vt, out
            torch.cuda.empty_cache()
    for L in (8192, 32768, 131072):
        for B in (1, 8, 64):
            log(f"sweep: decode B{B} H16 L{L} d128")
            inp = wl.decode_inputs(B, 16, L, 128, "bf16", seed=3100 + B, device=dev,
                                   rho_std=0.1)
            r = softmax_relative_decode(torch, plx, wl, inp, None, steps=steps,
                                        ahead=SWEEP_AHEAD)
            pts.append({"kind": "decode", "B": B, "H": 16, "L": L, "d": 128,
                        "split_keys": r["split_keys"],
                        "parallax_ms": r["parallax_ms"], "softmax_ms": r["softmax_ms"],
                        "time_ratio": r["time_ratio"], "parallax_GB/s": r["parallax_GB/s"],
                        "softmax_GB/s": r["softmax_GB/s"]})
            del inp
            torch.cuda.empty_cache()
    return pts


def extra_workloads(torch, plx, wl, dev, steps=10, softmax=True, backward=True):
    """Long ragged decode (B8 H16, 65536..131072 keys) and the d=64 prefill."""
    out, rel, bwd, rls, sums = [], [], None, [], {}
    w4 = wl.WORKLOADS[4]
    log("extra: decode workload 4")
    din = wl.make_workload(4, device=dev)
    sums[w4.name] = checksums(din)
    C = plx.decode_default_split(w4.B, w4.H, w4.Lmax, w4.d)
    S = -(-w4.Lmax // C)
    part = torch.empty((w4.B, w4.H, S, 2 * w4.d + 4), dtype=torch.float32, device=dev)
    dout = torch.empty((w4.B, w4.H, w4.d), dtype=torch.float32, device=dev)
    tm = Timer(torch)
    for i in range(steps + 2):
        tm.run("partials", lambda: plx.decode_partials(din["q"], din["kcache"], din["vcache"],
                                                       din["rho"], din["seqlens"], C,
                                                       partials=part))
        tm.run("combine", lambda: plx.decode_combine(part, din["gate"], din["seqlens"],
                                                     w4.Lmax, C, out=dout))
    torch.cuda.synchronize()
    nb = wl.decode_bytes(din["seqlens"].tolist(), w4.H, w4.d)
    ms = _median([a + b for a, b in zip(tm.times("partials", 2), tm.times("combine", 2))])
    n_rec = sum(-(-min(int(x), w4.Lmax) // C) for x in din["seqlens"].tolist()) * w4.H
    out.append({"workload": w4.name, "ms": round(ms, 4), "GB/s": round(nb / ms / 1e6, 1),
                "frac_of_hbm_peak": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4), "bytes": nb,
                "seqlens": din["seqlens"].tolist(), "split_keys": C,
                "kernels_ms": {"partials": tm.stats("partials", 2),
                               "combine": tm.stats("combine", 2)}})
    rls.append(roofline("decode_split_kernel", "decode_split_kernel<bf16,128>", w4.name, "hbm",
                        nb, tm.ms("partials", 2)))
    rls.append(roofline("decode_combine_kernel", "decode_combine_kernel<128>", w4.name, "hbm",
                        n_rec * (2 * w4.d + 4) * 4 + w4.B * w4.H * w4.d * 4,
                        tm.ms("combine", 2)))
    del part, dout
    if softmax:
        log("softmax-relative timing: workload 4")
        rel.append(softmax_relative_decode(torch, plx, wl, din, w4))
    del din
    torch.cuda.empty_cache()

    w5 = wl.WORKLOADS[5]
    log("extra: prefill workload 5")
    pin = wl.make_workload(5, device=dev)
    sums[w5.name] = checksums(pin)
    vt = torch.empty(plx.prefill_workspace_bytes(w5.B, w5.H, w5.L, w5.d), dtype=torch.uint8,
                     device=dev)
    pout = torch.empty((w5.B, w5.H, w5.L, w5.d), dtype=torch.float32, device=dev)
    tm = Timer(torch)
    for i in range(steps + 2):
        tm.run("stage_v", lambda: plx.prefill_stage_v(pin["v"], vt))
        tm.run("attend", lambda: plx.prefill_attend(pin["q"], pin["k"], vt, pin["rho"],
                                                    pin["gate"], out=pout))
    torch.cuda.synchronize()
    fl = wl.prefill_flops(w5.B, w5.H, w5.L, w5.d)
    ms_a = tm.ms("attend", 2)
    ms = _median([a + b for a, b in zip(tm.times("stage_v", 2), tm.times("attend", 2))])
    out.append({"workload": w5.name, "ms": round(ms, 4),
                "TFLOP/s": round(fl / ms / 1e9, 2),
                "frac_of_mfma_peak": round(fl / ms / 1e9 / PEAK_MFMA_BF16_TFLOPS, 4),
                "attend_ms": round(ms_a, 4), "attend_TFLOP/s": round(fl / ms_a / 1e9, 2),
                "kernels_ms": {"stage_v": tm.stats("stage_v", 2),
                               "attend": tm.stats("attend", 2)},
                "flops": fl})
    rls.append(roofline("prefill_bf16_kernel", "prefill_bf16_kernel<64>", w5.name, "mfma", fl,
                        ms_a))
    rls.append(roofline("stage_v_kernel", "stage_v_kernel<64>", w5.name, "hbm",
                        2 * w5.B * w5.H * w5.L * w5.d * 2, tm.ms("stage_v", 2)))
    if softmax:
        log("softmax-relative timing: workload 5")
        rel.append(softmax_relative_prefill(torch, plx, wl, pin, w5, vt, pout))
    del vt, pout
    if backward:
        log("backward: workload 5")
        bwd = backward_block(torch, plx, wl, pin, w5)
    del pin
    torch.cuda.empty_cache()
    return out, rel, bwd, rls, sums


if __name__ == "__main__":
    main()
