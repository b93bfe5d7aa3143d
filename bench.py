#!/usr/bin/env python3
"""Forward+backward throughput of the gated delta rule on one MI355X.

Workload: the Qwen3.5-9B linear_attn shape of mlx-lm PR #1217 (Performance
table): B=1, Hk=16, Hv=64, Dk=192, Dv=128, T=2048, bf16 q/k/v/g/beta/dy,
fp32 state, weak decay, normalised q/k, S0=0 (synthetic, seeded).  A step is
one gdr_forward (with save) plus one gdr_backward over that batch; inputs and
every output/scratch buffer are resident in HBM before timing starts.

Prints one JSON line (see README of the bench contract in the design doc).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_PEAK_TF = 157.3           # MI355X FP32: dense MFMA and (packed) vector, TFLOP/s
FLOPS_FWD = 7                  # per state element per step (S k, S q, decay+rank-1)
FLOPS_BWD = 15                 # per state element per step (reverse sweep)

# HBM bytes per gdr_backward call at the default workload (the sum over its
# three kernels), from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs scaled
# by a plain-copy calibration (profiles/hbm_bytes_qwen35-9b_T2048_bf16.md).
# They describe the kernels built from sources with this digest and are not
# reported otherwise.
BWD_TRAFFIC = {"sources_sha256_16": "432195f4dce64c7d",
               "read_bytes": 969.8e6, "write_bytes": 518.8e6}
BWD_SOURCES = ("gdr_api.hip", "gdr_device.h", "gdr_internal.h", "gdr_chunked_sweep.hip",
               "gdr_chunk.hip")


def sources_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_recurrence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--T", type=int, default=2048)
    ap.add_argument("--B", type=int, default=1)
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--dtype", default="bf16", choices=("bf16", "f32"))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-T", type=int, default=2048)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read + write), "
                         "the reference for scaling HBM byte counters, and exit")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="instead of the training step, time fwd+bwd at the long-context "
                         "shape (B=4, T=8192, Qwen3.5-9B heads, trainable S0) for the "
                         "chunk sizes 8..64 the library takes, one JSON line each, and exit")
    ap.add_argument("--decode", type=int, default=0, metavar="B",
                    help="instead of the training step, time single-step inference "
                         "(T=1, state updated in place, no save buffer) at batch B "
                         "with the same heads, and exit")
    return ap.parse_args()


def decode(args):
    """Inference decode: T=1 steps with the state in and out of one buffer.
    The steps are captured in a HIP graph (torch.cuda.CUDAGraph) so that the
    figure is GPU time, not Python launch overhead; one step streams the
    fp32 state once (read + write)."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib, inputs, ops
    dev = torch.device("cuda:0")
    _lib.load()
    B, nsteps = args.decode, 16
    p = inputs.draw(B, nsteps, 16, 64, 192, 128, seed=args.seed, normalised=True,
                    S0_std=0.05, dtype=args.dtype)
    dt = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    steps = [{n: t(getattr(p, n)[:, i:i + 1]) for n in ("q", "k", "v", "g", "beta")}
             for i in range(nsteps)]
    S = torch.from_numpy(p.S0.astype(np.float32)).to(dev)
    ys = [torch.empty((B, 1, 64, 128), dtype=dt, device=dev) for _ in range(nsteps)]

    def run():
        for i, st in enumerate(steps):
            ops.gdr_forward(st["q"], st["k"], st["v"], st["g"], st["beta"], S, save=False,
                            y=ys[i], S_T=S)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()  # warm-up outside the graph
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(args.steps, 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * nsteps)
    esz = 2 if args.dtype == "bf16" else 4
    nbytes = 2 * B * 64 * 128 * 192 * 4 + B * (2 * 16 * 192 + 2 * 64 * 128 + 2 * 64) * esz
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({"metric": "decode tokens/s (T=1 step, state in place), Qwen3.5-9B heads",
                      "value": B / (us * 1e-6), "unit": "tokens/s", "batch": B,
                      "us_per_step": us, "dtype": args.dtype, "data": "synthetic",
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                   "algorithmic_bytes_per_step": nbytes}}), flush=True)


def chunk_sweep(args):
    """Long-context training step (B=4, T=8192, Hk=16, Hv=64, Dk=192, Dv=128,
    S0 ~ N(0, 0.05), decay alternating weak/strong over value heads) for each
    chunk size C: median fwd and bwd times by HIP events, save-buffer and
    workspace sizes, algorithmic HBM bytes.  Inputs drawn on the device
    (inputs.draw_device: the draw() distributions)."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib, inputs, ops
    dev = torch.device("cuda:0")
    _lib.load()
    B, T, Hk, Hv, Dk, Dv = 4, 8192, 16, 64, 192, 128
    d = inputs.draw_device(B, T, Hk, Hv, Dk, Dv, device=dev, seed=args.seed, decay="mix",
                           S0_std=0.05, dtype=args.dtype)
    q, k, v, g, beta, dy, S0 = (d[n] for n in ("q", "k", "v", "g", "beta", "dy", "S0"))
    esz = 2 if args.dtype == "bf16" else 4
    for C in (8, 16, 32, 64):  # the library's range: a chunk is one 64-step tile
        shape = ops.shape_of(q, v, C, q.dtype)
        ckpt = torch.empty(_lib.checkpoint_bytes(shape), dtype=torch.uint8, device=dev)
        ws = torch.empty(_lib.backward_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        fws = torch.empty(max(_lib.forward_workspace_bytes(shape), 1), dtype=torch.uint8,
                          device=dev)
        y = torch.empty_like(v)
        S_T = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                torch.empty_like(g), torch.empty_like(beta), torch.empty_like(S_T))
        saved = ops.Saved(ckpt, C)

        def fwd():
            ops.gdr_forward(q, k, v, g, beta, S0, chunk=C, y=y, S_T=S_T, ckpt=ckpt,
                            workspace=fws)

        def bwd():
            ops.gdr_backward(q, k, g, beta, saved, dy, None, workspace=ws, out=outs)

        for _ in range(3):
            fwd()
            bwd()
        torch.cuda.synchronize()
        n = 10
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fwd()
            ev[i][1].record()
            bwd()
            ev[i][2].record()
        torch.cuda.synchronize()
        f = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        b = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
        nch = -(-T // C)
        tok_in = B * T * (2 * Hk * Dk + Hv * Dv + 2 * Hv) * esz
        rows32 = B * T * Hv * Dv * 4
        state = B * Hv * Dv * Dk * 4
        nbytes = (2 * tok_in + B * T * Hv * Dv * esz + 2 * rows32 + (2 * nch + 3) * state
                  + tok_in)
        print(json.dumps({"chunk_sweep": {
            "C": C, "B": B, "T": T, "dtype": args.dtype,
            "path": "chunked" if _lib.forward_workspace_bytes(shape) > 0 else "sweep",
            "fwd_ms_median": f, "bwd_ms_median": b, "tokens_per_s": B * T / ((f + b) * 1e-3),
            "checkpoint_MB": ckpt.numel() / 1e6, "workspace_fwd_MB": fws.numel() / 1e6,
            "workspace_bwd_MB": ws.numel() / 1e6,
            "algorithmic_bytes": nbytes,
            "hbm_frac_algorithmic": nbytes / ((f + b) * 1e-3) / 1e9 / HBM_PEAK_GBS}}),
            flush=True)
        del ckpt, ws, fws, y, S_T, outs, saved
        torch.cuda.empty_cache()


def copy_calibration(mib):
    """One warm-up and one measured dispatch of a plain contiguous fp32 copy
    (mib MiB read, mib MiB written): the HBM byte counters of the second
    dispatch, divided into its known size, give the counter scale factor."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4,
                                           "dispatches": 2}}), flush=True)


def cpu_baseline(T, seed, dtype, budget_s=25.0):
    """Time the float64 oracle (as it stands, one BLAS thread) on the same
    workload, one (batch row, kv group) at a time: forward + backward of the
    group's value heads over the full T.  Groups run until all are done or
    the time budget is spent; tokens are scaled by the share of groups run."""
    from threadpoolctl import threadpool_limits
    import oracle.gdr_oracle as O
    from gated_delta_rule_recurrence_amd import inputs
    p = inputs.qwen35_9b(T, seed=seed, dtype=dtype)
    rep = p.Hv // p.Hk
    groups = [(b, hk) for b in range(p.B) for hk in range(p.Hk)]
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for b, hk in groups:
            bs, ks, vs = slice(b, b + 1), slice(hk, hk + 1), slice(hk * rep, (hk + 1) * rep)
            O.forward(p.q[bs, :, ks], p.k[bs, :, ks], p.v[bs, :, vs], p.g[bs, :, vs],
                      p.beta[bs, :, vs])
            O.backward(p.q[bs, :, ks], p.k[bs, :, ks], p.v[bs, :, vs], p.g[bs, :, vs],
                       p.beta[bs, :, vs], p.dy[bs, :, vs])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    frac = done / len(groups)
    return {"value": p.B * T * frac / dt, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch row, kv group) units of the same "
                      f"workload (B={p.B}, T={T}, {rep} value heads each), forward + "
                      f"backward in {dt:.1f} s on 1 thread; tokens scaled by "
                      f"{done}/{len(groups)}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path "
              "shards by (batch row, kv head) with no communication, see DESIGN.md",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.decode:
        decode(args)
        return
    if args.chunk_sweep:
        chunk_sweep(args)
        return
    import torch
    from gated_delta_rule_recurrence_amd import _lib, inputs, ops

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    _lib.load()  # fail loudly if the HIP library is missing

    p = inputs.qwen35_9b(args.T, seed=args.seed, dtype=args.dtype, B=args.B)
    dt = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    q, k, v, g, beta, dy = (t(getattr(p, n)) for n in ("q", "k", "v", "g", "beta", "dy"))
    B, T, Hk, Hv, Dk, Dv = p.B, p.T, p.Hk, p.Hv, p.Dk, p.Dv

    # every buffer allocated up front
    shape = ops.shape_of(q, v, args.chunk, dt)
    ckpt = torch.empty(_lib.checkpoint_bytes(shape), dtype=torch.uint8, device=dev)
    ws = torch.empty(_lib.backward_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(_lib.forward_workspace_bytes(shape), 1), dtype=torch.uint8,
                      device=dev)
    y = torch.empty_like(v)
    S_T = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
            torch.empty_like(g), torch.empty_like(beta),
            torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev))
    saved = ops.Saved(ckpt, args.chunk)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        ops.gdr_forward(q, k, v, g, beta, None, chunk=args.chunk, y=y, S_T=S_T,
                        ckpt=ckpt, workspace=fws)

    def bwd():
        ops.gdr_backward(q, k, g, beta, saved, dy, None, workspace=ws, out=outs)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # timed region: K whole steps, events on the library's stream around each call
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in ev])

    # the same steps with the caches flushed before each (a 512 MiB write,
    # outside the timed events, evicts L2 and the 256 MB Infinity Cache)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    nflush = min(args.steps, 20)
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nflush)]
    for i in range(nflush):
        flush.zero_()
        evf[i][0].record(stream)
        fwd()
        bwd()
        evf[i][1].record(stream)
    torch.cuda.synchronize()
    flushed_ms = np.array([e[0].elapsed_time(e[1]) for e in evf])
    del flush
    peak_mb = torch.cuda.max_memory_allocated(dev) / 1e6
    ms = wall * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms / 1e3)

    elems = B * T * Hv * Dv * Dk  # state-element steps
    fwd_flops, bwd_flops = FLOPS_FWD * elems, FLOPS_BWD * elems
    fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12
    # the bf16-product sweep kernels take bf16 inputs with Dk % 8 == 0 and Dv % 4 == 0
    sfx = "_bf16" if (args.dtype == "bf16" and Dk % 8 == 0 and Dv % 4 == 0) else ""
    all_tf = (FLOPS_FWD + FLOPS_BWD) * elems / (ms * 1e-3) / 1e12
    # algorithmic HBM bytes, each tensor touched once: the forward reads q, k,
    # v, g, beta and writes y, the residual rows e (fp32), the chunk
    # checkpoints and S_T; the backward reads q, k, g, beta, dy, e and the
    # checkpoints and writes dq, dk, dv, dg, dbeta and dS0
    esz = 2 if args.dtype == "bf16" else 4
    nch = -(-T // args.chunk)
    tok_in = B * T * (2 * Hk * Dk + Hv * Dv + 2 * Hv) * esz   # q, k, (v | dy), g, beta
    rows32 = B * T * Hv * Dv * 4
    state = B * Hv * Dv * Dk * 4
    fwd_bytes = tok_in + B * T * Hv * Dv * esz + rows32 + (nch + 1) * state
    bwd_bytes = tok_in + rows32 + nch * state + tok_in + state
    traffic = None
    default_workload = (args.T, args.B, args.chunk, args.dtype) == (2048, 1, 64, "bf16")
    if default_workload and sources_digest(BWD_SOURCES) == BWD_TRAFFIC["sources_sha256_16"]:
        traffic = BWD_TRAFFIC["read_bytes"] + BWD_TRAFFIC["write_bytes"]

    ckpt_mb = ckpt.numel() / 1e6
    ws_mb = ws.numel() / 1e6
    rec = {
        "metric": "fwd+bwd tokens/s, Qwen3.5-9B gated-delta shape T=2048",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"Qwen3.5-9B linear_attn gated delta rule fwd+bwd, "
                               f"B={B} T={T} Hk={Hk} Hv={Hv} Dk={Dk} Dv={Dv}, "
                               f"{args.dtype} inputs, fp32 state, chunk={args.chunk}",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        # the dominant call: gdr_backward (about 0.55 of 0.78 ms), timed with
        # HIP events on the library's stream; its products deliver fp32
        # accuracy (fp32 MFMA, or bf16 MFMA on three-piece splits), so the
        # fp32 peak is the bar
        "roofline": {"bound": "mfma", "kernel": f"gdr_backward (prep_kernel<bwd>, "
                     f"bwd_chunked{sfx}_kernel, chunk_kernel)",
                     "achieved": bwd_tf, "peak": FP32_PEAK_TF,
                     "unit": "TFLOP/s", "frac": bwd_tf / FP32_PEAK_TF,
                     "traffic": traffic,
                     "flops_per_launch": bwd_flops,
                     "algorithmic_bytes_per_launch": bwd_bytes,
                     "hbm_frac_algorithmic": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "avg_launch_ms": bwd_ms},
        "forward": {"kernel": f"gdr_forward (prep_kernel<fwd>, fwd_chunked{sfx}_kernel)",
                    "achieved_tflops": fwd_tf, "frac": fwd_tf / FP32_PEAK_TF,
                    "flops_per_launch": fwd_flops, "algorithmic_bytes_per_launch": fwd_bytes,
                    "hbm_frac_algorithmic": fwd_bytes / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "avg_launch_ms": fwd_ms},
        "timing": {"wall_ms_per_step": ms, "step_ms_median": float(np.median(step_ms)),
                   "step_ms_min": float(step_ms.min()),
                   "flushed_step_ms_median": float(np.median(flushed_ms)),
                   "flushed_step_ms_min": float(flushed_ms.min()), "flushed_steps": nflush},
        "peak_device_memory_MB": peak_mb,
        "breakdown": {"fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                      "useful_tflops_whole_step": all_tf,
                      "frac_whole_step_vs_fp32_peak": all_tf / FP32_PEAK_TF,
                      "checkpoint_MB": ckpt_mb, "workspace_MB": ws_mb},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(min(args.cpu_sample_T, T), args.seed, args.dtype)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
