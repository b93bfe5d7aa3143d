#!/usr/bin/env python3
"""Forward+backward throughput of the gated delta rule on one MI355X.

Workload: the Qwen3.5-9B linear_attn shape of mlx-lm PR #1217 (Performance
table): B=1, Hk=16, Hv=64, Dk=192, Dv=128, T=2048, bf16 q/k/v/g/beta/dy,
fp32 state, weak decay, normalised q/k, S0=0 (synthetic, seeded).  A step is
one gdr_forward (with save) plus one gdr_backward over that batch; inputs and
every output/scratch buffer are resident in HBM before timing starts.

Default: prints one JSON line (the training step).  Other modes print one
JSON line per case and exit:
  --t-sweep       the same heads at T = 256, 512, 1024, 2048 (the Performance
                  table's lengths): fwd/bwd ms, tokens/s, peak device memory;
  --vjp-batch     the focused VJP shape of unsloth-zoo PR #776 (B = 1, 2, 4,
                  8, T=64, Hk=Hv=2, Dk=Dv=64, fp32): backward alone and fwd+bwd;
  --chunk-sweep   the long-context shape (B=4, T=8192) over checkpoint
                  intervals C;
  --decode B      single-step inference at batch B;
  --copy-calibration MIB   a plain device copy (for the HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
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
PREP_RECORD_BYTES = (3 * 64 * 64 + 4 * 64) * 4   # one per (batch row, value head, chunk)

# Counter figures for the default workload, from the rocprofv3 summaries
# under profiles/ (HBM bytes: FETCH_SIZE and WRITE_SIZE scaled by a plain
# copy; pipe utilisation: SQ counters).  They describe the kernels built from
# the sources with this digest and are reported only while the sources still
# hash to it (null otherwise).
PROFILE = {
    "sources_sha256_16": "5fc284b1d2f7f323",
    "source": "profiles/hbm_bytes_qwen35-9b_T2048_bf16.md and "
              "profiles/sq_counters_qwen35-9b_T2048_bf16.md (rocprofv3 --pmc)",
    "bwd_read_bytes": 974.4e6, "bwd_write_bytes": 507.9e6,
    "fwd_read_bytes": 162.3e6, "fwd_write_bytes": 472.9e6,
    # per kernel: SQ-counter pipe utilisation and the trace's average duration
    "kernels": {
        "prep_kernel<fwd>": {"mfma_busy_pct": 5.9, "valu_busy_pct": 25.8, "avg_us": 33.3},
        "fwd_chunked_bf16_kernel": {"mfma_busy_pct": 19.3, "valu_busy_pct": 49.4, "avg_us": 176.7},
        "prep_kernel<bwd>": {"mfma_busy_pct": 6.3, "valu_busy_pct": 26.1, "avg_us": 31.8},
        "bwd_chunked_bf16_kernel": {"mfma_busy_pct": 17.5, "valu_busy_pct": 50.4, "avg_us": 182.5},
        "chunk_bf16_kernel": {"mfma_busy_pct": 22.7, "valu_busy_pct": 37.8, "avg_us": 251.8},
    },
}
BWD_KERNELS = ("prep_kernel<bwd>", "bwd_chunked_bf16_kernel", "chunk_bf16_kernel")
FWD_KERNELS = ("prep_kernel<fwd>", "fwd_chunked_bf16_kernel")


def pipe_busy(names):
    """Time-weighted MFMA and VALU busy percentages over a call's kernels."""
    ks = [PROFILE["kernels"][n] for n in names]
    t = sum(k["avg_us"] for k in ks)
    return {"mfma_busy_pct": sum(k["mfma_busy_pct"] * k["avg_us"] for k in ks) / t,
            "valu_busy_pct": sum(k["valu_busy_pct"] * k["avg_us"] for k in ks) / t}
PROFILED_SOURCES = ("gdr_api.hip", "gdr_device.h", "gdr_internal.h", "gdr_chunked_sweep.hip",
                    "gdr_chunk.hip", "gdr_chunk_bf16.hip")


def sources_digest(files=PROFILED_SOURCES):
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
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (default: the CPU affinity size, at most 16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read + write), "
                         "the reference for scaling HBM byte counters, and exit")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="time fwd+bwd at the long-context shape (B=4, T=8192, "
                         "Qwen3.5-9B heads, trainable S0) for a range of checkpoint "
                         "intervals, one JSON line each, and exit")
    ap.add_argument("--chunks", default="16,32,64,128,256,512",
                    help="checkpoint intervals of --chunk-sweep")
    ap.add_argument("--t-sweep", action="store_true",
                    help="time fwd+bwd at the Qwen3.5-9B heads for T = 256, 512, 1024, "
                         "2048, one JSON line each, and exit")
    ap.add_argument("--vjp-batch", action="store_true",
                    help="time the backward alone (and fwd+bwd) at B = 1, 2, 4, 8, T=64, "
                         "Hk=Hv=2, Dk=Dv=64, fp32, one JSON line each, and exit")
    ap.add_argument("--dk-sweep", action="store_true",
                    help="time fwd+bwd at B=1, T=2048, Hk=16, Hv=64, Dv=128 for each key "
                         "width of --dks, one JSON line each, and exit")
    ap.add_argument("--dks", default="128,192,200,256,252",
                    help="key widths of --dk-sweep")
    ap.add_argument("--decode", type=int, default=0, metavar="B",
                    help="time single-step inference (T=1, state updated in place, no "
                         "save buffer) at batch B with the same heads, and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- helpers --
def algorithmic_bytes(B, T, Hk, Hv, Dk, Dv, esz, nch, s0=False, dst=False):
    """The minimum HBM bytes of each call, every tensor touched once: the
    forward reads q, k, v, g, beta (and S0) and writes y, the chunk
    checkpoints and S_T; the backward reads q, k, v, g, beta, dy (and dS_T)
    and the checkpoints and writes dq, dk, dv, dg, dbeta and dS0."""
    tok = B * T
    state = B * Hv * Dv * Dk * 4
    fwd = tok * (2 * Hk * Dk + 2 * Hv * Dv + 2 * Hv) * esz + nch * state + state
    bwd = tok * (4 * Hk * Dk + 3 * Hv * Dv + 4 * Hv) * esz + nch * state + state
    return fwd + (state if s0 else 0), bwd + (state if dst else 0)


def intermediate_bytes(B, T, Hv, Dv, Dk, nch, chunked):
    """HBM round trips of the design's own intermediates (written by one
    kernel, read by another): the fp32 residual e, the state-gradient
    checkpoints, the per-step vectors c and the per-chunk records."""
    rows32 = B * T * Hv * Dv * 4
    state = B * Hv * Dv * Dk * 4
    prep = B * Hv * nch * PREP_RECORD_BYTES if chunked else 0
    fwd = rows32 + 2 * prep                  # e written; records written + read
    bwd = rows32 + 2 * nch * state + 2 * rows32 + 2 * prep  # e read; H, c, records
    return fwd, bwd


class Step:
    """Every buffer of one fwd+bwd step at one shape, allocated up front, and
    the two library calls on the current stream."""

    def __init__(self, d, chunk, with_dST=False):
        import torch
        from gated_delta_rule_recurrence_amd import _lib, ops
        self.d = d
        q, v = d["q"], d["v"]
        dev = q.device
        B, T, Hk, Dk = q.shape
        Hv, Dv = v.shape[2], v.shape[3]
        self.shape = ops.shape_of(q, v, chunk, q.dtype)
        self.ckpt = torch.empty(_lib.checkpoint_bytes(self.shape), dtype=torch.uint8, device=dev)
        self.ws = torch.empty(_lib.backward_workspace_bytes(self.shape), dtype=torch.uint8,
                              device=dev)
        self.fws = torch.empty(max(_lib.forward_workspace_bytes(self.shape), 1),
                               dtype=torch.uint8, device=dev)
        self.chunked = _lib.forward_workspace_bytes(self.shape) > 0
        self.y = torch.empty_like(v)
        self.S_T = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
        self.outs = (torch.empty_like(q), torch.empty_like(d["k"]), torch.empty_like(v),
                     torch.empty_like(d["g"]), torch.empty_like(d["beta"]),
                     torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev))
        self.dST = (torch.randn((B, Hv, Dv, Dk), device=dev) if with_dST else None)
        self.saved = ops.Saved(self.ckpt, chunk, v=v if chunk > 64 else None)
        self.chunk = chunk
        self.nch = _lib.num_chunks(self.shape)
        self.stream = torch.cuda.current_stream(dev)

    def fwd(self):
        from gated_delta_rule_recurrence_amd import ops
        d = self.d
        ops.gdr_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("S0"),
                        chunk=self.chunk, y=self.y, S_T=self.S_T, ckpt=self.ckpt,
                        workspace=self.fws)

    def bwd(self):
        from gated_delta_rule_recurrence_amd import ops
        d = self.d
        ops.gdr_backward(d["q"], d["k"], d["g"], d["beta"], self.saved, d["dy"], self.dST,
                         workspace=self.ws, out=self.outs)

    def buffer_MB(self):
        return {"checkpoint_MB": self.ckpt.numel() / 1e6,
                "workspace_fwd_MB": (self.fws.numel() if self.chunked else 0) / 1e6,
                "workspace_bwd_MB": self.ws.numel() / 1e6}

    def time(self, n, warmup=3):
        """Median and min fwd, bwd and step ms over n steps (HIP events on
        the stream the library launches on)."""
        import torch
        for _ in range(warmup):
            self.fwd()
            self.bwd()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for e in ev:
            e[0].record(self.stream)
            self.fwd()
            e[1].record(self.stream)
            self.bwd()
            e[2].record(self.stream)
        torch.cuda.synchronize()
        f = np.array([e[0].elapsed_time(e[1]) for e in ev])
        b = np.array([e[1].elapsed_time(e[2]) for e in ev])
        return f, b


def live_kernel_ms(st, names_f, names_b, n=20):
    """Per-kernel durations of the two calls, by HIP events that the library
    records right after each of its kernel launches (gdr_set_launch_events:
    one event per kernel named plus one more, those past a call's last
    launch recorded at its end), over n steps run after the timed region:
    the median ms of each kernel, in launch order, for each call.  The extra
    event closes an interval with no kernel in it, whose median is the cost
    of the event records themselves (each kernel's figure includes it)."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib
    nf, nb = len(names_f) + 1, len(names_b) + 1
    rows = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + nf + nb)]
            for _ in range(n)]
    for row in rows:
        for e in row:
            e.record(st.stream)  # creates the underlying events
    torch.cuda.synchronize()
    try:
        for row in rows:
            _lib.check(_lib.set_launch_events([e.cuda_event for e in row[1:1 + nf]]),
                       "gdr_set_launch_events")
            row[0].record(st.stream)
            st.fwd()
            _lib.check(_lib.set_launch_events([e.cuda_event for e in row[2 + nf:]]),
                       "gdr_set_launch_events")
            row[1 + nf].record(st.stream)
            st.bwd()
    finally:
        _lib.set_launch_events([])
    torch.cuda.synchronize()
    med = lambda i: float(np.median([r[i].elapsed_time(r[i + 1]) for r in rows]))
    return {"gdr_forward": {names_f[i]: med(i) for i in range(nf - 1)},
            "gdr_backward": {names_b[i]: med(1 + nf + i) for i in range(nb - 1)},
            "event_gap_ms": med(nf - 1), "steps": n}


def device_problem(B, T, Hk, Hv, Dk, Dv, dev, seed, dtype, decay="weak", S0_std=None):
    from gated_delta_rule_recurrence_amd import inputs
    return inputs.draw_device(B, T, Hk, Hv, Dk, Dv, device=dev, seed=seed, normalised=True,
                              decay=decay, S0_std=S0_std, dtype=dtype)


def copy_bandwidth(dev, mib=1024, reps=5):
    """Attainable HBM bandwidth: a plain device copy of `mib` MiB (read +
    write), best of `reps` by HIP events."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (best * 1e-3) / 1e9


PROBE_LIB = os.path.join(ROOT, "tests", "probe", "libgdr_probe.so")


def compute_peaks(dev, reps=3):
    """Attainable compute rates: loops of one instruction kind from the
    test-only probe library (fp32 FMA on the vector ALU, non-packed as this
    build's vector code is; bf16 and fp32 MFMA), 2048 workgroups of 256
    threads, best of `reps` launches by HIP events on torch's stream.  None
    when the probe library is not built."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.gdr_probe_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    # kind, iterations, flops per launch
    kinds = {"fp32_fma_vector": (0, 1000, 256 * 256 * blocks),
             "bf16_mfma": (1, 5000, blocks * 4 * 4 * 16384),
             "fp32_mfma": (2, 4000, blocks * 4 * 4 * 2048)}
    res = {}
    for name, (kind, iters, per_iter) in kinds.items():
        if lib.gdr_probe_peak(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                              ctypes.c_void_p(stream)) != 0:
            raise RuntimeError(f"peak probe {name} failed to launch")
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lib.gdr_probe_peak(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                               ctypes.c_void_p(stream))
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[name + "_TFLOPs"] = per_iter * iters / (best * 1e-3) / 1e12
    del out
    return res


# ------------------------------------------------------------------ modes --
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
    checkpoint interval C: median fwd and bwd times by HIP events, save
    buffer and workspace sizes, algorithmic HBM bytes.  Inputs drawn on the
    device (inputs.draw_device: the draw() distributions)."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib
    dev = torch.device("cuda:0")
    _lib.load()
    B, T, Hk, Hv, Dk, Dv = 4, 8192, 16, 64, 192, 128
    d = device_problem(B, T, Hk, Hv, Dk, Dv, dev, args.seed, args.dtype, decay="mix",
                       S0_std=0.05)
    torch.cuda.synchronize()
    esz = 2 if args.dtype == "bf16" else 4
    for C in (int(c) for c in args.chunks.split(",")):
        torch.cuda.reset_peak_memory_stats(dev)
        st = Step(d, C)
        f, b = st.time(10)
        f, b = float(np.median(f)), float(np.median(b))
        fb, bb = algorithmic_bytes(B, T, Hk, Hv, Dk, Dv, esz, st.nch, s0=True)
        print(json.dumps({"chunk_sweep": {
            "C": C, "B": B, "T": T, "dtype": args.dtype,
            "path": "chunked" if st.chunked else "per-step sweeps",
            "fwd_ms_median": f, "bwd_ms_median": b, "tokens_per_s": B * T / ((f + b) * 1e-3),
            **st.buffer_MB(),
            "peak_device_memory_MB": torch.cuda.max_memory_allocated(dev) / 1e6,
            "algorithmic_bytes": fb + bb,
            "hbm_frac_algorithmic": (fb + bb) / ((f + b) * 1e-3) / 1e9 / HBM_PEAK_GBS}}),
            flush=True)
        del st
        torch.cuda.empty_cache()


def t_sweep(args):
    """The headline heads (B=1, Hk=16, Hv=64, Dk=192, Dv=128, bf16) at the
    lengths of the mlx-lm PR #1217 Performance table: median fwd, bwd and
    step ms (HIP events), tokens/s, save buffer and workspaces, and the peak
    device memory of the step (inputs included)."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib
    dev = torch.device("cuda:0")
    _lib.load()
    Hk, Hv, Dk, Dv = 16, 64, 192, 128
    esz = 2 if args.dtype == "bf16" else 4
    torch.zeros(1, device=dev)  # initialise the device before its memory statistics
    for T in (256, 512, 1024, 2048):
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        d = device_problem(1, T, Hk, Hv, Dk, Dv, dev, args.seed, args.dtype)
        st = Step(d, args.chunk)
        f, b = st.time(50, warmup=10)
        fm, bm = float(np.median(f)), float(np.median(b))
        sm = float(np.median(f + b))
        fb, bb = algorithmic_bytes(1, T, Hk, Hv, Dk, Dv, esz, st.nch)
        elems = T * Hv * Dv * Dk
        print(json.dumps({"t_sweep": {
            "T": T, "B": 1, "chunk": args.chunk, "dtype": args.dtype,
            "fwd_ms_median": fm, "bwd_ms_median": bm, "step_ms_median": sm,
            "tokens_per_s": T / (sm * 1e-3),
            "useful_tflops": (FLOPS_FWD + FLOPS_BWD) * elems / (sm * 1e-3) / 1e12,
            "frac_fp32_peak": (FLOPS_FWD + FLOPS_BWD) * elems / (sm * 1e-3) / 1e12
                              / FP32_PEAK_TF,
            "hbm_frac_algorithmic": (fb + bb) / (sm * 1e-3) / 1e9 / HBM_PEAK_GBS,
            **st.buffer_MB(),
            "peak_device_memory_MB": torch.cuda.max_memory_allocated(dev) / 1e6}}),
            flush=True)
        del st, d


def vjp_batch(args):
    """The focused VJP shape of unsloth-zoo PR #776 (T=64, Hk=Hv=2,
    Dk=Dv=64, fp32, no mask) at B = 1, 2, 4, 8: median backward ms and
    median fwd+bwd ms by HIP events over 200 steps."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib
    dev = torch.device("cuda:0")
    _lib.load()
    for B in (1, 2, 4, 8):
        d = device_problem(B, 64, 2, 2, 64, 64, dev, args.seed, "f32")
        st = Step(d, 64)
        f, b = st.time(200, warmup=20)
        print(json.dumps({"vjp_batch": {
            "B": B, "T": 64, "Hk": 2, "Hv": 2, "Dk": 64, "Dv": 64, "dtype": "f32",
            "bwd_ms_median": float(np.median(b)), "bwd_ms_min": float(b.min()),
            "fwd_bwd_ms_median": float(np.median(f + b))}}), flush=True)
        del st, d


def dk_sweep(args):
    """Key widths at the headline's other dims (B=1, T=2048, Hk=16, Hv=64,
    Dv=128, chunk 64): median fwd, bwd and step ms by HIP events over 50
    steps, and which forward path the shape takes (the chunked sweeps, or
    the per-step sweeps when the forward needs no workspace)."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib
    dev = torch.device("cuda:0")
    _lib.load()
    for Dk in (int(x) for x in args.dks.split(",")):
        d = device_problem(1, 2048, 16, 64, Dk, 128, dev, args.seed, args.dtype)
        st = Step(d, 64)
        f, b = st.time(50, warmup=10)
        sm = float(np.median(f + b))
        print(json.dumps({"dk_sweep": {
            "Dk": Dk, "B": 1, "T": 2048, "Hk": 16, "Hv": 64, "Dv": 128, "dtype": args.dtype,
            "path": "chunked" if st.chunked else "per-step sweeps",
            "fwd_ms_median": float(np.median(f)), "bwd_ms_median": float(np.median(b)),
            "step_ms_median": sm, "tokens_per_s": 2048 / (sm * 1e-3)}}), flush=True)
        del st, d
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


def cpu_baseline(T, seed, dtype, workers=0):
    """The float64 oracle as it stands, on the host cores: every (batch row,
    kv group) unit of the workload, forward + backward (oracle.backward runs
    the forward recurrence and then the reverse sweep), one unit per worker
    process at a time, one thread each.  Runs before the GPU is touched."""
    from oracle import pool
    from gated_delta_rule_recurrence_amd import inputs
    p = inputs.qwen35_9b(T, seed=seed, dtype=dtype)
    cpus, aff = pool.host_cores()
    workers = workers or min(aff, 16)
    units = [pool.unit_inputs(p, b, hk) for b in range(p.B) for hk in range(p.Hk)]
    wall, per_unit = pool.time_units(units, workers)
    rep = p.Hv // p.Hk
    return {"value": p.B * T / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"all {len(units)} (batch row, kv group) units of the workload (B={p.B}, "
                      f"T={T}, {rep} value heads each), forward + backward, on {workers} "
                      f"worker processes of one thread: {wall:.1f} s wall, "
                      f"{sum(per_unit):.1f} s of CPU work",
            "os_cpu_count": cpus, "affinity_cpus": aff, "workers": workers,
            "single_core_tokens_per_s": p.B * T / sum(per_unit)}


# ------------------------------------------------------------- main step --
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path "
              "shards by (batch row, kv head) with no communication between GPUs",
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
    if args.t_sweep:
        t_sweep(args)
        return
    if args.vjp_batch:
        vjp_batch(args)
        return
    if args.dk_sweep:
        dk_sweep(args)
        return

    # the CPU baseline first: its worker processes start before this process
    # touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.T, args.seed, args.dtype, args.cpu_workers)

    import torch
    from gated_delta_rule_recurrence_amd import _lib
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    _lib.load()  # fail loudly if the HIP library is missing

    from gated_delta_rule_recurrence_amd import inputs
    p = inputs.qwen35_9b(args.T, seed=args.seed, dtype=args.dtype, B=args.B)
    dt = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    d = {n: t(getattr(p, n)) for n in ("q", "k", "v", "g", "beta", "dy")}
    B, T, Hk, Hv, Dk, Dv = p.B, p.T, p.Hk, p.Hv, p.Dk, p.Dv
    st = Step(d, args.chunk)   # every buffer allocated up front
    stream = st.stream
    fwd, bwd = st.fwd, st.bwd

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
    copy_gbs = copy_bandwidth(dev)
    peaks = compute_peaks(dev)
    ms = wall * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms / 1e3)

    elems = B * T * Hv * Dv * Dk  # state-element steps
    fwd_flops, bwd_flops = FLOPS_FWD * elems, FLOPS_BWD * elems
    fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12
    # the bf16-product sweep kernels take bf16 inputs with Dk % 8 == 0 and Dv % 4 == 0
    sfx = "_bf16" if (args.dtype == "bf16" and Dk % 8 == 0 and Dv % 4 == 0) else ""
    chunk_name = ("chunk_bf16_kernel" if (args.dtype == "bf16" and Dk % 8 == 0 and Dv % 8 == 0
                                          and 48 < Dk <= 256) else "chunk_kernel")
    all_tf = (FLOPS_FWD + FLOPS_BWD) * elems / (ms * 1e-3) / 1e12
    esz = 2 if args.dtype == "bf16" else 4
    fwd_bytes, bwd_bytes = algorithmic_bytes(B, T, Hk, Hv, Dk, Dv, esz, st.nch)
    fwd_mid, bwd_mid = intermediate_bytes(B, T, Hv, Dv, Dk, st.nch, st.chunked)

    default_workload = (args.T, args.B, args.chunk, args.dtype) == (2048, 1, 64, "bf16")
    # the kernels of each call one by one (the chunked path at chunk <= 64;
    # a fourth backward interval is the head-group sum when the chunk kernel
    # splits the value heads, else empty)
    live = None
    if st.chunked and args.chunk <= 64:
        live = live_kernel_ms(st, ["prep_kernel<fwd>", f"fwd_chunked{sfx}_kernel"],
                              ["prep_kernel<bwd>", f"bwd_chunked{sfx}_kernel", chunk_name,
                               "head_sum_kernel"])
    prof_ok = (default_workload and PROFILE["sources_sha256_16"] is not None
               and sources_digest() == PROFILE["sources_sha256_16"])
    traffic = fwd_traffic = None
    counters = bwd_pipes = fwd_pipes = None
    if prof_ok:
        traffic = PROFILE["bwd_read_bytes"] + PROFILE["bwd_write_bytes"]
        fwd_traffic = PROFILE["fwd_read_bytes"] + PROFILE["fwd_write_bytes"]
        counters = PROFILE["kernels"]
        bwd_pipes, fwd_pipes = pipe_busy(BWD_KERNELS), pipe_busy(FWD_KERNELS)

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
        # the dominant call, gdr_backward, timed with HIP events on the
        # library's stream.  Its products deliver fp32 accuracy (fp32 MFMA,
        # or bf16 MFMA on exact three-piece splits), so the work is priced as
        # fp32: `achieved` counts the recurrence's useful fp32-equivalent
        # flops (15 per state element per step), not the issued piece
        # products.
        "roofline": {"bound": "mfma", "kernel": f"gdr_backward (prep_kernel<bwd>, "
                     f"bwd_chunked{sfx}_kernel, {chunk_name})",
                     "achieved": bwd_tf, "peak": FP32_PEAK_TF,
                     "unit": "TFLOP/s", "frac": bwd_tf / FP32_PEAK_TF,
                     "flops_basis": "useful fp32-equivalent, 15*B*T*Hv*Dv*Dk per call",
                     "traffic": traffic,
                     "traffic_source": PROFILE["source"] if prof_ok else None,
                     "flops_per_launch": bwd_flops,
                     "algorithmic_bytes_per_launch": bwd_bytes,
                     "intermediate_bytes_per_launch": bwd_mid,
                     "hbm_frac_algorithmic": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "hbm_frac_counters": (traffic / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
                                           if traffic else None),
                     # SQ counters, weighted by kernel time over the call
                     "pipes_counters": bwd_pipes,
                     "avg_launch_ms": bwd_ms},
        "forward": {"kernel": f"gdr_forward (prep_kernel<fwd>, fwd_chunked{sfx}_kernel)",
                    "achieved_tflops": fwd_tf, "frac": fwd_tf / FP32_PEAK_TF,
                    "flops_per_launch": fwd_flops, "algorithmic_bytes_per_launch": fwd_bytes,
                    "intermediate_bytes_per_launch": fwd_mid,
                    "traffic": fwd_traffic,
                    "pipes_counters": fwd_pipes,
                    "hbm_frac_algorithmic": fwd_bytes / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "avg_launch_ms": fwd_ms},
        "counters": counters,
        "kernels_live_ms": live,
        "achievable_hbm_GBps": copy_gbs,
        "achievable_compute": peaks,
        "timing": {"wall_ms_per_step": ms, "step_ms_median": float(np.median(step_ms)),
                   "step_ms_min": float(step_ms.min()),
                   "flushed_step_ms_median": float(np.median(flushed_ms)),
                   "flushed_step_ms_min": float(flushed_ms.min()), "flushed_steps": nflush},
        "peak_device_memory_MB": peak_mb,
        "breakdown": {"fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                      "useful_tflops_whole_step": all_tf,
                      "frac_whole_step_vs_fp32_peak": all_tf / FP32_PEAK_TF,
                      **st.buffer_MB()},
    }
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
