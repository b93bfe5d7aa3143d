"""Run the float64 oracle over independent (batch row, kv group) units in
worker processes.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the benchmark's CPU
baseline and the tests use it; nothing in the product path does.  The oracle
itself is unchanged; units are independent (a kv group's value heads never
meet another group's), so running them side by side is the same computation.
Workers are started with the "spawn" method (a fresh interpreter that imports
only numpy and this package) and run one unit at a time on one thread.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from . import gdr_oracle as O


def unit_inputs(p, b, hk):
    """The inputs of batch row b, kv group hk of a Problem-like object with
    fields q, k, v, g, beta, dy, S0, dST, Hk, Hv (plain numpy arrays)."""
    rep = p.Hv // p.Hk
    hs = slice(hk * rep, (hk + 1) * rep)
    bs = slice(b, b + 1)
    sl = lambda a: None if a is None else np.ascontiguousarray(a)
    return dict(q=sl(p.q[bs, :, hk:hk + 1]), k=sl(p.k[bs, :, hk:hk + 1]),
                v=sl(p.v[bs, :, hs]), g=sl(p.g[bs, :, hs]), beta=sl(p.beta[bs, :, hs]),
                dy=sl(p.dy[bs, :, hs]), S0=None if p.S0 is None else sl(p.S0[bs, hs]),
                dST=None if p.dST is None else sl(p.dST[bs, hs]))


def _time_backward(u):
    """One unit's forward + backward: O.backward runs the forward recurrence
    (every state and read-out) and then the reverse sweep.  Returns seconds."""
    t0 = time.perf_counter()
    O.backward(u["q"], u["k"], u["v"], u["g"], u["beta"], u["dy"], u["S0"], u["dST"])
    return time.perf_counter() - t0


def _init_worker():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"


def host_cores():
    """(os.cpu_count(), size of this process's CPU affinity mask)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return os.cpu_count() or 1, aff


def time_units(units, workers):
    """Run _time_backward over `units` (dicts from unit_inputs) on `workers`
    spawned processes.  Returns (wall seconds, per-unit seconds)."""
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=_init_worker) as ex:
        # start every worker (interpreter, imports) on a two-step slice first
        tiny = {n: (None if a is None or n in ("S0", "dST") else a[:, :2])
                for n, a in units[0].items()}
        tiny["S0"], tiny["dST"] = units[0]["S0"], units[0]["dST"]
        list(ex.map(_time_backward, [tiny] * workers))
        t0 = time.perf_counter()
        per_unit = list(ex.map(_time_backward, units))
        wall = time.perf_counter() - t0
    return wall, per_unit
