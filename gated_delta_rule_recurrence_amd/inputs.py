"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws random numbers and lays them out; it holds none of the
recurrence's arithmetic.  Both the float64 oracle tests and the GPU path take
their inputs from here, so the two sides see identical data.

Draw recipe (mlx issue #4614 "mx.fast.gated_delta_update VJP: wrong gradient
w.r.t. g", repro script, input-draw block):
  * q = unit(N(0,1)) * Dk**-0.5 and k = unit(N(0,1)) in the normalised draw,
    plain N(0,1) in the literal draw;
  * v ~ N(0,1);
  * log g = -exp(N(mu, 0.5)) with mu = -2 (weak decay) or +2 (strong decay);
  * beta = sigmoid(N(0,1));
  * the upstream cotangent dy ~ N(0,1).
Draw order: q, k, v, log g, beta, dy, then dS_T, then S0.  Every draw is
float64 from ``numpy.random.default_rng(seed)``; the caller casts.

Layouts (same page, recurrence helper): q, k [B,T,Hk,Dk]; v, y, dy
[B,T,Hv,Dv]; g, beta [B,T,Hv]; states [B,Hv,Dv,Dk].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Problem",
    "draw",
    "bf16_round",
    "toy",
    "batch_rows",
    "strong_decay",
    "qwen35_9b",
    "long_context",
]


@dataclass
class Problem:
    """One seeded problem instance (all arrays float64 unless stated)."""

    B: int
    T: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    dy: np.ndarray
    S0: Optional[np.ndarray] = None
    dST: Optional[np.ndarray] = None
    dtype: str = "f32"  # "f32" or "bf16": the element type handed to the kernels
    meta: Dict[str, object] = field(default_factory=dict)
    log_decay: bool = False  # g holds log of the decay
    mask: Optional[np.ndarray] = None  # [B, T] uint8, 0 = identity step

    def arrays(self):
        return dict(q=self.q, k=self.k, v=self.v, g=self.g, beta=self.beta,
                    dy=self.dy, S0=self.S0, dST=self.dST)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even), as float64.

    Goes through the float32 bit pattern: add 0x7FFF plus the lowest kept bit,
    then clear the low 16 bits.  NaN is kept NaN.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.nan
    return out.reshape(np.shape(x))


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def draw(B, T, Hk, Hv, Dk, Dv, *, seed=0, normalised=False, decay="weak",
         S0_std=None, dST_std=None, dtype="f32", log_decay=False) -> Problem:
    """Draw one problem.

    decay: "weak" (mu=-2), "strong" (mu=+2) or "mix" (value head hv even ->
    weak, odd -> strong).  S0_std / dST_std: None means the tensor is absent
    (zero).  dtype "bf16" rounds every input to bfloat16 (RNE) so that the
    oracle and the kernels see the same values.  log_decay: g holds the
    drawn log g itself (the same draws), for the log-decay input.
    """
    if Hv % Hk:
        raise ValueError("Hv must be a multiple of Hk")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    if normalised:
        q = _unit(q) * Dk ** -0.5
        k = _unit(k)
    v = rng.standard_normal((B, T, Hv, Dv))
    if decay == "weak":
        mu = np.full((Hv,), -2.0)
    elif decay == "strong":
        mu = np.full((Hv,), 2.0)
    elif decay == "mix":
        mu = np.where(np.arange(Hv) % 2 == 0, -2.0, 2.0)
    else:
        raise ValueError(decay)
    log_g = -np.exp(rng.normal(0.0, 0.5, (B, T, Hv)) + mu)
    g = np.exp(log_g)
    beta = _sigmoid(rng.standard_normal((B, T, Hv)))
    dy = rng.standard_normal((B, T, Hv, Dv))
    dST = None
    if dST_std is not None:
        dST = rng.normal(0.0, dST_std, (B, Hv, Dv, Dk))
    S0 = None
    if S0_std is not None:
        S0 = rng.normal(0.0, S0_std, (B, Hv, Dv, Dk))
    p = Problem(B, T, Hk, Hv, Dk, Dv, q, k, v, log_g if log_decay else g, beta, dy,
                S0, dST, dtype,
                meta=dict(seed=seed, normalised=normalised, decay=decay,
                          mean_log_g=float(log_g.mean()) if log_g.size else float("nan")),
                log_decay=log_decay)
    if dtype == "bf16":
        for name in ("q", "k", "v", "g", "beta", "dy"):
            setattr(p, name, bf16_round(getattr(p, name)))
        # states stay fp32 on the device side
        if p.S0 is not None:
            p.S0 = p.S0.astype(np.float32).astype(np.float64)
        if p.dST is not None:
            p.dST = p.dST.astype(np.float32).astype(np.float64)
    elif dtype == "f32":
        for name in ("q", "k", "v", "g", "beta", "dy", "S0", "dST"):
            a = getattr(p, name)
            if a is not None:
                setattr(p, name, a.astype(np.float32).astype(np.float64))
    else:
        raise ValueError(dtype)
    return p


def draw_device(B, T, Hk, Hv, Dk, Dv, *, device, seed=0, normalised=True, decay="weak",
                S0_std=None, dtype="bf16"):
    """The distributions of draw() sampled directly on a torch device (its
    own seeded generator, so not the same numbers as draw()): for timing
    workloads too large to draw on the host in float64.  Returns a dict of
    device tensors q, k, v, g, beta, dy (in `dtype`) and S0 (fp32 or None).
    decay "mix": weak on even value heads, strong on odd ones."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    f32 = dict(device=device, dtype=torch.float32, generator=gen)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    q = torch.randn((B, T, Hk, Dk), **f32)
    k = torch.randn((B, T, Hk, Dk), **f32)
    if normalised:
        q = unit(q) * Dk ** -0.5
        k = unit(k)
    v = torch.randn((B, T, Hv, Dv), **f32)
    if decay == "weak":
        mu = torch.full((Hv,), -2.0, device=device)
    elif decay == "strong":
        mu = torch.full((Hv,), 2.0, device=device)
    elif decay == "mix":
        mu = torch.where(torch.arange(Hv, device=device) % 2 == 0, -2.0, 2.0)
    else:
        raise ValueError(decay)
    g = torch.exp(-torch.exp(torch.randn((B, T, Hv), **f32) * 0.5 + mu))
    beta = torch.sigmoid(torch.randn((B, T, Hv), **f32))
    dy = torch.randn((B, T, Hv, Dv), **f32)
    S0 = None if S0_std is None else torch.randn((B, Hv, Dv, Dk), **f32) * S0_std
    out = {n: x.to(dt).contiguous() for n, x in
           dict(q=q, k=k, v=v, g=g, beta=beta, dy=dy).items()}
    out["S0"] = S0
    return out


# ---- the five workload recipes -------------------------------------------

def toy(seed=0, with_dST=False) -> Problem:
    """Toy shape of the mlx-lm PR #1217 finite-difference test (Correctness
    section): B=1, T=4, Hk=2, Hv=4, Dk=Dv=8, fp32, literal N(0,1) q/k,
    S0 ~ N(0, 0.1)."""
    return draw(1, 4, 2, 4, 8, 8, seed=seed, normalised=False, decay="weak",
                S0_std=0.1, dST_std=1.0 if with_dST else None)


def batch_rows(B=8, seed=0) -> Problem:
    """Focused-VJP shape of unsloth-zoo PR #776 (performance table): T=64,
    Hk=Hv=2, Dk=Dv=64, S0=0.  Draw B=8 once and slice, so row 0 is the same
    for every B (B=1 is the control case)."""
    p = draw(8, 64, 2, 2, 64, 64, seed=seed, normalised=True, decay="weak")
    if B != 8:
        for name in ("q", "k", "v", "g", "beta", "dy"):
            setattr(p, name, getattr(p, name)[:B].copy())
        p.B = B
    return p


def strong_decay(Hk, Hv, seed=0, normalised=False, T=128, D=128) -> Problem:
    """Strong-decay GQA numerics of mlx issue #4614 (accuracy table): B=1,
    T=128, Dk=Dv=128, log g = -exp(N(2, 0.5)) (mean about -8.3)."""
    return draw(1, T, Hk, Hv, D, D, seed=seed, normalised=normalised,
                decay="strong")


def qwen35_9b(T, seed=0, dtype="bf16", B=1) -> Problem:
    """Qwen3.5-9B linear_attn shape (mlx-lm PR #1217, Performance table):
    B=1, Hk=16, Hv=64, Dk=192, Dv=128, bf16 inputs, fp32 state, weak decay,
    normalised q/k, S0=0."""
    return draw(B, T, 16, 64, 192, 128, seed=seed, normalised=True,
                decay="weak", dtype=dtype)


def long_context(seed=0, T=8192, B=4, dtype="bf16") -> Problem:
    """Long-context training shape: B=4, T=8192, Qwen3.5-9B heads, nonzero
    trainable S0 ~ N(0, 0.05), weak/strong decay alternating over value
    heads."""
    return draw(B, T, 16, 64, 192, 128, seed=seed, normalised=True,
                decay="mix", S0_std=0.05, dtype=dtype)
