"""PyTorch-facing entry points with the same names as the C ABI.

PyTorch supplies device memory and the current HIP stream; the arithmetic all
happens in libgdr.so.  Tensors must be contiguous, on one GPU, and q, k, v,
g, beta, dy share one dtype (torch.float32 or torch.bfloat16); states are
torch.float32.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

DEFAULT_CHUNK = 64

_DTYPES = {torch.float32: _lib.GDR_F32, torch.bfloat16: _lib.GDR_BF16}


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _check_tensor(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class Saved:
    """What gdr_forward leaves for gdr_backward (opaque fp32 buffer), with
    the settings the backward must repeat."""

    ckpt: torch.Tensor
    chunk: int
    log_decay: bool = False
    mask: Optional[torch.Tensor] = None
    # the forward's v: the backward replays the tiles from it when chunk > 64
    v: Optional[torch.Tensor] = None


def shape_of(q, v, chunk, dtype, log_decay=False) -> _lib.GdrShape:
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    decay = _lib.GDR_DECAY_LOG if log_decay else _lib.GDR_DECAY_G
    return _lib.make_shape(B, T, Hk, Hv, Dk, Dv, chunk, _DTYPES[dtype], decay)


def _as_mask(mask, B, T, device):
    if mask is None:
        return None
    if mask.dtype == torch.bool:
        mask = mask.to(torch.uint8)
    _check_tensor("mask", mask, (B, T), torch.uint8, device)
    return mask


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def gdr_forward(q, k, v, g, beta, S0=None, *, chunk=DEFAULT_CHUNK, save=True,
                out_state=True, y=None, S_T=None, ckpt=None, workspace=None,
                log_decay=False, mask=None):
    """Forward pass.  Returns (y, S_T or None, Saved or None).

    q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; g, beta [B,T,Hv]; S0 [B,Hv,Dv,Dk] fp32
    or None.  Output and scratch buffers may be passed in to avoid allocation.
    log_decay: g holds the log of the decay (GDR_DECAY_LOG).
    mask: [B,T] torch.uint8 (or bool) or None; a step with mask 0 leaves the
    state unchanged (an identity step).  S_T may be S0 (in place).
    """
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev, dt = q.device, q.dtype
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    _check_tensor("q", q, (B, T, Hk, Dk), dt, dev)
    _check_tensor("k", k, (B, T, Hk, Dk), dt, dev)
    _check_tensor("v", v, (B, T, Hv, Dv), dt, dev)
    _check_tensor("g", g, (B, T, Hv), dt, dev)
    _check_tensor("beta", beta, (B, T, Hv), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, Hv, Dv, Dk), torch.float32, dev)
    mask = _as_mask(mask, B, T, dev)
    shape = shape_of(q, v, chunk, dt, log_decay)
    if y is None:
        y = torch.empty((B, T, Hv, Dv), dtype=dt, device=dev)
    _check_tensor("y", y, (B, T, Hv, Dv), dt, dev)
    if out_state and S_T is None:
        S_T = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if not out_state:
        S_T = None
    saved = None
    if save:
        nbytes = _lib.checkpoint_bytes(shape)
        if ckpt is None:
            ckpt = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        if ckpt.numel() * ckpt.element_size() < nbytes:
            raise ValueError("ckpt buffer too small")
        saved = Saved(ckpt, chunk, bool(log_decay), mask, v if chunk > 64 else None)
    wbytes = _lib.forward_workspace_bytes(shape)
    if wbytes > 0 and workspace is None:
        workspace = torch.empty((wbytes,), dtype=torch.uint8, device=dev)
    if wbytes > 0 and workspace.numel() * workspace.element_size() < wbytes:
        raise ValueError("forward workspace too small")
    st = _lib.forward_raw(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                          _ptr(S0), _ptr(y), _ptr(S_T),
                          _ptr(saved.ckpt) if saved else 0,
                          _ptr(workspace) if wbytes > 0 else 0, wbytes, _stream(dev),
                          mask=_ptr(mask))
    _lib.check(st, "gdr_forward")
    return y, S_T, saved


def gdr_backward(q, k, g, beta, saved: Saved, dy, dS_T=None, *, want_dS0=True,
                 workspace=None, out=None):
    """Backward pass.  Returns (dq, dk, dv, dg, dbeta, dS0 or None).

    With a log-decay forward (saved.log_decay), dg is dL/d(log g).  For
    chunk > 64 the backward replays the forward tiles from saved.v, the
    forward's v."""
    dev, dt = q.device, q.dtype
    B, T, Hk, Dk = q.shape
    Hv, Dv = dy.shape[2], dy.shape[3]
    _check_tensor("q", q, (B, T, Hk, Dk), dt, dev)
    _check_tensor("k", k, (B, T, Hk, Dk), dt, dev)
    _check_tensor("g", g, (B, T, Hv), dt, dev)
    _check_tensor("beta", beta, (B, T, Hv), dt, dev)
    _check_tensor("dy", dy, (B, T, Hv, Dv), dt, dev)
    if dS_T is not None:
        _check_tensor("dS_T", dS_T, (B, Hv, Dv, Dk), torch.float32, dev)
    shape = shape_of(q, dy, saved.chunk, dt, saved.log_decay)
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty((B, T, Hv, Dv), dtype=dt, device=dev)
        dg = torch.empty_like(g)
        dbeta = torch.empty_like(beta)
        dS0 = (torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
               if want_dS0 else None)
    else:
        dq, dk, dv, dg, dbeta, dS0 = out
    nbytes = _lib.backward_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    st = _lib.backward_raw(shape, _ptr(q), _ptr(k), _ptr(g), _ptr(beta),
                           _ptr(saved.ckpt), _ptr(dy), _ptr(dS_T), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dS0),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(dev), mask=_ptr(saved.mask), v=_ptr(saved.v))
    _lib.check(st, "gdr_backward")
    return dq, dk, dv, dg, dbeta, dS0


class GatedDeltaRule(torch.autograd.Function):
    """y, S_T = gated_delta_rule(q, k, v, g, beta, S0) with the library VJP."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, S0, chunk, log_decay=False, mask=None):
        y, S_T, saved = gdr_forward(q, k, v, g, beta, S0, chunk=chunk,
                                    log_decay=log_decay, mask=mask)
        ctx.has_S0 = S0 is not None
        # v is needed again only when the backward replays the tiles (chunk >
        # 64); it then goes through save_for_backward like the other inputs
        ctx.with_v = saved.v is not None
        saved.v = None
        ctx.saved = saved
        ctx.save_for_backward(q, k, g, beta, *((v,) if ctx.with_v else ()))
        return y, S_T

    @staticmethod
    def backward(ctx, dy, dS_T):
        q, k, g, beta, *rest = ctx.saved_tensors
        if ctx.with_v:
            ctx.saved.v = rest[0]
        # autograd materialises absent cotangents as zeros
        dy = dy.contiguous()
        dS_T = None if dS_T is None else dS_T.contiguous()
        dq, dk, dv, dg, dbeta, dS0 = gdr_backward(
            q, k, g, beta, ctx.saved, dy, dS_T, want_dS0=ctx.has_S0)
        return dq, dk, dv, dg, dbeta, (dS0 if ctx.has_S0 else None), None, None, None


def gated_delta_rule(q, k, v, g, beta, S0=None, chunk=DEFAULT_CHUNK, log_decay=False,
                     mask=None):
    """Autograd-enabled forward: returns (y, S_T).  With log_decay, g holds
    the log of the decay and its gradient is dL/d(log g); mask [B,T] marks
    identity steps with 0."""
    return GatedDeltaRule.apply(q, k, v, g, beta, S0, chunk, log_decay, mask)
