"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the float64 oracle on the same seeded inputs and compare them."""
from __future__ import annotations

import sys

import numpy as np

import oracle.gdr_oracle as O

OUTS = ("y", "S_T", "dq", "dk", "dv", "dg", "dbeta", "dS0")
TOL = {"f32": 1e-5, "bf16": 1e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype, dev):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return t.to(dtype).contiguous()


def torch_dtype(p):
    import torch
    return torch.float32 if p.dtype == "f32" else torch.bfloat16


def device_inputs(p, dev):
    import torch
    dt = torch_dtype(p)
    d = {n: to_dev(getattr(p, n), dt, dev) for n in ("q", "k", "v", "g", "beta", "dy")}
    d["S0"] = None if p.S0 is None else to_dev(p.S0, torch.float32, dev)
    d["dST"] = None if p.dST is None else to_dev(p.dST, torch.float32, dev)
    return d


def run_gpu(p, dev, chunk=64, d=None, want_saved=False):
    """Forward + backward through libgdr; returns float64 numpy outputs."""
    import torch
    from gated_delta_rule_recurrence_amd import ops
    d = d or device_inputs(p, dev)
    mask = None
    if p.mask is not None:
        mask = torch.from_numpy(np.ascontiguousarray(p.mask, np.uint8)).to(dev)
    y, ST, saved = ops.gdr_forward(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                   d["S0"], chunk=chunk, log_decay=p.log_decay, mask=mask)
    dq, dk, dv, dg, db, dS0 = ops.gdr_backward(d["q"], d["k"], d["g"], d["beta"],
                                               saved, d["dy"], d["dST"])
    torch.cuda.synchronize()
    outs = dict(y=y, S_T=ST, dq=dq, dk=dk, dv=dv, dg=dg, dbeta=db, dS0=dS0)
    res = {k: v.float().cpu().numpy().astype(np.float64) for k, v in outs.items()}
    if want_saved:
        res["_saved"] = saved
    return res


def run_oracle(p, b=None, hk=None):
    """Oracle outputs; optionally only batch row b and kv group hk (the kv
    groups are independent, so a group is computed on its own)."""
    q, k, v, g, beta, dy, S0, dST = p.q, p.k, p.v, p.g, p.beta, p.dy, p.S0, p.dST
    mask = p.mask
    if b is not None:
        rep = p.Hv // p.Hk
        hs = slice(hk * rep, (hk + 1) * rep)
        bs = slice(b, b + 1)
        q, k = q[bs, :, hk:hk + 1], k[bs, :, hk:hk + 1]
        v, g, beta, dy = v[bs, :, hs], g[bs, :, hs], beta[bs, :, hs], dy[bs, :, hs]
        S0 = None if S0 is None else S0[bs, hs]
        dST = None if dST is None else dST[bs, hs]
        mask = None if mask is None else mask[bs]
    y, ST = O.forward(q, k, v, g, beta, S0, log_decay=p.log_decay, mask=mask)
    dq, dk, dv, dg, db, dS0 = O.backward(q, k, v, g, beta, dy, S0, dST,
                                         log_decay=p.log_decay, mask=mask)
    return dict(y=y, S_T=ST, dq=dq, dk=dk, dv=dv, dg=dg, dbeta=db, dS0=dS0)


def slice_group(res, p, b, hk):
    rep = p.Hv // p.Hk
    hs = slice(hk * rep, (hk + 1) * rep)
    bs = slice(b, b + 1)
    out = {}
    for name, a in res.items():
        if name.startswith("_"):
            continue
        if name in ("dq", "dk"):
            out[name] = a[bs, :, hk:hk + 1]
        elif name in ("S_T", "dS0"):
            out[name] = a[bs, hs]
        else:
            out[name] = a[bs, :, hs]
    return out


def compare(gpu, ref, tol, label=""):
    errs = {n: O.rel_l2(gpu[n], ref[n]) for n in OUTS}
    log(f"  {label} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{label}: rel L2 above {tol}: {bad}"
    for n in OUTS:
        assert np.isfinite(gpu[n]).all(), f"{label}: non-finite {n}"
    return errs
