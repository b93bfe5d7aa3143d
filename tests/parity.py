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


def row_errors(a, b, floor_frac=0.1):
    """Relative L2 error of every row (the last axis) of a against b.

    A row's error is ||a_row - b_row|| / max(||b_row||, floor), with the floor
    a fraction of the tensor's RMS row norm, so that rows whose reference is
    (near) zero are held to an absolute bound on the tensor's own scale.
    Rows are (batch row, step, head) for y, dv, dq, dk, (batch row, head,
    state row) for S_T, dS0, and (batch row, step) over the value heads for
    dg, dbeta: one corrupted (step, head) entry shows up in its own row.
    """
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return np.zeros(0)
    n = b.shape[-1]
    a2, b2 = a.reshape(-1, n), b.reshape(-1, n)
    rn = np.linalg.norm(b2, axis=1)
    floor = floor_frac * float(np.sqrt(np.mean(rn ** 2)))
    return np.linalg.norm(a2 - b2, axis=1) / np.maximum(rn, max(floor, 1e-300))


def row_tol_for(tol):
    """Per-row bar that goes with a whole-tensor bar: 2e-2 for the bf16 bar
    (output rounding alone puts a row near 2^-9 relative), 100 times the bar
    otherwise."""
    return 2e-2 if tol >= 1e-3 else 100.0 * tol


def compare(gpu, ref, tol, label="", row_tol=None, names=OUTS):
    """Every output within `tol` relative L2 over the whole tensor and within
    `row_tol` on every row (row_errors), and finite."""
    row_tol = row_tol_for(tol) if row_tol is None else row_tol
    errs = {n: O.rel_l2(gpu[n], ref[n]) for n in names}
    rows = {n: float(row_errors(gpu[n], ref[n]).max(initial=0.0)) for n in names}
    log(f"  {label} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items())
        + " | max row " + " ".join(f"{n}={rows[n]:.1e}" for n in names))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{label}: rel L2 above {tol}: {bad}"
    bad = {n: e for n, e in rows.items() if not e <= row_tol}
    assert not bad, f"{label}: a row's rel L2 above {row_tol}: {bad}"
    for n in names:
        assert np.isfinite(gpu[n]).all(), f"{label}: non-finite {n}"
    return errs


def compare_groups(gpu, p, tol, label="", units=None, state_tol=None):
    """Compare every (batch row, kv group) unit of `units` (default: all of
    them) with the oracle run on that unit alone, one after another (the
    units are independent, so this is the whole-problem comparison split
    into pieces the oracle finishes quickly).  state_tol, if given, is the
    bar for the fp32 outputs S_T and dS0.  Returns the worst error per
    output."""
    units = units or [(b, hk) for b in range(p.B) for hk in range(p.Hk)]
    worst = {n: 0.0 for n in OUTS}
    for b, hk in units:
        errs = compare(slice_group(gpu, p, b, hk), run_oracle(p, b, hk), tol,
                       f"{label} b{b} kv{hk}")
        for n in OUTS:
            worst[n] = max(worst[n], errs[n])
        if state_tol is not None:
            for n in ("S_T", "dS0"):
                assert errs[n] <= state_tol, f"{label} b{b} kv{hk}: {n} {errs[n]:.2e}"
    return worst
