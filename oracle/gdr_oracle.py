"""Float64 CPU oracle for the gated delta rule forward pass and its VJP.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP kernels and is deliberately plain and slow.

What it computes (mlx issue #4614 "mx.fast.gated_delta_update VJP: wrong
gradient w.r.t. g", the recurrence statement under the accuracy table and the
``recurrence()`` helper of the repro script): for every batch row b and value
head h, reading kv head h // (Hv/Hk) (a block "repeat" mapping, not a tile),
with the state S of shape [Dv, Dk] and S = S0 (zeros when absent):

    for t = 0 .. T-1:
        S   <- g_t * S                      (decay)
        u_t  = S k_t                        (read on the decayed state)
        e_t  = v_t - u_t
        S   <- S + outer(beta_t * e_t, k_t) (rank-1 delta update)
        y_t  = S q_t                        (read-out on the updated state)

The backward is the reverse-mode derivative of exactly that loop, written out
by hand (the pages give no formulas; the derivation follows the chain rule
step by step, in the same order as the forward).  With G = dL/dS flowing
backwards from dS_T (zeros when absent), for t = T-1 .. 0:

    G     += outer(dy_t, q_t)               (y_t = S_t q_t)
    dq_t   = S_t^T dy_t                     (per value head, summed per kv head)
    c      = G k_t
    dv_t   = beta_t c
    dbeta_t= e_t . c
    dk_t   = G^T (beta_t e_t) - beta_t A_t^T c          (A_t = g_t S_{t-1})
    dA     = G - beta_t outer(c, k_t)
    dg_t   = <dA, S_{t-1}>_F
    G      = g_t dA
    dS0    = G (after the loop)

dq and dk of the value heads that share a kv head are summed in ascending
head order.  Float64 throughout; inputs are promoted to float64.

Log-decay input (``log_decay=True``): the g argument holds lg = log of the
decay, as in the repro script of mlx issue #4614, which draws log g and
takes g = exp(log g), and as the issue's note on training the decay through
its log (A_log/dt_bias) requires.  The forward uses g = exp(lg); the
backward returns dL/dlg = g * dL/dg (chain rule through the exponential) in
place of dL/dg.

Step mask (``mask``, [B, T], nonzero = valid): the pages name a mask argument
of gated_delta_update (mlx-lm PR #1217, "What this PR adds") without defining
it.  The reading taken: a step with mask 0 is an identity step.  The state is
left as it was (no decay, no update); y_t is still the read-out of that
state; g_t, beta_t, v_t and k_t do not enter, so their gradients at that step
are 0, while q_t and dy_t still meet through the read-out.

Pins: tests/test_oracle.py checks this module against central finite
differences, hand-expanded closed forms for T=1 and T=2, the delta-rule
invariant, the g=1/beta=0 identity case, linearity, the adjoint identity,
batch-row independence and the GQA/repeat equivalence.
"""
from __future__ import annotations

import numpy as np

__all__ = ["forward", "backward", "rel_l2", "head_map"]


def head_map(Hk: int, Hv: int) -> np.ndarray:
    """kv head read by each value head: h // (Hv/Hk) (repeat, not tile)."""
    if Hk <= 0 or Hv % Hk:
        raise ValueError("Hv must be a positive multiple of Hk")
    return np.arange(Hv) // (Hv // Hk)


def _f64(x):
    """Promote to float64 (complex128 stays complex, which lets the tests
    take complex-step derivatives of the same code)."""
    if x is None:
        return None
    x = np.asarray(x)
    return x.astype(np.result_type(x.dtype, np.float64), copy=False)


def forward(q, k, v, g, beta, S0=None, keep_states=False, log_decay=False, mask=None):
    """Run the recurrence.

    q, k: [B,T,Hk,Dk]; v: [B,T,Hv,Dv]; g, beta: [B,T,Hv]; S0: [B,Hv,Dv,Dk]
    or None (zeros).  Returns (y [B,T,Hv,Dv], S_T [B,Hv,Dv,Dk]) and, when
    keep_states, also the list of T+1 states S_0 .. S_T (each [B,Hv,Dv,Dk]).
    With log_decay, g holds log of the decay.  mask [B,T]: 0 marks an
    identity step.
    """
    q, k, v, g, beta, S0 = map(_f64, (q, k, v, g, beta, S0))
    if log_decay:
        g = np.exp(g)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    kv = head_map(Hk, Hv)
    dt = np.result_type(q, k, v, g, beta, *(() if S0 is None else (S0,)))
    S = np.zeros((B, Hv, Dv, Dk), dt) if S0 is None else S0.astype(dt)
    y = np.empty((B, T, Hv, Dv), dt)
    states = [S.copy()] if keep_states else None
    for t in range(T):
        kt = k[:, t, kv, :]                      # [B,Hv,Dk]
        qt = q[:, t, kv, :]
        S_before = S
        S = g[:, t, :, None, None] * S           # decay
        u = np.einsum("bhij,bhj->bhi", S, kt)    # S k_t on the decayed state
        e = v[:, t] - u
        d = beta[:, t, :, None] * e
        S = S + d[..., :, None] * kt[..., None, :]
        if mask is not None:                     # identity steps keep the state
            keep = np.asarray(mask)[:, t] != 0
            S = np.where(keep[:, None, None, None], S, S_before)
        y[:, t] = np.einsum("bhij,bhj->bhi", S, qt)
        if keep_states:
            states.append(S.copy())
    if keep_states:
        return y, S, states
    return y, S


def backward(q, k, v, g, beta, dy, S0=None, dST=None, log_decay=False, mask=None):
    """Gradients of L = <dy, y> + <dST, S_T> with respect to every input.

    Returns (dq, dk, dv, dg, dbeta, dS0) with the shapes of (q, k, v, g,
    beta, S0-or-state).  dq/dk are summed over the value heads of each kv
    head in ascending order.  With log_decay, g holds log of the decay and
    the returned dg is the gradient with respect to that log.  mask: as in
    forward.
    """
    q, k, v, g, beta, dy, S0, dST = map(_f64, (q, k, v, g, beta, dy, S0, dST))
    if log_decay:
        g = np.exp(g)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    kv = head_map(Hk, Hv)
    rep = Hv // Hk
    _, _, states = forward(q, k, v, g, beta, S0, keep_states=True, mask=mask)
    keep_all = (np.ones((B, T), bool) if mask is None else np.asarray(mask) != 0)

    dq_h = np.zeros((B, T, Hv, Dk))
    dk_h = np.zeros((B, T, Hv, Dk))
    dv = np.zeros((B, T, Hv, Dv))
    dg = np.zeros((B, T, Hv))
    dbeta = np.zeros((B, T, Hv))
    G = np.zeros((B, Hv, Dv, Dk)) if dST is None else dST.copy()
    for t in range(T - 1, -1, -1):
        kt = k[:, t, kv, :]
        qt = q[:, t, kv, :]
        gt = g[:, t, :, None, None]
        bt = beta[:, t, :, None]
        S_prev = states[t]                       # state before step t
        S_cur = states[t + 1]                    # state after step t
        A = gt * S_prev                          # decayed state
        u = np.einsum("bhij,bhj->bhi", A, kt)
        e = v[:, t] - u
        d = bt * e
        # y_t = S_t q_t
        G = G + dy[:, t][..., :, None] * qt[..., None, :]
        dq_h[:, t] = np.einsum("bhij,bhi->bhj", S_cur, dy[:, t])
        keep = keep_all[:, t]
        if not keep.any():                       # identity step in every row
            continue
        # S_t = A + outer(d, k)
        c = np.einsum("bhij,bhj->bhi", G, kt)    # G k
        dd = c                                    # dL/dd
        dk_h[:, t] = np.einsum("bhij,bhi->bhj", G, d)
        # d = beta * e, e = v - A k
        dv[:, t] = bt * dd
        dbeta[:, t] = np.einsum("bhi,bhi->bh", e, dd)
        de_u = -bt * dd                          # dL/du
        dk_h[:, t] += np.einsum("bhij,bhi->bhj", A, de_u)
        dA = G + de_u[..., :, None] * kt[..., None, :]
        # A = g S_prev
        dg[:, t] = np.einsum("bhij,bhij->bh", dA, S_prev)
        G_prev = gt * dA
        if not keep.all():                       # identity steps: nothing enters
            kb = keep[:, None]
            dk_h[:, t] = np.where(kb[..., None], dk_h[:, t], 0.0)
            dv[:, t] = np.where(kb[..., None], dv[:, t], 0.0)
            dbeta[:, t] = np.where(kb, dbeta[:, t], 0.0)
            dg[:, t] = np.where(kb, dg[:, t], 0.0)
            G_prev = np.where(kb[..., None, None], G_prev, G)
        G = G_prev
    dq = np.zeros((B, T, Hk, Dk))
    dk = np.zeros((B, T, Hk, Dk))
    for h in range(Hv):                          # ascending value-head order
        dq[:, :, h // rep] += dq_h[:, :, h]
        dk[:, :, h // rep] += dk_h[:, :, h]
    if log_decay:
        dg = g * dg                              # d g / d log g = g
    return dq, dk, dv, dg, dbeta, G


def rel_l2(a, b) -> float:
    """Relative L2 error of the flattened tensors in float64:
    ||a - b|| / max(||b||, 1e-300) (mlx issue #4614, ``rel()`` of the
    repro script)."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
