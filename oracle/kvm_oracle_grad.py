"""CPU oracle of the Key-Value Means layer's backward pass.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package.  The HIP library never uses it.

What is differentiated.  [KVM abstract]: the layer supports chunk-wise
parallelizable training, so the gradient of a loss with respect to the layer's
inputs (q, k, v and the gate logits) is part of the method.  The forward is
kvm_oracle.prefill.  Its discrete choices, the winner-take-all row of each
merged token and the set of appended (most surprising) tokens ([KVM summary,
Core mechanisms 2-3]), are piecewise constant in the inputs; (reading) they are
held fixed, as the decisions the forward took, and the gradient flows through
everything else:

  - the one softmax over [state || window] ([KVM summary, Methodology]),
  - RoPE on the window path ([KVM summary, Core mechanisms 4]),
  - the just-in-time read form: LayerNorm of K/n and the value rho * V/|V|
    ([KVM summary, Core mechanisms 2]; the plain mean V/n without value-length
    normalisation),
  - the gated raw sums [KVM lay summary, "smart merge"] and the radius of a
    row, the norm of its creating value,
  - the gate sigmoid(l).

Counts are integers and carry no gradient.  Plain NumPy float64, step by step:
recompute the forward, back through the attention of every query chunk, back
through the read form of every snapshot, then back through the chunk
recurrence from the last absorbed chunk to the first.

Public entry point: prefill_grad.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from oracle import kvm_oracle as O


@dataclass
class GradResult:
    dq: np.ndarray        # [N, 64]
    dk: np.ndarray        # [N, 64]
    dv: np.ndarray        # [N, 64]
    dl: np.ndarray        # [N] gate logits
    fwd: O.SeqResult      # the forward it differentiates (decisions, snapshots, output)


def rope_transpose(dy, pos, rope_dims: int = 32, theta: float = 10000.0):
    """Transpose of RoPE at `pos` applied to a gradient: the rotation by the opposite angle."""
    return O.rope(dy, -np.asarray(pos, dtype=np.float64), rope_dims, theta)


def read_form_grad(K, V, n, rho, dkhat_live, dvhat, p: O.Params):
    """Back through the read form of one snapshot.

    Forward ([KVM summary, Core mechanisms 2]; readings of kvm_oracle.read_form):
    x = K/n, khat_live = (x - mean x) / sqrt(var x + eps) over the live dims,
    vhat = rho V/|V| (0 if |V| = 0), or V/n without value-length normalisation.
    Returns dK [S, dk], dV [S, dv], drho [S]."""
    x = K / n[:, None]
    d = x.shape[1]
    mu = x.mean(axis=1, keepdims=True)
    xc = x - mu
    var = (xc ** 2).mean(axis=1, keepdims=True)
    inv = 1.0 / np.sqrt(var + p.ln_eps)
    xhat = xc * inv
    g = dkhat_live
    # LayerNorm (no affine): dx = inv * (g - mean(g) - xhat * mean(g * xhat))
    dx = inv * (g - g.mean(axis=1, keepdims=True) - xhat * (g * xhat).mean(axis=1, keepdims=True))
    dK = dx / n[:, None]
    assert dK.shape[1] == d
    if not p.value_norm:
        return dK, dvhat / n[:, None], np.zeros(len(n))
    nv = np.linalg.norm(V, axis=1)
    dV = np.zeros_like(V)
    drho = np.zeros(len(n))
    ok = nv > 0
    u = V[ok] / nv[ok, None]
    gv = dvhat[ok]
    # vhat = rho * u, u = V/|V|:  d(rho) = u.g ;  dV = rho/|V| * (g - u (u.g))
    ug = np.sum(u * gv, axis=1)
    drho[ok] = ug
    dV[ok] = (rho[ok] / nv[ok])[:, None] * (gv - u * ug[:, None])
    return dK, dV, drho


def prefill_grad(q, k, v, ell, d_out, p: O.Params, forced: Optional[dict] = None) -> GradResult:
    """Gradient of sum(d_out * out) with respect to q, k, v and the gate logits, where out is
    kvm_oracle.prefill(q, k, v, ell, p, forced) and its decisions are held fixed."""
    q, k, v, ell, d_out = (np.asarray(a, dtype=np.float64) for a in (q, k, v, ell, d_out))
    N, d = q.shape
    C, W, dr = p.chunk, p.window, p.rope_dims
    fwd = O.prefill(q, k, v, ell, p, forced=forced, keep_snapshots=True)
    pos = np.arange(N)
    qr = O.rope(q, pos, dr, p.rope_theta)
    kr = O.rope(k, pos, dr, p.rope_theta)
    ktil = k[:, dr:]
    g = O.merge_weights(ell, p)
    s = O.logit_scale(p)

    dq = np.zeros((N, d))            # unrotated query (state logits)
    dqr = np.zeros((N, d))           # rotated query (window logits)
    dkr = np.zeros((N, d))           # rotated keys
    dv = np.zeros((N, v.shape[1]))
    n_snap = len(fwd.rows_after)
    dkhat = [None] * n_snap          # per snapshot: gradient of its read-form keys (live dims)
    dvhat = [None] * n_snap

    # ---- 1. back through the attention of every query chunk ([KVM summary, Methodology])
    for c in range(-(-N // C)):
        j = c - W // C - 1           # the snapshot chunk c reads (none if j < 0)
        if j >= 0:
            khat, vhat = O.read_form(fwd.snapshots[j], p)
        else:
            khat, vhat = np.zeros((0, d)), np.zeros((0, v.shape[1]))
        rows = np.arange(c * C, min(N, (c + 1) * C))
        lo = max(0, c * C - W)
        keys = np.arange(lo, rows[-1] + 1)
        Ls = s * (q[rows] @ khat.T)
        Lw = s * (qr[rows] @ kr[keys].T)
        Lw = np.where(keys[None, :] <= rows[:, None], Lw, -np.inf)
        L = np.hstack([Ls, Lw])
        L = L - L.max(axis=1, keepdims=True)
        P = np.exp(L)
        P /= P.sum(axis=1, keepdims=True)
        ns = khat.shape[0]
        Vall = np.vstack([vhat, v[keys]])
        dO = d_out[rows]
        dP = dO @ Vall.T                                   # [r, ns + w]
        dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
        # state part: logits s q.khat (unrotated q)
        dq[rows] += s * (dS[:, :ns] @ khat)
        # window part: logits s qr.kr
        dqr[rows] += s * (dS[:, ns:] @ kr[keys])
        dkr[keys] += s * (dS[:, ns:].T @ qr[rows])
        dv[keys] += P[:, ns:].T @ dO
        if j >= 0:
            dk_snap = s * (dS[:, :ns].T @ q[rows])           # [ns, d]; rotary dims of khat are constant 0
            dv_snap = P[:, :ns].T @ dO
            dkhat[j] = dk_snap[:, dr:] if dkhat[j] is None else dkhat[j] + dk_snap[:, dr:]
            dvhat[j] = dv_snap if dvhat[j] is None else dvhat[j] + dv_snap

    # ---- 2. back through the read form of every snapshot, then 3. through the
    # chunk recurrence, last absorbed chunk first: the gradient of row i's sums
    # after chunk j is the sum of the read-form gradients of every snapshot
    # j' >= j that holds row i ([KVM lay summary, "smart merge"]: the sums only grow)
    S_cap = fwd.state.rows
    dKt = np.zeros((S_cap, d - dr))
    dVt = np.zeros((S_cap, v.shape[1]))
    drt = np.zeros(S_cap)
    dktil = np.zeros((N, d - dr))
    dg = np.zeros(N)
    for j in range(n_snap - 1, -1, -1):
        snap = fwd.snapshots[j]
        S = snap.rows
        if dkhat[j] is not None:
            K, V, n, rho, _ = snap.arrays()
            dK, dV, drho = read_form_grad(K, V, n.astype(np.float64), rho, dkhat[j], dvhat[j], p)
            dKt[:S] += dK
            dVt[:S] += dV
            drt[:S] += drho
        # the tokens of chunk j: merged ones took g_t * (k_t, v_t) into their row; creators set it
        for t in range(j * C, (j + 1) * C):
            i = int(fwd.slot[t])
            kind = int(fwd.kind[t])
            if kind == O.KIND_MERGE:
                dktil[t] += g[t] * dKt[i]
                dv[t] += g[t] * dVt[i]
                dg[t] += ktil[t] @ dKt[i] + v[t] @ dVt[i]
        for t in range(j * C, (j + 1) * C):
            i = int(fwd.slot[t])
            if int(fwd.kind[t]) in (O.KIND_SINK, O.KIND_APPEND):
                # K_i = ktil_t, V_i = v_t (unscaled), rho_i = |v_t|
                dktil[t] += dKt[i]
                nv = np.linalg.norm(v[t])
                dv[t] += dVt[i] + (drt[i] * v[t] / nv if nv > 0 else 0.0)
                dKt[i] = 0.0
                dVt[i] = 0.0
                drt[i] = 0.0

    # ---- 4. gate and RoPE transposes, assembled per input
    if p.merge_gate:
        gate = O.gate(ell)
        dl = dg * gate * (1.0 - gate)
    else:
        dl = np.zeros(N)
    dq = dq + rope_transpose(dqr, pos, dr, p.rope_theta)
    dk = rope_transpose(dkr, pos, dr, p.rope_theta)
    dk[:, dr:] += dktil
    return GradResult(dq=dq, dk=dk, dv=dv, dl=dl, fwd=fwd)
