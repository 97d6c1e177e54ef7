"""CPU oracle of the projections around the Key-Value Means layer.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package.  The HIP library never uses it.

[KVM abstract]: KVM is an attention layer, so a block feeds it queries, keys and
values projected from the token representations and projects its output back;
[KVM summary, Core mechanisms 2]: the merge gate is a data-dependent scalar, so
its logit is one more projection of the same input, one per head.
(reading) Plain linear maps without bias for q, k, v and the output, an
optional per-head bias on the gate logit (it sets the gate's resting value);
weights stored as [out features, in features]; the features of q, k and v are
head-major (feature h * 64 + d is dimension d of head h), the sequence index of
head h of batch b is b * H + h, as in the layer's own tensors.

Plain NumPy float64: the contraction is a matrix product.
"""
from __future__ import annotations

import numpy as np


def project_in(x, w_in, b_gate, heads: int, head_dim: int = 64):
    """x [B, N, D] (D = heads * head_dim), w_in [3D + heads, D], b_gate [heads] or None.

    Returns q, k, v [B * heads, N, head_dim] and gate logits [B * heads, N]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_in, dtype=np.float64)
    B, N, D = x.shape
    H = heads
    assert D == H * head_dim and w.shape == (3 * D + H, D)
    y = x.reshape(B * N, D) @ w.T                       # [B*N, 3D + H]
    def heads_of(block):                                 # [B*N, D] -> [B*H, N, hd]
        return block.reshape(B, N, H, head_dim).transpose(0, 2, 1, 3).reshape(B * H, N, head_dim)
    q = heads_of(y[:, :D])
    k = heads_of(y[:, D:2 * D])
    v = heads_of(y[:, 2 * D:3 * D])
    g = y[:, 3 * D:]                                     # [B*N, H]
    if b_gate is not None:
        g = g + np.asarray(b_gate, dtype=np.float64)[None, :]
    gl = g.reshape(B, N, H).transpose(0, 2, 1).reshape(B * H, N)
    return q, k, v, gl


def project_out(o, w_out, batch: int, head_dim: int = 64):
    """o [B * H, N, head_dim] (the layer's output), w_out [D, D] -> y [B, N, D]."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w_out, dtype=np.float64)
    BH, N, hd = o.shape
    H = BH // batch
    D = H * hd
    assert w.shape == (D, D)
    x = o.reshape(batch, H, N, hd).transpose(0, 2, 1, 3).reshape(batch * N, D)
    return (x @ w.T).reshape(batch, N, D)
