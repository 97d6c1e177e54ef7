"""Seeded synthetic workloads for the Key-Value Means (KVM) attention layer.

This module only draws inputs: shapes, value distributions and structure
(Gaussian key clusters, planted isolated keys, log-normal value norms).  It
holds none of the layer's arithmetic, so the CPU oracle and the HIP path can
both be fed from it without sharing any computation.

The pages describe 120M/350M-parameter models trained at 8k context
("Experimental results" of the technical summary) but print no activations;
the draws below stand in for those activations.  Every sequence (b, h) has
its own counter-free NumPy stream seeded by (1000 + workload index, b*H + h),
so any subset of sequences can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["LayerConfig", "WORKLOADS", "make_inputs", "make_sequence", "Inputs"]


@dataclass(frozen=True)
class LayerConfig:
    """One KVM layer workload: shapes, schedule and generator recipe."""

    name: str
    batch: int
    heads: int
    n_tokens: int
    chunk: int
    window: int
    n_sinks: int
    sched: str                 # "fixed" | "sqrt" | "saturating" | "power"
    max_slots: int = 0         # fixed / saturating ceiling
    alpha: int = 0             # sqrt / saturating: capacity = ceil(alpha * sqrt(T))
    dtype: str = "bf16"        # "f32" | "bf16"
    head_dim: int = 64
    rope_dims: int = 32
    rope_theta: float = 10000.0
    ln_eps: float = 1e-5
    softmax_scale: float = 0.0  # logit scale, 0 = 1/sqrt(head_dim)
    exponent: float = 0.5      # power: capacity = ceil(alpha * T**exponent)
    value_norm: bool = True    # layer variants (False = the ablation without it)
    sink_protect: bool = True
    merge_gate: bool = True
    # generator recipe
    key_gen: str = "normal"    # "normal" | "clustered"
    n_clusters: int = 0
    cluster_noise_norm: float = 0.3
    planted: int = 0           # planted isolated unit keys per sequence
    planted_first_chunk: int = 64
    planted_max_per_chunk: int = 2
    value_gen: str = "normal"  # "normal" | "lognormal_norm"
    decode_steps: int = 0      # extra tokens drawn after n_tokens for decode
    seed_base: int = 1000
    index: int = 0

    @property
    def seqs(self) -> int:
        return self.batch * self.heads

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


WORKLOADS = [
    # Tiny fp32 layer, fixed 32-slot state incl. 4 sinks.
    LayerConfig(name="tiny_f32_fixed32", batch=1, heads=1, n_tokens=1024, chunk=64, window=128,
                n_sinks=4, sched="fixed", max_slots=32, dtype="f32", key_gen="normal", index=0),
    # 120M-shaped layer, fixed 256-slot state.
    LayerConfig(name="120m_fixed256_n8192", batch=4, heads=12, n_tokens=8192, chunk=128, window=256,
                n_sinks=4, sched="fixed", max_slots=256, dtype="bf16", key_gen="clustered",
                n_clusters=512, index=1),
    # 350M-shaped layer, sqrt-growing state, planted isolated keys.
    LayerConfig(name="350m_sqrt8_n32768", batch=2, heads=16, n_tokens=32768, chunk=128, window=256,
                n_sinks=4, sched="sqrt", alpha=8, dtype="bf16", key_gen="clustered",
                n_clusters=512, planted=256, index=2),
    # Long extrapolation prefill, saturating schedule.
    LayerConfig(name="long_sat4096_n131072", batch=1, heads=16, n_tokens=131072, chunk=256, window=512,
                n_sinks=8, sched="saturating", alpha=16, max_slots=4096, dtype="bf16",
                key_gen="clustered", n_clusters=2048, value_gen="lognormal_norm", index=3),
    # Batched decode: sqrt-schedule prefill of 16384 tokens, then single-token steps.
    LayerConfig(name="decode_b64_sqrt8_n16384", batch=64, heads=16, n_tokens=16384, chunk=128,
                window=256, n_sinks=4, sched="sqrt", alpha=8, dtype="bf16", key_gen="clustered",
                n_clusters=512, planted=64, planted_max_per_chunk=1, decode_steps=512, index=4),
]


@dataclass
class Inputs:
    """Inputs for a set of sequences, already rounded to the workload dtype.

    q, k, v: [S, T, 64] torch tensors in the workload dtype (CPU)
    gate_logits: [S, T] float32
    planted_pos: per sequence, the positions of planted keys (may be empty)
    T = n_tokens + decode_steps.
    """

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gate_logits: torch.Tensor
    planted_pos: list = field(default_factory=list)


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_sequence(cfg: LayerConfig, seq: int, n_total: Optional[int] = None):
    """Draw one sequence (q, k, v, gate logits, planted positions) as float32 numpy.

    Draw order: q, v, gate logits, cluster centres, cluster ids, key noise,
    planted positions, planted directions.
    """
    T = cfg.n_tokens + cfg.decode_steps if n_total is None else n_total
    d = cfg.head_dim
    rng = np.random.default_rng((cfg.seed_base + cfg.index, seq))
    q = rng.standard_normal((T, d), dtype=np.float32)
    if cfg.value_gen == "normal":
        v = rng.standard_normal((T, d), dtype=np.float32)
    elif cfg.value_gen == "lognormal_norm":
        dirs = rng.standard_normal((T, d), dtype=np.float32)
        dirs /= np.maximum(np.linalg.norm(dirs, axis=1, keepdims=True), 1e-30)
        norms = rng.lognormal(0.0, 0.5, size=(T, 1)).astype(np.float32)
        v = dirs * norms
    else:
        raise ValueError(cfg.value_gen)
    gl = rng.standard_normal(T, dtype=np.float32)
    planted_pos = np.zeros(0, dtype=np.int64)
    if cfg.key_gen == "normal":
        k = rng.standard_normal((T, d), dtype=np.float32)
    elif cfg.key_gen == "clustered":
        centres = rng.standard_normal((cfg.n_clusters, d))
        centres /= np.linalg.norm(centres, axis=1, keepdims=True)
        ids = rng.integers(0, cfg.n_clusters, size=T)
        # noise whose expected norm is cluster_noise_norm: per-coordinate std = norm / sqrt(d)
        noise = rng.standard_normal((T, d), dtype=np.float32) * np.float32(cfg.cluster_noise_norm / np.sqrt(d))
        k = (centres[ids].astype(np.float32) + noise).astype(np.float32)
        if cfg.planted > 0:
            planted_pos = _planted_positions(cfg, rng, T)
            pdirs = rng.standard_normal((len(planted_pos), d))
            pdirs /= np.linalg.norm(pdirs, axis=1, keepdims=True)
            k[planted_pos] = pdirs.astype(np.float32)
    else:
        raise ValueError(cfg.key_gen)
    return q, k, v, gl, planted_pos


def _planted_positions(cfg: LayerConfig, rng, T: int) -> np.ndarray:
    """Distinct positions in absorbed chunks [planted_first_chunk, last absorbed chunk],
    at most planted_max_per_chunk per chunk."""
    C, W = cfg.chunk, cfg.window
    n_chunks = -(-T // C)
    last_absorbed = n_chunks - 1 - W // C - 1   # last chunk absorbed by the final query chunk
    first = cfg.planted_first_chunk
    chunks = np.arange(first, last_absorbed + 1)
    if len(chunks) == 0:
        return np.zeros(0, dtype=np.int64)
    slots = np.repeat(chunks, cfg.planted_max_per_chunk)
    n = min(cfg.planted, len(slots))
    pick = np.sort(rng.choice(len(slots), size=n, replace=False))
    chosen = slots[pick]
    pos = []
    for c in np.unique(chosen):
        cnt = int(np.sum(chosen == c))
        offs = np.sort(rng.choice(C, size=cnt, replace=False))
        pos.extend(int(c) * C + int(o) for o in offs)
    return np.asarray(sorted(pos), dtype=np.int64)


def make_inputs(cfg: LayerConfig, seqs=None, n_total: Optional[int] = None) -> Inputs:
    """Draw the listed sequences (default: all B*H) and round them to the workload dtype."""
    if seqs is None:
        seqs = range(cfg.seqs)
    seqs = list(seqs)
    dt = _torch_dtype(cfg.dtype)
    qs, ks, vs, gs, pp = [], [], [], [], []
    for s in seqs:
        q, k, v, gl, pos = make_sequence(cfg, s, n_total)
        qs.append(torch.from_numpy(q).to(dt))
        ks.append(torch.from_numpy(k).to(dt))
        vs.append(torch.from_numpy(v).to(dt))
        gs.append(torch.from_numpy(gl))
        pp.append(pos)
    return Inputs(q=torch.stack(qs), k=torch.stack(ks), v=torch.stack(vs),
                  gate_logits=torch.stack(gs), planted_pos=pp)
