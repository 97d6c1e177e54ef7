"""Python binding of the C-ABI library libkvm.so (include/kvm.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory (the workspace and the tensors) and
the current HIP stream.  If libkvm.so is missing, loading fails loudly; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields
from typing import Optional

import torch

__all__ = [
    "KvmConfig", "KvmState", "KvmError", "library", "workspace_bytes", "schedule", "prefill_noalloc", "project_in",
    "project_out", "SCHED", "DTYPE",
    "KVM_OK", "KVM_E_INVALID_ARG", "KVM_E_WORKSPACE", "KVM_E_CAPACITY", "KVM_E_STATE", "KVM_E_HIP",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvm.so")

KVM_OK, KVM_E_INVALID_ARG, KVM_E_WORKSPACE, KVM_E_CAPACITY, KVM_E_STATE, KVM_E_HIP = range(6)
KVM_FLAG_TRACE = 1
KVM_FLAG_NO_VALUE_NORM = 2
KVM_FLAG_NO_SINK_PROTECT = 4
KVM_FLAG_NO_MERGE_GATE = 8
KVM_FLAG_SERIAL_PREFILL = 16
SCHED = {"fixed": 0, "sqrt": 1, "saturating": 2, "power": 3}
DTYPE = {"f32": 0, "bf16": 1}
_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_READ_DTYPE = {"f32": torch.float32, "bf16": torch.float16}   # read-form storage type


class KvmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_dims", ctypes.c_int32), ("chunk", ctypes.c_int32), ("window", ctypes.c_int32),
        ("n_sinks", ctypes.c_int32), ("sched", ctypes.c_int32), ("max_slots", ctypes.c_int32),
        ("alpha", ctypes.c_int32), ("max_tokens", ctypes.c_int64), ("rope_theta", ctypes.c_float),
        ("ln_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("exponent", ctypes.c_double),
    ]


class _View(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in
                 ("n_rows", "key_sum", "val_sum", "count", "rho", "key_read", "val_read", "trace_slot", "trace_kind")]
                + [("position", ctypes.c_int64)]
                + [(n, ctypes.c_void_p) for n in ("ring_k", "ring_v", "ring_l")])


class _Info(ctypes.Structure):
    _fields_ = [("position", ctypes.c_int64), ("absorbed_chunks", ctypes.c_int64), ("rows", ctypes.c_int32),
                ("max_rows", ctypes.c_int32), ("max_chunks", ctypes.c_int64), ("poisoned", ctypes.c_int32),
                ("scan_groups", ctypes.c_int32), ("per_sequence", ctypes.c_int32)]


class _Prof(ctypes.Structure):
    _fields_ = [("scan_ms", ctypes.c_double), ("scan_launches", ctypes.c_int64),
                ("attn_ms", ctypes.c_double), ("attn_launches", ctypes.c_int64),
                ("ring_ms", ctypes.c_double), ("ring_launches", ctypes.c_int64),
                ("dec_absorb_ms", ctypes.c_double), ("dec_absorb_launches", ctypes.c_int64),
                ("dec_attn_ms", ctypes.c_double), ("dec_attn_launches", ctypes.c_int64),
                ("prep_ms", ctypes.c_double), ("prep_launches", ctypes.c_int64)]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libkvm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m compressed_kv_state_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.kvm_workspace_bytes.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_size_t)]
        L.kvm_schedule.argtypes = [ctypes.POINTER(_Config), i64, vp, vp, vp]
        L.kvm_state_create.argtypes = [ctypes.POINTER(_Config), vp, ctypes.c_size_t, vp, ctypes.POINTER(vp)]
        L.kvm_state_destroy.argtypes = [vp]
        L.kvm_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp]
        L.kvm_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.kvm_prefill_noalloc.argtypes = [ctypes.POINTER(_Config), vp, vp, vp, vp, vp, i64, vp]
        L.kvm_prefill_ragged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, vp]
        L.kvm_decode_step_ragged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.kvm_state_reset_sequence.argtypes = [vp, ctypes.c_int32, vp]
        L.kvm_state_positions.argtypes = [vp, vp]
        L.kvm_project_in.argtypes = [ctypes.POINTER(_Config), vp, vp, vp, vp, vp, vp, vp, i64, vp]
        L.kvm_project_out.argtypes = [ctypes.POINTER(_Config), vp, vp, vp, i64, vp]
        L.kvm_backward_workspace_bytes.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_size_t)]
        L.kvm_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.kvm_state_read.argtypes = [vp, i64, ctypes.POINTER(_View), vp]
        L.kvm_state_load.argtypes = [vp, ctypes.POINTER(_View), vp]
        L.kvm_snapshot_read.argtypes = [vp, i64, vp, vp, vp, vp]
        L.kvm_state_get_info.argtypes = [vp, ctypes.POINTER(_Info)]
        L.kvm_state_reset.argtypes = [vp, vp]
        L.kvm_state_check.argtypes = [vp, vp]
        L.kvm_profile_enable.argtypes = [vp, st]
        L.kvm_profile_read.argtypes = [vp, ctypes.POINTER(_Prof)]
        L.kvm_status_str.argtypes = [st]
        L.kvm_status_str.restype = ctypes.c_char_p
        L.kvm_last_error.argtypes = []
        L.kvm_last_error.restype = ctypes.c_char_p
        for name in ("kvm_workspace_bytes", "kvm_schedule", "kvm_state_create", "kvm_state_destroy", "kvm_prefill",
                     "kvm_prefill_noalloc", "kvm_backward_workspace_bytes", "kvm_prefill_backward",
                     "kvm_project_in", "kvm_project_out", "kvm_prefill_ragged", "kvm_decode_step_ragged",
                     "kvm_state_reset_sequence", "kvm_state_positions",
                     "kvm_decode_step", "kvm_state_read", "kvm_state_load", "kvm_snapshot_read", "kvm_state_get_info",
                     "kvm_state_reset", "kvm_state_check", "kvm_profile_enable", "kvm_profile_read"):
            getattr(L, name).restype = st
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return library().kvm_status_str(s).decode()
    except Exception:
        return f"status {s}"


def _check(status: int):
    if status != KVM_OK:
        raise KvmError(status, library().kvm_last_error().decode())


@dataclass
class KvmConfig:
    """Mirror of kvm_config.  sched: 'fixed' | 'sqrt' | 'saturating' | 'power'; dtype: 'f32' | 'bf16'.
    value_norm / sink_protect / merge_gate False select the ablation variants (flag bits)."""

    batch: int
    heads: int
    chunk: int
    window: int
    n_sinks: int
    sched: str
    max_tokens: int
    max_slots: int = 0
    alpha: int = 0
    dtype: str = "bf16"
    head_dim: int = 64
    rope_dims: int = 32
    rope_theta: float = 10000.0
    ln_eps: float = 1e-5
    softmax_scale: float = 0.0
    trace: bool = False
    exponent: float = 0.5
    value_norm: bool = True
    sink_protect: bool = True
    merge_gate: bool = True
    serial_prefill: bool = False

    @property
    def seqs(self) -> int:
        return self.batch * self.heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    @property
    def read_dtype(self) -> torch.dtype:
        """Storage type of the state's read-form keys (fp16 on the bf16 path); read-form
        values use the input dtype."""
        return _READ_DTYPE[self.dtype]

    @staticmethod
    def of(obj, max_tokens: int, trace: bool = False) -> "KvmConfig":
        """From any object with the same attribute names (e.g. a workload description)."""
        names = {f.name for f in fields(KvmConfig)} - {"max_tokens", "trace"}
        kw = {n: getattr(obj, n) for n in names if hasattr(obj, n)}
        return KvmConfig(max_tokens=max_tokens, trace=trace, **kw)

    def to_c(self) -> _Config:
        if self.sched not in SCHED:
            raise ValueError(f"unknown schedule {self.sched!r}")
        if self.dtype not in DTYPE:
            raise ValueError(f"unknown dtype {self.dtype!r}")
        flags = ((KVM_FLAG_TRACE if self.trace else 0) | (0 if self.value_norm else KVM_FLAG_NO_VALUE_NORM)
                 | (0 if self.sink_protect else KVM_FLAG_NO_SINK_PROTECT)
                 | (0 if self.merge_gate else KVM_FLAG_NO_MERGE_GATE)
                 | (KVM_FLAG_SERIAL_PREFILL if self.serial_prefill else 0))
        return _Config(self.batch, self.heads, self.head_dim, self.rope_dims, self.chunk, self.window,
                       self.n_sinks, SCHED[self.sched], self.max_slots, self.alpha, self.max_tokens,
                       self.rope_theta, self.ln_eps, self.softmax_scale, DTYPE[self.dtype], flags,
                       float(self.exponent))


def workspace_bytes(cfg: KvmConfig) -> int:
    n = ctypes.c_size_t()
    c = cfg.to_c()
    _check(library().kvm_workspace_bytes(ctypes.byref(c), ctypes.byref(n)))
    return int(n.value)


def schedule(cfg: KvmConfig, n_chunks: int):
    """(sinks, appends, rows_after) per absorbed chunk, as int32 CPU tensors."""
    out = [torch.zeros(n_chunks, dtype=torch.int32) for _ in range(3)]
    c = cfg.to_c()
    _check(library().kvm_schedule(ctypes.byref(c), n_chunks, *(t.data_ptr() for t in out)))
    return tuple(out)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _contig(t, name, dtype, numel, dev):
    if not isinstance(t, torch.Tensor) or t.device != dev or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name}: contiguous {dtype} tensor on {dev} expected")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t


def project_in(cfg: KvmConfig, x, w_in, b_gate=None):
    """kvm_project_in: x [B, n, D] -> (q, k, v [B*H, n, 64] in cfg.dtype, gate_logits [B*H, n] float32);
    w_in [3D + H, D] in cfg.dtype, b_gate [H] float32 or None."""
    n = x.shape[-2]
    dev = x.device
    D, H, S = cfg.heads * 64, cfg.heads, cfg.seqs
    _contig(x, "x", cfg.torch_dtype, cfg.batch * n * D, dev)
    _contig(w_in, "w_in", cfg.torch_dtype, (3 * D + H) * D, dev)
    if b_gate is not None:
        _contig(b_gate, "b_gate", torch.float32, H, dev)
    q, k, v = (torch.empty(S, n, 64, dtype=cfg.torch_dtype, device=dev) for _ in range(3))
    gl = torch.empty(S, n, dtype=torch.float32, device=dev)
    c = cfg.to_c()
    _check(library().kvm_project_in(ctypes.byref(c), x.data_ptr(), w_in.data_ptr(),
                                    b_gate.data_ptr() if b_gate is not None else None, q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), gl.data_ptr(), n, _stream(dev)))
    return q, k, v, gl


def project_out(cfg: KvmConfig, o, w_out):
    """kvm_project_out: o [B*H, n, 64] -> y [B, n, D] with w_out [D, D] (cfg.dtype)."""
    n = o.shape[-2]
    dev = o.device
    D = cfg.heads * 64
    _contig(o, "o", cfg.torch_dtype, cfg.seqs * n * 64, dev)
    _contig(w_out, "w_out", cfg.torch_dtype, D * D, dev)
    y = torch.empty(cfg.batch, n, D, dtype=cfg.torch_dtype, device=dev)
    c = cfg.to_c()
    _check(library().kvm_project_out(ctypes.byref(c), o.data_ptr(), w_out.data_ptr(), y.data_ptr(), n, _stream(dev)))
    return y


def prefill_noalloc(cfg: KvmConfig, q, k, v, gate_logits, out) -> torch.Tensor:
    """kvm_prefill_noalloc: one prefill from an empty state with the workspace in the library's
    static device scratch (no allocation by the library).  q, k, v, out [B*H, n, 64] in cfg.dtype,
    gate_logits [B*H, n] float32, all contiguous on one GPU; `out` is written in place."""
    n = q.shape[-2]
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.device != dev or not t.is_contiguous() or t.dtype != cfg.torch_dtype or t.shape[-1] != cfg.head_dim:
            raise ValueError(f"{name}: contiguous {cfg.torch_dtype} [B*H, n, {cfg.head_dim}] on {dev} expected")
        if t.numel() != cfg.seqs * n * cfg.head_dim:
            raise ValueError(f"{name}: expected {cfg.seqs} x {n} x {cfg.head_dim} elements")
    if (gate_logits.device != dev or not gate_logits.is_contiguous() or gate_logits.dtype != torch.float32
            or gate_logits.numel() != cfg.seqs * n):
        raise ValueError("gate_logits: contiguous float32 [B*H, n] expected")
    c = cfg.to_c()
    _check(library().kvm_prefill_noalloc(ctypes.byref(c), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         gate_logits.data_ptr(), out.data_ptr(), n, _stream(dev)))
    return out


class KvmState:
    """A KVM layer state bound to a torch-allocated device workspace."""

    def __init__(self, cfg: KvmConfig, device: Optional[torch.device] = None):
        self.cfg = cfg
        dev = torch.device(device if device is not None else "cuda")
        if dev.type != "cuda":
            raise ValueError("KvmState needs a GPU device")
        self.device = dev if dev.index is not None else torch.device("cuda", torch.cuda.current_device())
        self._c = cfg.to_c()
        nbytes = workspace_bytes(cfg)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(library().kvm_state_create(ctypes.byref(self._c), self.workspace.data_ptr(), nbytes,
                                          _stream(self.device), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            library().kvm_state_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ checks
    def _seq_tensor(self, x: torch.Tensor, name: str, tail) -> torch.Tensor:
        if not isinstance(x, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if x.device != self.device:
            raise ValueError(f"{name} must be on {self.device}")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        S = self.cfg.seqs
        if x.dim() == len(tail) + 2:
            if x.shape[0] != self.cfg.batch or x.shape[1] != self.cfg.heads:
                raise ValueError(f"{name}: leading dims must be (batch, heads)")
            x = x.reshape(S, *x.shape[2:])
        if x.dim() != len(tail) + 1 or x.shape[0] != S or any(t is not None and a != t for a, t in zip(x.shape[1:], tail)):
            raise ValueError(f"{name}: expected shape [B*H, {', '.join(str(t) for t in tail)}], got {tuple(x.shape)}")
        return x

    def _data(self, x, name, n=None):
        x = self._seq_tensor(x, name, (n, self.cfg.head_dim) if n is not None else (self.cfg.head_dim,))
        if x.dtype != self.cfg.torch_dtype:
            raise TypeError(f"{name} must be {self.cfg.torch_dtype}")
        return x

    def _gate(self, x, n=None):
        x = self._seq_tensor(x, "gate_logits", (n,) if n is not None else ())
        if x.dtype != torch.float32:
            raise TypeError("gate_logits must be float32")
        return x

    # ------------------------------------------------------------------ calls
    def prefill(self, q, k, v, gate_logits, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """kvm_prefill over n tokens: q, k, v [B*H, n, 64] (or [B, H, n, 64]); gate_logits [B*H, n]."""
        n = q.shape[-2]
        q2, k2, v2 = (self._data(t, nm, n) for t, nm in ((q, "q"), (k, "k"), (v, "v")))
        g2 = self._gate(gate_logits, n)
        if out is None:
            out = torch.empty_like(q)
        o2 = self._data(out, "out", n)
        _check(library().kvm_prefill(self._h, q2.data_ptr(), k2.data_ptr(), v2.data_ptr(), g2.data_ptr(),
                                     o2.data_ptr(), n, _stream(self.device)))
        return out

    def decode_step(self, q, k, v, gate_logits, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """kvm_decode_step: q, k, v [B*H, 64]; gate_logits [B*H]."""
        q2, k2, v2 = (self._data(t, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v")))
        g2 = self._gate(gate_logits)
        if out is None:
            out = torch.empty_like(q)
        o2 = self._data(out, "out")
        _check(library().kvm_decode_step(self._h, q2.data_ptr(), k2.data_ptr(), v2.data_ptr(), g2.data_ptr(),
                                         o2.data_ptr(), _stream(self.device)))
        return out

    def backward(self, q, k, v, gate_logits, d_out, workspace: Optional[torch.Tensor] = None):
        """kvm_prefill_backward: gradients of sum(d_out * out) for the prefill this state ran over
        positions [0, n) with these inputs (the state needs trace=True).  Returns float32
        (d_q, d_k, d_v [B*H, n, 64], d_gate [B*H, n]).  `workspace` (uint8, at least
        kvm_backward_workspace_bytes) is allocated here when not given."""
        n = q.shape[-2]
        q2, k2, v2, o2 = (self._data(t, nm, n) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (d_out, "d_out")))
        g2 = self._gate(gate_logits, n)
        S = self.cfg.seqs
        dq, dk, dv = (torch.empty(S, n, self.cfg.head_dim, dtype=torch.float32, device=self.device) for _ in range(3))
        dg = torch.empty(S, n, dtype=torch.float32, device=self.device)
        need = ctypes.c_size_t()
        _check(library().kvm_backward_workspace_bytes(ctypes.byref(self._c), ctypes.byref(need)))
        if workspace is None:
            workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=self.device)
        _check(library().kvm_prefill_backward(self._h, q2.data_ptr(), k2.data_ptr(), v2.data_ptr(), g2.data_ptr(),
                                              o2.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                              dg.data_ptr(), n, workspace.data_ptr(), workspace.numel(),
                                              _stream(self.device)))
        return dq, dk, dv, dg

    def prefill_ragged(self, n_tokens, q, k, v, gate_logits, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """kvm_prefill_ragged: sequence s takes n_tokens[s] tokens at its own position; q, k, v
        [B*H, n_max, 64], gate_logits [B*H, n_max] (rows past n_tokens[s] are ignored); returns out
        of the same shape (rows past n_tokens[s] are left as they were)."""
        n_max = q.shape[-2]
        q2, k2, v2 = (self._data(t, nm, n_max) for t, nm in ((q, "q"), (k, "k"), (v, "v")))
        g2 = self._gate(gate_logits, n_max)
        if out is None:
            out = torch.zeros_like(q)
        o2 = self._data(out, "out", n_max)
        n = torch.as_tensor(list(n_tokens), dtype=torch.int64).contiguous()
        if n.numel() != self.cfg.seqs:
            raise ValueError("n_tokens needs one entry per sequence")
        _check(library().kvm_prefill_ragged(self._h, n.data_ptr(), q2.data_ptr(), k2.data_ptr(), v2.data_ptr(),
                                            g2.data_ptr(), o2.data_ptr(), n_max, _stream(self.device)))
        return out

    def decode_step_ragged(self, active, q, k, v, gate_logits, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """kvm_decode_step_ragged: one step for the sequences with active[s]; q, k, v [B*H, 64]."""
        q2, k2, v2 = (self._data(t, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v")))
        g2 = self._gate(gate_logits)
        if out is None:
            out = torch.zeros_like(q)
        o2 = self._data(out, "out")
        a = torch.as_tensor([1 if x else 0 for x in active], dtype=torch.uint8).contiguous()
        if a.numel() != self.cfg.seqs:
            raise ValueError("active needs one entry per sequence")
        _check(library().kvm_decode_step_ragged(self._h, a.data_ptr(), q2.data_ptr(), k2.data_ptr(), v2.data_ptr(),
                                                g2.data_ptr(), o2.data_ptr(), _stream(self.device)))
        return out

    def reset_sequence(self, s: int):
        """kvm_state_reset_sequence: sequence slot s back to position 0, empty (the others continue)."""
        _check(library().kvm_state_reset_sequence(self._h, int(s), _stream(self.device)))

    def positions(self):
        """Each sequence's position."""
        p = torch.zeros(self.cfg.seqs, dtype=torch.int64)
        _check(library().kvm_state_positions(self._h, p.data_ptr()))
        return p.tolist()

    def reset(self):
        """Back to position 0 with an empty state (queued on the current stream)."""
        _check(library().kvm_state_reset(self._h, _stream(self.device)))

    def check(self):
        """Raise KvmError if an absorption scan gave up at a cross-workgroup exchange
        (synchronises the current stream)."""
        _check(library().kvm_state_check(self._h, _stream(self.device)))

    def profile(self, enable=True):
        """Record HIP events around later kernel launches: True = every phase, False = none,
        or a mask of KVM_PROFILE_* phase bits."""
        mask = enable if isinstance(enable, int) and not isinstance(enable, bool) else (63 if enable else 0)
        _check(library().kvm_profile_enable(self._h, mask))

    def profile_read(self) -> dict:
        """Per-phase device milliseconds and launch counts since the last read (waits for the events)."""
        p = _Prof()
        _check(library().kvm_profile_read(self._h, ctypes.byref(p)))
        return {f[0]: getattr(p, f[0]) for f in _Prof._fields_}

    def info(self) -> dict:
        i = _Info()
        _check(library().kvm_state_get_info(self._h, ctypes.byref(i)))
        return {f[0]: getattr(i, f[0]) for f in _Info._fields_}

    def read(self, trace: bool = False, chunk: int = -1, ring: bool = False, sums: Optional[bool] = None) -> dict:
        """Copy the state into new device tensors (queued on the current stream).

        chunk -1: the current state (raw sums, counts, radii, read form; the window ring
        with ring=True; the per-token trace with trace=True).  chunk j >= 0: the state
        right after absorbed chunk j (counts, radii and read form; the library refuses
        the raw sums of a past chunk, sums=True asks for them anyway)."""
        inf = self.info()
        S, Sc, dt = self.cfg.seqs, inf["max_rows"], self.cfg.read_dtype
        dev = self.device
        res = {
            "count": torch.empty(S, Sc, dtype=torch.int32, device=dev),
            "rho": torch.empty(S, Sc, dtype=torch.float32, device=dev),
            "key_read": torch.empty(S, Sc, 32, dtype=dt, device=dev),
            "val_read": torch.empty(S, Sc, 64, dtype=self.cfg.torch_dtype, device=dev),
        }
        if sums if sums is not None else chunk < 0:
            res["key_sum"] = torch.empty(S, Sc, 32, dtype=torch.float32, device=dev)
            res["val_sum"] = torch.empty(S, Sc, 64, dtype=torch.float32, device=dev)
        n_rows = torch.zeros(S, dtype=torch.int32)
        view = _View()
        view.n_rows = n_rows.data_ptr()
        for k_, t in res.items():
            setattr(view, k_, t.data_ptr())
        if trace:
            res["trace_slot"] = torch.empty(S, self.cfg.max_tokens, dtype=torch.int32, device=dev)
            res["trace_kind"] = torch.empty(S, self.cfg.max_tokens, dtype=torch.uint8, device=dev)
            view.trace_slot = res["trace_slot"].data_ptr()
            view.trace_kind = res["trace_kind"].data_ptr()
        if ring:
            R = self.cfg.window + self.cfg.chunk
            res["ring_k"] = torch.empty(S, R, 64, dtype=self.cfg.torch_dtype, device=dev)
            res["ring_v"] = torch.empty(S, R, 64, dtype=self.cfg.torch_dtype, device=dev)
            res["ring_l"] = torch.empty(S, R, dtype=torch.float32, device=dev)
            for k_ in ("ring_k", "ring_v", "ring_l"):
                setattr(view, k_, res[k_].data_ptr())
        _check(library().kvm_state_read(self._h, chunk, ctypes.byref(view), _stream(dev)))
        res["n_rows"] = n_rows
        if chunk < 0:
            res["position"] = int(view.position)
        return res

    def load(self, saved: dict):
        """kvm_state_load from a dict made by read(ring=True) (and trace=True for a traced state)
        of a state with the same configuration.  The tensors must stay alive until the current
        stream has run the load."""
        view = _View()
        view.position = int(saved["position"])
        keep = []
        for k_ in ("key_sum", "val_sum", "count", "rho", "ring_k", "ring_v", "ring_l", "trace_slot", "trace_kind"):
            t = saved.get(k_)
            if t is not None:
                t = t.contiguous()
                keep.append(t)
                setattr(view, k_, t.data_ptr())
        n_rows = saved.get("n_rows")
        if n_rows is not None:
            n_rows = n_rows.to(torch.int32).cpu().contiguous()
            keep.append(n_rows)
            view.n_rows = n_rows.data_ptr()
        _check(library().kvm_state_load(self._h, ctypes.byref(view), _stream(self.device)))
        self._load_keep = keep

    def snapshot(self, j: int):
        """Read form of the state after absorbed chunk j: key [B*H, rows_j, 32] (read_dtype),
        value rho * u [B*H, rows_j, 64] (input dtype) and radius [B*H, rows_j] float32."""
        rows = int(schedule(self.cfg, j + 1)[2][j])
        dt = self.cfg.read_dtype
        kr = torch.empty(self.cfg.seqs, rows, 32, dtype=dt, device=self.device)
        ur = torch.empty(self.cfg.seqs, rows, 64, dtype=self.cfg.torch_dtype, device=self.device)
        rr = torch.empty(self.cfg.seqs, rows, dtype=torch.float32, device=self.device)
        _check(library().kvm_snapshot_read(self._h, j, kr.data_ptr(), ur.data_ptr(), rr.data_ptr(),
                                           _stream(self.device)))
        return kr, ur, rr
