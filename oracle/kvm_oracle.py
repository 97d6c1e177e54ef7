"""CPU oracle of the Key-Value Means (KVM) attention layer.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package.  The HIP library never uses it, and it
shares no code, tables or constants with the HIP library.

Plain, slow, NumPy float64.  The method is a block recurrence with a
data-dependent compression, not an exact function computed faster, so this
file follows the method's steps in the order the pages give them:

  [KVM summary, Core mechanisms 1]  input is processed in chunks; a fixed-size
      block-sliding window (BSWA) keeps recent tokens exactly, a separate state
      holds older tokens; a block that overflows the window updates the state.
  [KVM summary, Core mechanisms 2]  overflowed keys are merged winner-take-all
      into the single most similar state key (cosine similarity); state keys
      are LayerNorm-ed and state values rescaled to the row's read radius rho_i
      just in time, at read; a data-dependent scalar gate scales what is merged.
  [KVM summary, Core mechanisms 3]  the most surprising (least redundant)
      overflowed tokens are appended as new rows, the rest merged; the state
      size follows a schedule (fixed, power-law sqrt, saturating; see
      "Experimental results").
  [KVM summary, Core mechanisms 4]  the rotary subspace of state keys is zero;
      unrotated queries meet the state, rotated queries the window, in one pass.
  [KVM summary, Core mechanisms 5]  a protected set of initial rows (sinks).
  [KVM lay summary, "smart merge"]  rows are kept as raw sums and counts and
      divided only when read.
  [KVM abstract]  one softmax attention layer; chunk-parallel prefill.

Where the pages leave a step open the plainest reading is taken; each is
stated at the function that uses it.  "(reading)" marks those places.

Public entry points: gate, rope, capacity, schedule, prefill, decode,
brute_force.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

KIND_NONE = -1   # token not absorbed (still in the window)
KIND_SINK = 0
KIND_APPEND = 1
KIND_MERGE = 2


@dataclass(frozen=True)
class Params:
    """Layer constants.  sched: 'fixed' | 'sqrt' | 'saturating' | 'power'.

    The last four fields select the variants of [KVM summary, Experimental
    results] (power-law schedules) and of its ablation study (value-length
    normalisation, sink protection and the merge gate, each removable).
    """

    chunk: int
    window: int
    n_sinks: int
    sched: str
    max_slots: int = 0
    alpha: int = 0
    head_dim: int = 64
    rope_dims: int = 32
    rope_theta: float = 10000.0
    ln_eps: float = 1e-5
    exponent: float = 0.5          # 'power' schedule: capacity ceil(alpha * T**exponent)
    value_norm: bool = True        # read values at the row's radius (else the plain mean V/n)
    sink_protect: bool = True      # sink rows are never merge targets nor surprise references
    merge_gate: bool = True        # merged tokens are scaled by sigmoid(l) (else by 1)
    softmax_scale: float = 0.0     # logit scale; 0 means 1/sqrt(head_dim)

    @staticmethod
    def of(cfg) -> "Params":
        """Build from any object with the same attribute names (e.g. a workload config)."""
        return Params(chunk=cfg.chunk, window=cfg.window, n_sinks=cfg.n_sinks, sched=cfg.sched,
                      max_slots=cfg.max_slots, alpha=cfg.alpha, head_dim=cfg.head_dim,
                      rope_dims=cfg.rope_dims, rope_theta=cfg.rope_theta, ln_eps=cfg.ln_eps,
                      exponent=getattr(cfg, "exponent", 0.5), value_norm=getattr(cfg, "value_norm", True),
                      sink_protect=getattr(cfg, "sink_protect", True),
                      merge_gate=getattr(cfg, "merge_gate", True),
                      softmax_scale=getattr(cfg, "softmax_scale", 0.0))


# --------------------------------------------------------------------------
# Elementary pieces
# --------------------------------------------------------------------------

def logit_scale(p: Params) -> float:
    """The one softmax scale shared by state and window logits.

    [KVM summary, Methodology]: one softmax attention layer over state and
    window.  (reading) The usual 1/sqrt(head_dim) unless a scale is given.
    """
    return float(p.softmax_scale) if p.softmax_scale > 0 else 1.0 / math.sqrt(p.head_dim)


def merge_weights(ell, p: Params):
    """The per-token merge weight: the gate, or 1 without it ([KVM summary,
    Experimental results, ablations]: the merge gate can be removed)."""
    if p.merge_gate:
        return gate(ell)
    return np.ones_like(np.asarray(ell, dtype=np.float64))


def gate(ell):
    """Merge gate g = sigmoid(l).

    [KVM summary, Core mechanisms 2, merge gate]: a data-dependent scalar that
    scales how much of an incoming overflowed key/value the state absorbs.
    (reading) The pages do not give the gate's form; it is the logistic
    sigmoid of a given per-token logit.
    """
    ell = np.asarray(ell, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-ell))


def rope(x, pos, rope_dims: int = 32, theta: float = 10000.0):
    """Rotary position embedding on the first `rope_dims` dims of x (rows at positions `pos`).

    [KVM summary, Core mechanisms 4]: the window keeps full RoPE.
    (reading) Rotate-half pairing: dim j pairs with dim j + rope_dims/2,
    frequency f_j = theta^(-2j/rope_dims), angle = position * f_j; dims beyond
    rope_dims are left unchanged.  Positions are absolute, from 0.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    pos = np.asarray(pos, dtype=np.float64).reshape(-1)
    half = rope_dims // 2
    j = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * j / rope_dims)
    ang = pos[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., :half].copy()
    b = x[..., half:rope_dims].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rope_dims] = b * c + a * s
    return x


def _ceil_sqrt_int(x: int) -> int:
    r = math.isqrt(x)
    return r if r * r == x else r + 1


def capacity(T: int, p: Params) -> int:
    """Target number of state rows (sinks included) once T tokens have been absorbed.

    [KVM summary, Core mechanisms 3] sublinear growth such as O(sqrt N);
    [KVM summary, Experimental results] fixed (256), power-law ("KVM sqrt")
    and saturating schedules.
    (reading) fixed: max_slots; sqrt: ceil(alpha*sqrt(T)); saturating:
    min(max_slots, ceil(alpha*sqrt(T))).  ceil(alpha*sqrt(T)) is taken as the
    exact integer ceiling of sqrt(alpha^2 * T) (alpha an integer).  power:
    ceil(alpha * T**exponent) in IEEE double (the power-law family the sqrt
    variant belongs to; the exact integer form above is kept for sqrt).
    """
    if p.sched == "fixed":
        return p.max_slots
    if p.sched == "power":
        return int(math.ceil(float(p.alpha) * float(T) ** float(p.exponent)))
    c = _ceil_sqrt_int(p.alpha * p.alpha * int(T))
    if p.sched == "sqrt":
        return c
    if p.sched == "saturating":
        return min(p.max_slots, c)
    raise ValueError(p.sched)


def schedule(n_absorbed_chunks: int, p: Params):
    """Per absorbed chunk j: (sinks created, appends m_j, rows after chunk j).

    Data-independent: follows from the capacity rule and the sink count alone.
    """
    out = []
    rows = 0
    sinks = 0
    for j in range(n_absorbed_chunks):
        cand = p.chunk
        s = min(p.n_sinks - sinks, cand)
        sinks += s
        rows += s
        cand -= s
        T = (j + 1) * p.chunk
        m = min(max(capacity(T, p) - rows, 0), cand)
        rows += m
        out.append((s, m, rows))
    return out


def cosine_matrix(X, Y):
    """cos(x_a, y_b) for every row pair, shape [len(X), len(Y)]; 0 where a norm is 0."""
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    nx = np.linalg.norm(X, axis=1)
    ny = np.linalg.norm(Y, axis=1)
    dots = X @ Y.T
    den = nx[:, None] * ny[None, :]
    out = np.zeros_like(dots)
    np.divide(dots, den, out=out, where=den > 0)
    return out


# --------------------------------------------------------------------------
# State
# --------------------------------------------------------------------------

@dataclass
class State:
    """Ordered state rows: raw key sum K_i (live dims), raw value sum V_i,
    count n_i, read radius rho_i, sink flag.

    [KVM lay summary, "smart merge"]: raw sums and counts, divided only when read.
    (reading) State keys keep only the non-rotary dims: the rotary subspace of
    state keys is zero [KVM summary, Core mechanisms 4], so it is dropped
    before the cosine, the sums and the LayerNorm.
    """

    dk: int
    dv: int
    K: List[np.ndarray] = field(default_factory=list)
    V: List[np.ndarray] = field(default_factory=list)
    n: List[int] = field(default_factory=list)
    rho: List[float] = field(default_factory=list)
    sink: List[bool] = field(default_factory=list)

    @property
    def rows(self) -> int:
        return len(self.K)

    @property
    def n_sinks(self) -> int:
        return int(sum(self.sink))

    def add_row(self, ktil, v, sink: bool):
        # (reading) the read radius is the norm of the row's creating value,
        # fixed at creation [KVM summary, Core mechanisms 2, JIT renormalisation]
        self.K.append(np.array(ktil, dtype=np.float64))
        self.V.append(np.array(v, dtype=np.float64))
        self.n.append(1)
        self.rho.append(float(np.linalg.norm(v)))
        self.sink.append(bool(sink))

    def copy(self) -> "State":
        return State(self.dk, self.dv, [a.copy() for a in self.K], [a.copy() for a in self.V],
                     list(self.n), list(self.rho), list(self.sink))

    def arrays(self):
        S = self.rows
        K = np.array(self.K).reshape(S, self.dk)
        V = np.array(self.V).reshape(S, self.dv)
        return K, V, np.array(self.n, dtype=np.int64), np.array(self.rho), np.array(self.sink, dtype=bool)


@dataclass
class ChunkLog:
    """What absorbing one chunk decided, plus the margins that decided it."""

    j: int
    m: int
    appended: List[int]
    mu: Dict[int, float]                 # surprise of each candidate position
    append_margin: float                 # mu gap across the append boundary (+inf if no choice)
    assign: Dict[int, int]               # merged position -> row
    assign_margin: Dict[int, float]      # merged position -> top1 - top2 cosine (+inf if one candidate)
    sinks: List[int]


def absorb_chunk(st: State, j: int, ktil, v, g, p: Params, forced: Optional[dict] = None) -> ChunkLog:
    """Absorb overflowed chunk j (positions [jC, jC+C)) into the state.

    ktil, v, g are indexed by absolute position.  Steps (a)-(f) below.

    forced: optional {position: (kind, row)} decisions to apply instead of this
    oracle's own (teacher forcing).  The oracle's own decisions and margins are
    still computed and returned, so a caller can compare them with the forced
    ones step by step.
    """
    C = p.chunk
    P = list(range(j * C, (j + 1) * C))
    first_row = st.rows
    # rows that take part as references and merge targets: all of them, except
    # protected sinks ([KVM summary, Experimental results, ablations]: removing
    # sink protection makes the sink rows ordinary rows)
    def eligible(i):
        return not (st.sink[i] and p.sink_protect)

    # (a) sinks [KVM summary, Core mechanisms 5]: (reading) the earliest tokens
    # of the sequence become protected rows, created unscaled, never merge targets.
    sinks = []
    while st.n_sinks < p.n_sinks and P:
        t = P.pop(0)
        st.add_row(ktil[t], v[t], sink=True)
        sinks.append(t)

    # (b) how many rows to append [KVM summary, Core mechanisms 3]
    T = (j + 1) * C
    m = min(max(capacity(T, p) - st.rows, 0), len(P))

    # (c) surprise: the best cosine against the non-sink rows that existed
    # before this chunk (reading: -inf when there are none).
    E = [i for i in range(first_row) if eligible(i)]
    mu = {}
    if E and P:
        KE = np.array([st.K[i] for i in E])
        best = cosine_matrix(ktil[P], KE).max(axis=1)
        for t, b in zip(P, best):
            mu[t] = float(b)
    else:
        for t in P:
            mu[t] = -math.inf

    # (d) append the m most surprising (smallest surprise score, earlier
    # position on ties); rows are created in position order.
    ranked = sorted(P, key=lambda t: (mu[t], t))
    A_own = sorted(ranked[:m])
    if 0 < m < len(P) and E:
        append_margin = mu[ranked[m]] - mu[ranked[m - 1]]
    else:
        append_margin = math.inf

    if forced is not None:
        A = sorted(t for t in P if forced[t][0] == KIND_APPEND)
        if len(A) != m:
            raise ValueError(f"chunk {j}: forced append count {len(A)} != schedule {m}")
    else:
        A = A_own
    for t in A:
        st.add_row(ktil[t], v[t], sink=False)
    cand = E + [i for i in range(first_row, st.rows) if eligible(i)]

    # (e) winner-take-all assignment [KVM summary, Core mechanisms 2]: each
    # remaining token goes to the single candidate row of highest cosine,
    # judged against the sums as they stand after the appends and before any
    # merge of this chunk (reading: chunk-synchronous update); ties go to the
    # lowest row index.
    M = [t for t in P if t not in set(A)]
    Kc = np.array([st.K[i] for i in cand]) if cand else np.zeros((0, st.dk))
    assign, assign_margin = {}, {}
    own_assign = {}
    if M:
        if not cand:
            raise ValueError("no candidate row for a merged token (capacity must exceed the sink count)")
        cs = cosine_matrix(ktil[M], Kc)                # [|M|, |cand|]
        best = np.argmax(cs, axis=1)                   # first maximum = lowest row index
        if cs.shape[1] > 1:
            top2 = -np.partition(-cs, 1, axis=1)[:, :2]
            margin = top2[:, 0] - top2[:, 1]
        else:
            margin = np.full(len(M), math.inf)
        for a, t in enumerate(M):
            own_assign[t] = cand[int(best[a])]
            assign_margin[t] = float(margin[a])
    if forced is not None:
        for t in M:
            kind, row = forced[t]
            if kind != KIND_MERGE:
                raise ValueError(f"position {t}: forced kind {kind}, expected merge")
            assign[t] = int(row)
    else:
        assign = dict(own_assign)

    # (f) merge: gated raw sums; the count grows by one per token (reading:
    # counts are not gated).
    for t in M:
        i = assign[t]
        st.K[i] = st.K[i] + g[t] * ktil[t]
        st.V[i] = st.V[i] + g[t] * v[t]
        st.n[i] += 1

    return ChunkLog(j=j, m=m, appended=A_own, mu=mu, append_margin=append_margin,
                    assign=own_assign, assign_margin=assign_margin, sinks=sinks)


def read_form(st: State, p: Params):
    """Just-in-time read form of every row.

    [KVM summary, Core mechanisms 2, JIT renormalisation]: state keys pass
    through LayerNorm before attention; state values are rescaled to the
    row's read radius rho_i, keeping magnitude and letting direction change.
    [KVM lay summary]: division by the count happens only now.
    (reading) LayerNorm over the live dims of K_i / n_i, biased variance,
    eps = ln_eps, no affine parameters; the rotary dims of the key are zero.
    v_hat = rho_i * V_i / |V_i| (0 if |V_i| = 0).  Without value-length
    normalisation ([KVM summary, Experimental results, ablations]) the value
    is read as the plain mean V_i / n_i.
    Returns k_hat [S, head_dim], v_hat [S, head_dim].
    """
    d, dr = p.head_dim, p.rope_dims
    S = st.rows
    khat = np.zeros((S, d))
    vhat = np.zeros((S, st.dv))
    if S == 0:
        return khat, vhat
    K, V, n, rho, _ = st.arrays()
    x = K / n[:, None]
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
    khat[:, dr:] = (x - mean) / np.sqrt(var + p.ln_eps)
    if not p.value_norm:
        return khat, V / n[:, None]
    nv = np.linalg.norm(V, axis=1)
    ok = nv > 0
    vhat[ok] = rho[ok, None] * V[ok] / nv[ok, None]
    return khat, vhat


def attend_one(t: int, q_t, qr_t, khat, vhat, kr, v, p: Params, c: int):
    """One query at position t in query chunk c, one softmax over [state || window].

    [KVM summary, Methodology; Core mechanisms 4]: a single softmax attention
    layer; the unrotated query scores the state keys, the rotated query scores
    the window keys.  (reading) One scale, logit_scale(p), for both parts; the
    window is [max(0, cC - W), t].
    """
    s = logit_scale(p)
    lo = max(0, c * p.chunk - p.window)
    logits_state = s * (khat @ q_t) if khat.shape[0] else np.zeros(0)
    logits_win = s * (kr[lo:t + 1] @ qr_t)
    allv = np.concatenate([logits_state, logits_win])
    mx = allv.max()
    w = np.exp(allv - mx)
    w /= w.sum()
    ns = khat.shape[0]
    out = w[:ns] @ vhat if ns else np.zeros(p.head_dim)
    return out + w[ns:] @ v[lo:t + 1]


def attend_chunk(c: int, N: int, q, qr, khat, vhat, kr, v, p: Params):
    """attend_one for every query of chunk c at once (same arithmetic, array form)."""
    s = logit_scale(p)
    C = p.chunk
    rows = np.arange(c * C, min(N, (c + 1) * C))
    lo = max(0, c * C - p.window)
    keys = np.arange(lo, rows[-1] + 1)
    Ls = s * (q[rows] @ khat.T)                                   # [r, S]
    Lw = s * (qr[rows] @ kr[keys].T)                              # [r, w]
    Lw = np.where(keys[None, :] <= rows[:, None], Lw, -np.inf)    # causal inside the window
    L = np.hstack([Ls, Lw])
    L = L - L.max(axis=1, keepdims=True)
    w = np.exp(L)
    w /= w.sum(axis=1, keepdims=True)
    ns = khat.shape[0]
    return w[:, :ns] @ vhat + w[:, ns:] @ v[keys]


# --------------------------------------------------------------------------
# Whole layer, one sequence
# --------------------------------------------------------------------------

@dataclass
class SeqResult:
    out: np.ndarray                       # [N, head_dim]
    state: State                          # final state
    kind: np.ndarray                      # [N] per position
    slot: np.ndarray                      # [N] row a position created or merged into (-1 if none)
    logs: List[ChunkLog]
    rows_after: List[int]                 # rows after each absorbed chunk
    snapshots: Optional[List[State]] = None


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def prefill(q, k, v, ell, p: Params, forced: Optional[dict] = None, keep_snapshots: bool = False,
            attend_chunks=None) -> SeqResult:
    """Chunk-by-chunk layer output for one sequence of N tokens.

    [KVM abstract]: chunk-wise prefill.  For query chunk c = 0, 1, ...:
      1. absorb every chunk j <= c - W/C - 1 not yet absorbed (the tokens that
         left the window) [KVM summary, Core mechanisms 1];
      2. build the read form [Core mechanisms 2];
      3. attend each query of the chunk over [state || window] [Core mechanisms 4].
    (reading) Query chunk c sees window keys [cC - W, t] and a state made of the
    tokens before cC - W: the past is split with no overlap.
    q, k, v: [N, head_dim]; ell: [N] gate logits.
    forced: optional {position: (kind, row)} (teacher forcing, see absorb_chunk).
    attend_chunks: optional set of query chunks whose outputs are computed
    (sampling for long inputs); other rows of `out` are NaN.  Absorption
    always runs over every chunk.
    """
    q, k, v, ell = _as64(q), _as64(k), _as64(v), _as64(ell)
    N, d = q.shape
    C, W, dr = p.chunk, p.window, p.rope_dims
    if W % C != 0:
        raise ValueError("window must be a multiple of chunk")
    pos = np.arange(N)
    qr = rope(q, pos, dr, p.rope_theta)
    kr = rope(k, pos, dr, p.rope_theta)
    ktil = k[:, dr:]                      # the live (non-rotary) key dims
    g = merge_weights(ell, p)
    st = State(dk=d - dr, dv=v.shape[1])
    kind = np.full(N, KIND_NONE, dtype=np.int64)
    slot = np.full(N, -1, dtype=np.int64)
    logs, rows_after, snaps = [], [], []
    out = np.zeros((N, v.shape[1]))
    absorbed = 0
    n_q_chunks = -(-N // C)
    for c in range(n_q_chunks):
        while absorbed <= c - W // C - 1:
            j = absorbed
            before = st.rows
            lg = absorb_chunk(st, j, ktil, v, g, p, forced)
            _record(lg, st, before, kind, slot, forced, j, p)
            logs.append(lg)
            rows_after.append(st.rows)
            if keep_snapshots:
                snaps.append(st.copy())
            absorbed += 1
        if attend_chunks is not None and c not in attend_chunks:
            out[c * C:min(N, (c + 1) * C)] = np.nan
            continue
        khat, vhat = read_form(st, p)
        out[c * C:min(N, (c + 1) * C)] = attend_chunk(c, N, q, qr, khat, vhat, kr, v, p)
    return SeqResult(out=out, state=st, kind=kind, slot=slot, logs=logs, rows_after=rows_after,
                     snapshots=snaps if keep_snapshots else None)


def _record(lg: ChunkLog, st: State, before: int, kind, slot, forced, j: int, p: Params):
    """Per-position record of what absorbing chunk j did (the applied decisions)."""
    C = p.chunk
    rows_created = list(range(before, st.rows))
    r = 0
    for t in lg.sinks:
        kind[t] = KIND_SINK
        slot[t] = rows_created[r]
        r += 1
    if forced is not None:
        appended = sorted(t for t in range(j * C, (j + 1) * C) if forced[t][0] == KIND_APPEND)
    else:
        appended = lg.appended
    for t in appended:
        kind[t] = KIND_APPEND
        slot[t] = rows_created[r]
        r += 1
    for t in range(j * C, (j + 1) * C):
        if kind[t] == KIND_NONE:
            kind[t] = KIND_MERGE
            slot[t] = forced[t][1] if forced is not None else lg.assign[t]


class Decoder:
    """Token-at-a-time form of the same layer (decode).

    [KVM summary, Significance: hybrid use and long-context decoding];
    [KVM summary, Problem statement: per-token cost].  At position t: when t
    starts a chunk and t >= W + C, the chunk [t - W - C, t - W) leaves the
    window and is absorbed; then the single query t attends over
    [state || window [cC - W, t]].  Reproduces prefill exactly.
    """

    def __init__(self, p: Params, head_dim: int = 64):
        self.p = p
        self.st = State(dk=head_dim - p.rope_dims, dv=head_dim)
        self.q, self.k, self.v, self.ell = [], [], [], []
        self.absorbed = 0
        self.logs: List[ChunkLog] = []

    def prime(self, res: SeqResult, q, k, v, ell):
        """Continue after a prefill of len(q) tokens whose result is `res`."""
        self.st = res.state.copy()
        self.q = list(_as64(q))
        self.k = list(_as64(k))
        self.v = list(_as64(v))
        self.ell = list(_as64(ell))
        self.absorbed = len(res.rows_after)
        self.logs = list(res.logs)

    def step(self, q_t, k_t, v_t, ell_t, forced: Optional[dict] = None):
        p = self.p
        C, W, dr = p.chunk, p.window, p.rope_dims
        t = len(self.q)
        self.q.append(_as64(q_t))
        self.k.append(_as64(k_t))
        self.v.append(_as64(v_t))
        self.ell.append(float(ell_t))
        c = t // C
        if t % C == 0 and t >= W + C:
            j = (t - W - C) // C
            assert j == self.absorbed
            K = np.array(self.k)
            V = np.array(self.v)
            lg = absorb_chunk(self.st, j, K[:, dr:], V, merge_weights(np.array(self.ell), p), p, forced)
            self.logs.append(lg)
            self.absorbed += 1
        khat, vhat = read_form(self.st, p)
        lo = max(0, c * C - W)
        pos = np.arange(lo, t + 1)
        K = np.array(self.k[lo:t + 1])
        kr = np.zeros((t + 1, K.shape[1]))
        kr[lo:] = rope(K, pos, dr, p.rope_theta)
        V = np.zeros((t + 1, len(v_t)))
        V[lo:] = np.array(self.v[lo:t + 1])
        qr_t = rope(self.q[t][None, :], [t], dr, p.rope_theta)[0]
        return attend_one(t, self.q[t], qr_t, khat, vhat, kr, V, p, c)


def decode(q, k, v, ell, p: Params) -> np.ndarray:
    """All N outputs produced one token at a time with Decoder."""
    dec = Decoder(p, head_dim=np.shape(q)[1])
    return np.array([dec.step(q[t], k[t], v[t], ell[t]) for t in range(len(q))])


# --------------------------------------------------------------------------
# Second formulation, for tiny inputs only
# --------------------------------------------------------------------------

def brute_force(q, k, v, ell, p: Params) -> np.ndarray:
    """Same layer in matrix form, recomputed from scratch for every query chunk.

    For each query chunk c the state is rebuilt by replaying every overflowed
    chunk from an empty state, with the update written as a one-hot
    (maximally sparse) update matrix applied to a matrix of tokens [KVM
    summary, Core mechanisms 2: similarity metric]; then every query of the
    chunk attends over [read-form state || all N tokens] with a dense N-wide
    mask that keeps only [max(0, cC - W), t].  Shares no helper with the
    incremental form above except `gate`, `rope` and `capacity`.  The ablation
    variants of Params are written out here on their own: merge weight 1
    without the gate; unprotected sinks are ordinary rows (surprise references
    and merge targets); without value-length normalisation a row reads its
    mean value.
    """
    q, k, v, ell = _as64(q), _as64(k), _as64(v), _as64(ell)
    N, d = q.shape
    C, W, dr = p.chunk, p.window, p.rope_dims
    pos = np.arange(N)
    qr = rope(q, pos, dr, p.rope_theta)
    kr = rope(k, pos, dr, p.rope_theta)
    kt = k[:, dr:]
    g = gate(ell) if p.merge_gate else np.ones(N)
    scale = p.softmax_scale if p.softmax_scale > 0 else d ** -0.5
    out = np.zeros((N, v.shape[1]))
    for c in range(-(-N // C)):
        Ks = np.zeros((0, d - dr))
        Vs = np.zeros((0, v.shape[1]))
        cnt = np.zeros(0)
        rad = np.zeros(0)
        is_sink = np.zeros(0, dtype=bool)
        for j in range(0, c - W // C):
            toks = np.arange(j * C, (j + 1) * C)
            n_new_sinks = min(p.n_sinks - int(is_sink.sum()), len(toks))
            sk = toks[:n_new_sinks]
            rest = toks[n_new_sinks:]
            Ks = np.vstack([Ks, kt[sk]])
            Vs = np.vstack([Vs, v[sk]])
            cnt = np.concatenate([cnt, np.ones(len(sk))])
            rad = np.concatenate([rad, np.linalg.norm(v[sk], axis=1)])
            is_sink = np.concatenate([is_sink, np.ones(len(sk), dtype=bool)])
            m = min(max(capacity((j + 1) * C, p) - len(Ks), 0), len(rest))
            protected = is_sink if p.sink_protect else np.zeros(len(Ks), dtype=bool)
            n_before = len(Ks) - len(sk)               # rows that existed before this chunk
            old = np.where(~protected[:n_before])[0]

            def unit(X):
                nr = np.linalg.norm(X, axis=1, keepdims=True)
                return np.where(nr > 0, X / np.where(nr > 0, nr, 1.0), 0.0)

            if len(old):
                sims = unit(kt[rest]) @ unit(Ks[old]).T
                surprise = sims.max(axis=1)
            else:
                surprise = np.full(len(rest), -np.inf)
            order = np.lexsort((rest, surprise))        # by surprise, then position
            app = np.sort(rest[order[:m]])
            mer = np.setdiff1d(rest, app)
            Ks = np.vstack([Ks, kt[app]])
            Vs = np.vstack([Vs, v[app]])
            cnt = np.concatenate([cnt, np.ones(len(app))])
            rad = np.concatenate([rad, np.linalg.norm(v[app], axis=1)])
            is_sink = np.concatenate([is_sink, np.zeros(len(app), dtype=bool)])
            cands = np.where(~is_sink)[0] if p.sink_protect else np.arange(len(Ks))
            if len(mer):
                sims = unit(kt[mer]) @ unit(Ks[cands]).T
                win = cands[np.argmax(sims, axis=1)]
                U = np.zeros((len(Ks), len(mer)))           # one nonzero per column
                U[win, np.arange(len(mer))] = 1.0
                Ks = Ks + U @ (g[mer][:, None] * kt[mer])
                Vs = Vs + U @ (g[mer][:, None] * v[mer])
                cnt = cnt + U.sum(axis=1)
        x = Ks / cnt[:, None] if len(Ks) else Ks
        if len(Ks):
            mu = x.mean(axis=1, keepdims=True)
            sd = np.sqrt(((x - mu) ** 2).mean(axis=1, keepdims=True) + p.ln_eps)
            kh = np.hstack([np.zeros((len(Ks), dr)), (x - mu) / sd])
            if p.value_norm:
                vn = np.linalg.norm(Vs, axis=1, keepdims=True)
                vh = np.where(vn > 0, rad[:, None] * Vs / np.where(vn > 0, vn, 1.0), 0.0)
            else:
                vh = Vs / cnt[:, None]
        else:
            kh = np.zeros((0, d))
            vh = np.zeros((0, v.shape[1]))
        rows = np.arange(c * C, min(N, (c + 1) * C))
        Ls = scale * (q[rows] @ kh.T)                          # [r, S]
        Lw = scale * (qr[rows] @ kr.T)                         # [r, N]
        mask = (pos[None, :] >= max(0, c * C - W)) & (pos[None, :] <= rows[:, None])
        Lw = np.where(mask, Lw, -np.inf)
        L = np.hstack([Ls, Lw])
        L = L - L.max(axis=1, keepdims=True)
        P = np.exp(L)
        P /= P.sum(axis=1, keepdims=True)
        out[rows] = P[:, :len(Ks)] @ vh + P[:, len(Ks):] @ v
    return out
