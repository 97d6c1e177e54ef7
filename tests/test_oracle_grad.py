"""Pins of the oracle's backward pass (CPU only).

The backward (oracle/kvm_oracle_grad.py) holds the forward's decisions fixed.
It is checked against things other than itself:

  - central finite differences of the oracle forward (teacher-forced with the
    base decisions, so that a perturbation cannot flip a decision), along
    random directions of each input separately, for the schedules, the
    ablation variants and a given softmax scale;
  - with the window covering the sequence the layer is causal RoPE attention:
    torch autograd of scaled_dot_product_attention (float64);
  - with every absorbed token appended the layer is dense attention over
    LayerNorm-ed keys and the tokens' own values: torch autograd of
    F.layer_norm + scaled_dot_product_attention (float64).

The `check_*` helpers take the module so that planted mistakes can be run
against them (test_oracle_grad_mutations below).
"""
import sys
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.kvm_oracle as O
import oracle.kvm_oracle_grad as G
from tests.test_oracle_pins import rand_seq, rope_complex

pytestmark = pytest.mark.filterwarnings("ignore")


def loss_and_grad(mod, q, k, v, ell, w, p):
    res = mod.prefill_grad(q, k, v, ell, w, p)
    forced = {int(t): (int(res.fwd.kind[t]), int(res.fwd.slot[t])) for t in np.nonzero(res.fwd.kind >= 0)[0]}
    return res, forced


def fd_check(mod, p, N, seed, clustered=4, eps=1e-5, dirs=2, rtol=2e-6):
    """Directional derivatives of sum(w * out) against central differences, per input."""
    q, k, v, ell = rand_seq(N, seed, clustered=clustered)
    rng = np.random.default_rng(seed + 100)
    w = rng.standard_normal((N, 64))
    res, forced = loss_and_grad(mod, q, k, v, ell, w, p)
    assert len(forced) > 0 or N <= p.window

    def loss(q_, k_, v_, l_):
        return float(np.sum(w * O.prefill(q_, k_, v_, l_, p, forced=forced or None).out))

    grads = {"q": res.dq, "k": res.dk, "v": res.dv, "l": res.dl}
    base = {"q": q, "k": k, "v": v, "l": ell}
    for name in ("q", "k", "v", "l"):
        for _ in range(dirs):
            D = rng.standard_normal(base[name].shape)
            plus = dict(base)
            minus = dict(base)
            plus[name] = base[name] + eps * D
            minus[name] = base[name] - eps * D
            fd = (loss(plus["q"], plus["k"], plus["v"], plus["l"]) -
                  loss(minus["q"], minus["k"], minus["v"], minus["l"])) / (2 * eps)
            an = float(np.sum(grads[name] * D))
            scale = max(1.0, abs(fd), float(np.sum(np.abs(grads[name] * D))) * 1e-3)
            assert abs(fd - an) <= rtol * scale, f"d/d{name}: finite difference {fd} vs analytic {an}"


CASES = {
    "sqrt with sinks": (dict(chunk=8, window=16, n_sinks=2, sched="sqrt", alpha=2), 90),
    "fixed, merge-only after the first chunks": (dict(chunk=8, window=16, n_sinks=3, sched="fixed", max_slots=9), 100),
    "no merge gate": (dict(chunk=8, window=8, n_sinks=1, sched="sqrt", alpha=2, merge_gate=False), 80),
    "no value-length normalisation": (dict(chunk=8, window=16, n_sinks=2, sched="sqrt", alpha=2,
                                           value_norm=False), 90),
    "unprotected sinks": (dict(chunk=8, window=8, n_sinks=3, sched="fixed", max_slots=6, sink_protect=False), 80),
    "given softmax scale": (dict(chunk=8, window=16, n_sinks=2, sched="sqrt", alpha=2, softmax_scale=0.31), 90),
}


def check_fd_all(mod):
    for i, (kw, N) in enumerate(CASES.values()):
        fd_check(mod, O.Params(**kw), N, 40 + i)


@pytest.mark.parametrize("case", sorted(CASES))
def test_gradient_matches_finite_differences(case):
    kw, N = CASES[case]
    fd_check(G, O.Params(**kw), N, 40 + sorted(CASES).index(case))


def sdpa_grads(qm, km, vm, mask, w, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None].requires_grad_(True)
    Q, K, V = t(qm), t(km), t(vm)
    o = F.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    (o[0, 0] * torch.from_numpy(w)).sum().backward()
    return Q.grad[0, 0].numpy(), K.grad[0, 0].numpy(), V.grad[0, 0].numpy()


def check_window_covers_all_grad(mod):
    """W >= N: the layer is causal RoPE attention; its gradient is autograd's."""
    N, C = 61, 8
    p = O.Params(chunk=C, window=64, n_sinks=2, sched="fixed", max_slots=8)
    q, k, v, ell = rand_seq(N, 51)
    w = np.random.default_rng(52).standard_normal((N, 64))
    res = mod.prefill_grad(q, k, v, ell, w, p)
    pos = np.arange(N)
    # autograd through RoPE too: rotate inside torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).requires_grad_(True)
    Q, K, V = t(q), t(k), t(v)
    half = 16
    f = torch.from_numpy(np.power(10000.0, -np.arange(half) / half))
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * f[None, :]
    cs, sn = torch.cos(ang), torch.sin(ang)

    def rot(X):
        a, b = X[:, :half], X[:, half:32]
        return torch.cat([a * cs - b * sn, b * cs + a * sn, X[:, 32:]], dim=1)

    mask = torch.from_numpy(np.tril(np.ones((N, N), dtype=bool)))[None, None]
    o = F.scaled_dot_product_attention(rot(Q)[None, None], rot(K)[None, None], V[None, None], attn_mask=mask)
    (o[0, 0] * torch.from_numpy(w)).sum().backward()
    np.testing.assert_allclose(res.dq, Q.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(res.dk, K.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(res.dv, V.grad.numpy(), atol=1e-11)
    np.testing.assert_array_equal(res.dl, 0.0)


def test_window_covering_the_sequence_gradient_is_autograd_of_causal_rope_attention():
    check_window_covers_all_grad(G)


def check_append_everything_grad(mod):
    """Every absorbed token appended (n = 1 everywhere): dense attention over [LN(k_live) rows
    || window], values v at radius |v| (= v itself); autograd of layer_norm + SDPA."""
    N, C, W, ns = 58, 8, 16, 3
    p = O.Params(chunk=C, window=W, n_sinks=ns, sched="fixed", max_slots=10_000)
    q, k, v, ell = rand_seq(N, 61)
    w = np.random.default_rng(62).standard_normal((N, 64))
    res = mod.prefill_grad(q, k, v, ell, w, p)
    pos = np.arange(N)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).requires_grad_(True)
    Q, K, V = t(q), t(k), t(v)
    half = 16
    f = torch.from_numpy(np.power(10000.0, -np.arange(half) / half))
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * f[None, :]
    cs, sn = torch.cos(ang), torch.sin(ang)

    def rot(X):
        a, b = X[:, :half], X[:, half:32]
        return torch.cat([a * cs - b * sn, b * cs + a * sn, X[:, 32:]], dim=1)

    khat = torch.cat([torch.zeros(N, 32, dtype=torch.float64), F.layer_norm(K[:, 32:], (32,), eps=1e-5)], dim=1)
    # value read form rho * V/|V| with rho = |v| and V = v: written out so that autograd sees the radius
    nv = V.norm(dim=1, keepdim=True)
    vhat = nv.detach() * 0 + nv                                    # rho = |v|, same tensor path
    vhat = vhat * V / nv
    mask = np.zeros((N, 2 * N), dtype=bool)
    for tt in range(N):
        lo = max(0, (tt // C) * C - W)
        mask[tt, :lo] = True
        mask[tt, N + lo:N + tt + 1] = True
    keys = torch.cat([khat, rot(K)], dim=0)
    vals = torch.cat([vhat, V], dim=0)
    o = F.scaled_dot_product_attention(rot(Q)[None, None], keys[None, None], vals[None, None],
                                       attn_mask=torch.from_numpy(mask)[None, None])
    (o[0, 0] * torch.from_numpy(w)).sum().backward()
    np.testing.assert_allclose(res.dq, Q.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(res.dk, K.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(res.dv, V.grad.numpy(), atol=1e-10)
    np.testing.assert_array_equal(res.dl, 0.0)       # nothing merges: the gate has no effect


def test_append_everything_gradient_is_autograd_of_dense_attention_on_normalised_keys():
    check_append_everything_grad(G)


# ------------------------------------------------------------------ planted mistakes

SRC = open(G.__file__).read()

GRAD_MUTANTS = {
    "gate factor dropped from merged keys": ("dktil[t] += g[t] * dKt[i]", "dktil[t] += dKt[i]"),
    "gate factor dropped from merged values": ("dv[t] += g[t] * dVt[i]", "dv[t] += dVt[i]"),
    "gate logit chain rule dropped": ("dl = dg * gate * (1.0 - gate)", "dl = dg"),
    "layernorm mean term dropped": ("dx = inv * (g - g.mean(axis=1, keepdims=True) - xhat",
                                    "dx = inv * (g - xhat"),
    "layernorm variance term dropped": (" - xhat * (g * xhat).mean(axis=1, keepdims=True))", ")"),
    "count not divided out": ("dK = dx / n[:, None]", "dK = dx"),
    "radius gradient dropped": ("dv[t] += dVt[i] + (drt[i] * v[t] / nv if nv > 0 else 0.0)", "dv[t] += dVt[i]"),
    "direction projection dropped": ("(gv - u * ug[:, None])", "gv"),
    "rope transpose with the forward angle": ("O.rope(dy, -np.asarray(pos, dtype=np.float64)",
                                              "O.rope(dy, np.asarray(pos, dtype=np.float64)"),
    "softmax row-sum term dropped": ("dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))", "dS = P * dP"),
    "state gradients not carried to earlier chunks": ("        dktil = dktil\n", "        dktil = dktil\n"),
    "suffix sums reset every chunk": ("        snap = fwd.snapshots[j]\n        S = snap.rows\n",
                                      "        snap = fwd.snapshots[j]\n        S = snap.rows\n"
                                      "        dKt[:] = 0.0\n        dVt[:] = 0.0\n        drt[:] = 0.0\n"),
    "window value gradient dropped": ("        dv[keys] += P[:, ns:].T @ dO\n", "\n"),
    "state query gradient dropped": ("        dq[rows] += s * (dS[:, :ns] @ khat)\n", "\n"),
    "scale missing on key gradients": ("dkr[keys] += s * (dS[:, ns:].T @ qr[rows])",
                                       "dkr[keys] += (dS[:, ns:].T @ qr[rows])"),
}
# the placeholder above is not a mutation; drop it
GRAD_MUTANTS.pop("state gradients not carried to earlier chunks")


def load_grad_mutant(old, new):
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = SRC.replace(old, new, 1)
    name = f"kvm_oracle_grad_mutant_{abs(hash((old, new)))}"
    mod = types.ModuleType(name)
    mod.__file__ = G.__file__
    sys.modules[name] = mod
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


GRAD_CHECKS = [check_fd_all, check_window_covers_all_grad, check_append_everything_grad]


@pytest.mark.parametrize("name", sorted(GRAD_MUTANTS))
def test_oracle_grad_mutations_are_caught(name):
    mod = load_grad_mutant(*GRAD_MUTANTS[name])
    caught = []
    for chk in GRAD_CHECKS:
        try:
            chk(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(chk.__name__)
    assert caught, f"no pin caught the planted mistake in the backward: {name}"
