"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Each mutant is the oracle's source with one plausible slip (a dropped term, a
wrong sign or index, a swapped rule), loaded as a separate module; the real
oracle is never modified.
"""
import sys
import types

import numpy as np
import pytest

import oracle.kvm_oracle as O
import tests.test_oracle_pins as pins

SRC_PATH = O.__file__
with open(SRC_PATH) as f:
    SRC = f.read()


def load_mutant(old: str, new: str, count: int = 1) -> types.ModuleType:
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = SRC.replace(old, new, count)
    name = f"kvm_oracle_mutant_{abs(hash((old, new)))}"
    mod = types.ModuleType(name)
    mod.__file__ = SRC_PATH
    sys.modules[name] = mod
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def fails(check, mod, *args) -> bool:
    try:
        check(mod, *args)
    except (AssertionError, ValueError, IndexError, KeyError, FloatingPointError):
        return True
    return False


def i9(mod):
    """test_I9_tie_rules against a module."""
    p = mod.Params(chunk=4, window=4, n_sinks=0, sched="fixed", max_slots=5)
    N = 16
    k = np.zeros((N, 64))
    e = np.eye(32)
    for t, r in [(0, 0), (1, 1), (2, 1), (3, 2), (4, 1), (5, 5), (6, 5)]:
        k[t, 32:] = e[r]
    rng = np.random.default_rng(0)
    q, v = rng.standard_normal((N, 64)), rng.standard_normal((N, 64))
    res = mod.prefill(q, k, v, np.zeros(N), p)
    assert list(res.kind[:8]) == [1, 1, 1, 1, 2, 1, 2, 2]
    assert list(res.slot[:8]) == [0, 1, 2, 3, 1, 4, 4, 0]


def i13(mod):
    p = mod.Params(chunk=8, window=16, n_sinks=2, sched="sqrt", alpha=2)
    q, k, v, ell = pins.rand_seq(90, 5, clustered=4)
    np.testing.assert_allclose(mod.prefill(q, k, v, ell, p).out, O.brute_force(q, k, v, ell, p), atol=1e-11)


def i11(mod):
    p = mod.Params(chunk=8, window=16, n_sinks=2, sched="sqrt", alpha=2)
    q, k, v, ell = pins.rand_seq(70, 6, clustered=4)
    np.testing.assert_allclose(mod.decode(q, k, v, ell, p), O.prefill(q, k, v, ell, p).out, atol=1e-12)


ALL = [
    pins.check_gate, pins.check_rope, pins.check_window_covers_all, pins.check_append_everything,
    pins.check_read_form, lambda m: pins.check_sums_and_counts(m, "random"), pins.check_assignment_rules,
    pins.check_attention_with_state, i9, i13, i11,
    pins.check_no_gate_is_saturated_gate, pins.check_mean_read_without_value_norm, pins.check_unprotected_sinks,
    pins.check_power_schedule, pins.check_softmax_scale,
]

MUTANTS = {
    "gate sign flipped": ("return 1.0 / (1.0 + np.exp(-ell))", "return 1.0 / (1.0 + np.exp(ell))"),
    "rope rotates the other way": ("x[..., :half] = a * c - b * s", "x[..., :half] = a * c + b * s"),
    "rope pairs adjacent dims": ("b = x[..., half:rope_dims].copy()", "b = x[..., half + 1:rope_dims + 1].copy()"),
    "rope frequency exponent": ("freq = theta ** (-2.0 * j / rope_dims)", "freq = theta ** (-1.0 * j / rope_dims)"),
    "layernorm eps dropped": ("np.sqrt(var + p.ln_eps)", "np.sqrt(var)"),
    "count not divided out": ("x = K / n[:, None]", "x = K"),
    "value radius ignored": ("vhat[ok] = rho[ok, None] * V[ok] / nv[ok, None]", "vhat[ok] = V[ok] / n[ok, None]"),
    "merge ungated": ("st.K[i] = st.K[i] + g[t] * ktil[t]", "st.K[i] = st.K[i] + ktil[t]"),
    "value merge ungated": ("st.V[i] = st.V[i] + g[t] * v[t]", "st.V[i] = st.V[i] + v[t]"),
    "count not incremented": ("st.n[i] += 1", "st.n[i] += 0"),
    "dot product instead of cosine": ("np.divide(dots, den, out=out, where=den > 0)", "out[...] = dots"),
    "append the least surprising": ("ranked = sorted(P, key=lambda t: (mu[t], t))",
                                    "ranked = sorted(P, key=lambda t: (-mu[t], t))"),
    "ties to the later position": ("ranked = sorted(P, key=lambda t: (mu[t], t))",
                                   "ranked = sorted(P, key=lambda t: (mu[t], -t))"),
    "ties to the highest row": ("best = np.argmax(cs, axis=1)",
                                "best = cs.shape[1] - 1 - np.argmax(cs[:, ::-1], axis=1)"),
    "sinks are merge candidates": ("return not (st.sink[i] and p.sink_protect)", "return True"),
    "merge candidates exclude this chunk's new rows": ("cand = E + [i for i in range(first_row, st.rows) if eligible(i)]",
                                                       "cand = E"),
    "unprotected sinks still excluded": ("return not (st.sink[i] and p.sink_protect)", "return not st.sink[i]"),
    "gate kept when removed": ("    if p.merge_gate:\n        return gate(ell)", "    if True:\n        return gate(ell)"),
    "radius kept when value normalisation is removed": ("    if not p.value_norm:\n        return khat, V / n[:, None]",
                                                        "    if False:\n        return khat, V / n[:, None]"),
    "power exponent ignored": ("float(T) ** float(p.exponent)", "float(T) ** 0.5"),
    "window one token short": ("lo = max(0, c * C - p.window)\n    keys", "lo = max(0, c * C - p.window + 1)\n    keys"),
    "absorb one chunk late": ("while absorbed <= c - W // C - 1:", "while absorbed <= c - W // C - 2:"),
    "softmax scale squared": ("else 1.0 / math.sqrt(p.head_dim)", "else 1.0 / p.head_dim"),
    "given softmax scale ignored": ("return float(p.softmax_scale) if p.softmax_scale > 0",
                                    "return 1.0 / math.sqrt(p.head_dim) if p.softmax_scale > 0"),
    "rotary dims of state keys not zeroed": ("khat = np.zeros((S, d))\n    vhat", "khat = np.ones((S, d))\n    vhat"),
    "capacity floor instead of ceil": ("return r if r * r == x else r + 1", "return r"),
    "radius of the current sum": ("self.rho.append(float(np.linalg.norm(v)))", "self.rho.append(1.0)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    mod = load_mutant(old, new)
    caught = [i for i, chk in enumerate(ALL) if fails(chk, mod)]
    assert caught, f"no pin caught the planted mistake: {name}"


def test_unmutated_copy_passes_every_pin():
    mod = load_mutant("KIND_NONE = -1", "KIND_NONE = -1")
    bad = [i for i, chk in enumerate(ALL) if fails(chk, mod)]
    assert not bad
