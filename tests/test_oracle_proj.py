"""Pins of the projection oracle (CPU only): brute-force sums on tiny inputs, the
identity-weight closed form (q, k, v are the heads of x), linearity, and planted
mistakes (transposed weights, heads in the wrong order, bias missing) that must fail."""
import sys
import types

import numpy as np
import pytest

import oracle.kvm_oracle_proj as P

SRC = open(P.__file__).read()


def brute_in(x, w, bg, H, hd):
    B, N, D = x.shape
    q = np.zeros((B * H, N, hd)); k = np.zeros_like(q); v = np.zeros_like(q); gl = np.zeros((B * H, N))
    for b in range(B):
        for t in range(N):
            for h in range(H):
                for d in range(hd):
                    f = h * hd + d
                    q[b * H + h, t, d] = sum(x[b, t, i] * w[f, i] for i in range(D))
                    k[b * H + h, t, d] = sum(x[b, t, i] * w[D + f, i] for i in range(D))
                    v[b * H + h, t, d] = sum(x[b, t, i] * w[2 * D + f, i] for i in range(D))
                gl[b * H + h, t] = sum(x[b, t, i] * w[3 * D + h, i] for i in range(D)) + (bg[h] if bg is not None else 0)
    return q, k, v, gl


def brute_out(o, w, B, hd):
    BH, N, _ = o.shape
    H = BH // B
    D = H * hd
    y = np.zeros((B, N, D))
    for b in range(B):
        for t in range(N):
            for f in range(D):
                y[b, t, f] = sum(o[b * H + h, t, d] * w[f, h * hd + d] for h in range(H) for d in range(hd))
    return y


def check_brute(mod):
    rng = np.random.default_rng(3)
    B, N, H, hd = 2, 3, 2, 4
    D = H * hd
    x = rng.standard_normal((B, N, D))
    w = rng.standard_normal((3 * D + H, D))
    bg = rng.standard_normal(H)
    for got, want in zip(mod.project_in(x, w, bg, H, hd), brute_in(x, w, bg, H, hd)):
        np.testing.assert_allclose(got, want, atol=1e-12)
    o = rng.standard_normal((B * H, N, hd))
    wo = rng.standard_normal((D, D))
    np.testing.assert_allclose(mod.project_out(o, wo, B, hd), brute_out(o, wo, B, hd), atol=1e-12)


def check_identity(mod):
    """W_in = [I; 2I; 3I; 0]: q, k, v are x's heads scaled by 1, 2, 3; gate logit = bias.
    W_out = I: project_out is the inverse of the head split."""
    rng = np.random.default_rng(4)
    B, N, H, hd = 2, 5, 3, 4
    D = H * hd
    x = rng.standard_normal((B, N, D))
    I = np.eye(D)
    w = np.vstack([I, 2 * I, 3 * I, np.zeros((H, D))])
    bg = np.array([0.5, -1.0, 2.0])
    q, k, v, gl = mod.project_in(x, w, bg, H, hd)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(q[b * H + h], x[b, :, h * hd:(h + 1) * hd], atol=0)
            np.testing.assert_allclose(k[b * H + h], 2 * x[b, :, h * hd:(h + 1) * hd], atol=0)
            np.testing.assert_allclose(v[b * H + h], 3 * x[b, :, h * hd:(h + 1) * hd], atol=0)
            np.testing.assert_allclose(gl[b * H + h], bg[h], atol=0)
    np.testing.assert_allclose(mod.project_out(q, I, B, hd), x, atol=0)


def check_linearity(mod):
    rng = np.random.default_rng(5)
    B, N, H, hd = 1, 7, 2, 8
    D = H * hd
    x1, x2 = rng.standard_normal((2, B, N, D))
    w = rng.standard_normal((3 * D + H, D))
    a = mod.project_in(1.5 * x1 + x2, w, None, H, hd)
    b1 = mod.project_in(x1, w, None, H, hd)
    b2 = mod.project_in(x2, w, None, H, hd)
    for got, u, z in zip(a, b1, b2):
        np.testing.assert_allclose(got, 1.5 * u + z, atol=1e-12)


CHECKS = [check_brute, check_identity, check_linearity]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_projection_oracle(check):
    check(P)


MUTANTS = {
    "weights transposed": ("y = x.reshape(B * N, D) @ w.T", "y = x.reshape(B * N, D) @ w[:D, :].T @ np.eye(D, 3 * D + H)"),
    "heads and positions swapped": ("reshape(B, N, H, head_dim).transpose(0, 2, 1, 3)",
                                    "reshape(B, H, N, head_dim).transpose(0, 1, 2, 3)"),
    "k and v swapped": ("k = heads_of(y[:, D:2 * D])", "k = heads_of(y[:, 2 * D:3 * D])"),
    "gate bias ignored": ("g = g + np.asarray(b_gate", "g = g + 0 * np.asarray(b_gate"),
    "output weights not transposed": ("return (x @ w.T).reshape(batch, N, D)", "return (x @ w).reshape(batch, N, D)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_projection_mutants_are_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, old
    mod = types.ModuleType(f"proj_mutant_{abs(hash(name))}")
    mod.__file__ = P.__file__
    exec(compile(SRC.replace(old, new, 1), "<mutant>", "exec"), mod.__dict__)
    caught = 0
    for chk in CHECKS:
        try:
            chk(mod)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught, f"no pin caught: {name}"
