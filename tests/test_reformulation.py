"""The algebra behind the GPU path's Gram-space head, checked exactly in fp64.

The HIP library runs the first iterations of the quintic Newton-Schulz
iteration (Notes on Muon blog, "Newton-Schulz") for matrices with n >= 2 m in
the m x m Gram space: with A0 = X0 X0^T and P_j = a I + b A_j + c A_j^2, every
iterate is X_j = (P_{j-1} .. P_0) X0 and its Gram matrix is
A_{j+1} = P_j A_j P_j, so the n-sized products reduce to one apply. The
accumulated product is kept shifted, R_j = P_j .. P_0 - a^{j+1} I, formed as
R_1 = P_1 P_0 - a^2 I and R_j = P_j R_{j-1} + a^j P_j - a^{j+1} I, and
X_k = R_{k-1} X0 + a^k X0. These tests restate that recurrence in numpy fp64
and require it to reproduce the oracle's iteration to rounding, so a wrong
term in the recurrence the kernels implement fails here on the CPU; a planted
wrong term must fail the same check. The GPU parity tests then compare the
kernels with the oracle at the bf16 tolerance.
"""
import numpy as np
import pytest

import oracle

A_, B_, C_ = oracle.NS_A, oracle.NS_B, oracle.NS_C


def _normalised_wide(m):
    x = m / (np.linalg.norm(m) + oracle.NS_EPS)
    return (x.T if x.shape[0] > x.shape[1] else x), x.shape[0] > x.shape[1]


def _poly(a_mat):
    return A_ * np.eye(a_mat.shape[0]) + B_ * a_mat + C_ * (a_mat @ a_mat)


def _head(x0, k, drop_term=False):
    """X_k through the shifted Gram-space recurrence (k >= 2)."""
    eye = np.eye(x0.shape[0])
    a_mat = x0 @ x0.T
    p0 = _poly(a_mat)
    a_mat = p0 @ (a_mat @ p0)                       # A_1
    p = _poly(a_mat)                                 # P_1
    r = p @ p0 - A_ ** 2 * eye                       # R_1
    for j in range(2, k):
        a_mat = p @ (a_mat @ p)                      # A_j
        p = _poly(a_mat)                             # P_j
        r = p @ r + (0.0 if drop_term else A_ ** j) * p - A_ ** (j + 1) * eye
    return r @ x0 + A_ ** k * x0


def _x_space(x, steps):
    for _ in range(steps):
        g = x @ x.T
        x = A_ * x + (B_ * g + C_ * (g @ g)) @ x
    return x


@pytest.mark.parametrize("shape", [(24, 80), (80, 24), (40, 96), (33, 70)])
@pytest.mark.parametrize("k", [2, 3])
def test_head_then_x_space_equals_the_iteration(shape, k):
    rng = np.random.default_rng(100 + k + shape[0])
    m = rng.standard_normal(shape)
    x0, tall = _normalised_wide(m)
    xk = _head(x0, k)
    got = _x_space(xk, oracle.NS_STEPS - k)
    want = oracle.newton_schulz(m)
    want = want.T if tall else want
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)
    # the head alone is k plain iterations
    want_k = oracle.newton_schulz(m, steps=k)
    want_k = want_k.T if tall else want_k
    assert np.linalg.norm(xk - want_k) <= 1e-12 * np.linalg.norm(want_k)


def test_head_on_a_decaying_spectrum():
    """Singular values spread over three decades: the identity holds for every
    direction, the small ones (where Q is close to a^k I) included."""
    rng = np.random.default_rng(7)
    u, _ = np.linalg.qr(rng.standard_normal((32, 32)))
    v, _ = np.linalg.qr(rng.standard_normal((90, 32)))
    m = (u * np.logspace(0, -3, 32)) @ v.T
    x0, _ = _normalised_wide(m)
    got = _x_space(_head(x0, 3), 2)
    want = oracle.newton_schulz(m)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


def test_planted_wrong_term_fails():
    """Without the a^j P_j term of R_j (j >= 2) the recurrence no longer
    forms P_j Q_{j-1}, and the check above must see it."""
    rng = np.random.default_rng(3)
    m = rng.standard_normal((24, 80))
    x0, _ = _normalised_wide(m)
    want = oracle.newton_schulz(m, steps=3)
    bad = _head(x0, 3, drop_term=True)
    assert np.linalg.norm(bad - want) > 1e-3 * np.linalg.norm(want)
