"""Pins for the oracle's condition number of Fhat (CPU only).

Section 1.1 of "Mixed-precision FFTMatvec performance optimization on AMD
GPUs" scales its error bound by kappa(Fhat). These operators have singular
values known in closed form:
  - F_n = delta_{n,0} G: every block Fhat_k equals G;
  - F_n = delta_{n,s} G: Fhat_k = exp(-2 pi i s k / N) G, same singular values;
  - F_n = a_n G with a = (1, r): Fhat_k = (1 + r exp(-pi i k / Nt)) G, whose
    singular values are |1 + r exp(-pi i k / Nt)| times those of G -- largest
    at k = 0 (1 + r), smallest at k = Nt (1 - r);
  - a G with a zero singular value: kappa is infinite.
G = U diag(s) V^T is built from orthonormal U, V and chosen s. A wrong sign
or index in the setup transform, a dropped block or a transposed operand
changes at least one of these values.
"""
import numpy as np
import pytest

import oracle


def known_matrix(rows, cols, s, seed):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((rows, rows)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, cols)))
    S = np.zeros((rows, cols))
    S[np.arange(len(s)), np.arange(len(s))] = s
    return U @ S @ V.T


def operator_from(G, coeffs, Nt):
    F = np.zeros((Nt,) + G.shape)
    for n, a in enumerate(coeffs):
        F[n] = a * G
    return F


@pytest.mark.parametrize("rows,cols", [(4, 9), (9, 4), (5, 5)])
@pytest.mark.parametrize("shift", [0, 3])
def test_single_block_keeps_the_singular_values(rows, cols, shift):
    s = np.array([7.0, 3.0, 2.0, 0.5, 0.25][: min(rows, cols)])
    G = known_matrix(rows, cols, s, seed=rows * 10 + cols)
    Nt = 10
    coeffs = [0.0] * shift + [1.0]
    kappa, smax, smin = oracle.condition(oracle.setup(operator_from(G, coeffs, Nt)))
    assert kappa == pytest.approx(s.max() / s.min(), rel=1e-12)
    np.testing.assert_allclose(smax, s.max(), rtol=1e-12)
    np.testing.assert_allclose(smin, s.min(), rtol=1e-12)


@pytest.mark.parametrize("Nt", [1, 8, 25])
def test_two_term_sequence_closed_form(Nt):
    r = 0.5
    s = np.array([4.0, 1.0, 0.5])
    G = known_matrix(3, 6, s, seed=Nt)
    coeffs = [1.0, r] if Nt > 1 else [1.0]
    kappa, smax, smin = oracle.condition(oracle.setup(operator_from(G, coeffs, Nt)))
    k = np.arange(Nt + 1)
    if Nt > 1:
        scale = np.abs(1.0 + r * np.exp(-1j * np.pi * k / Nt))
        want_kappa = (1 + r) * s.max() / ((1 - r) * s.min())
    else:
        scale = np.ones(Nt + 1)
        want_kappa = s.max() / s.min()
    np.testing.assert_allclose(smax, scale * s.max(), rtol=1e-12)
    np.testing.assert_allclose(smin, scale * s.min(), rtol=1e-12)
    assert kappa == pytest.approx(want_kappa, rel=1e-12)


def test_singular_block_gives_infinite_kappa():
    G = known_matrix(4, 6, np.array([2.0, 1.0, 1.0, 0.0]), seed=5)
    kappa, _, smin = oracle.condition(oracle.setup(operator_from(G, [1.0], 6)))
    assert np.all(smin < 1e-14)
    # rounding leaves tiny nonzero values: kappa is huge or infinite
    assert kappa > 1e13
