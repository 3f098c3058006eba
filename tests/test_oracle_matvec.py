"""Pins for the oracle's five-stage matvec and its frequency blocks (CPU only).

The five-stage FFT path (section 1.1 of "Mixed-precision FFTMatvec
performance optimization on AMD GPUs") is checked against the definition of
the block lower-triangular Toeplitz operator (section 1): the dense matrix
built block by block, the direct double sum, hand-worked values, the adjoint
identity, zero/delta/delay/block-diagonal inputs, Nt = 1 (a plain GEMV) and
Nd = Nm = 1 (numpy.convolve). The frequency blocks are checked against
closed forms and numpy.fft.rfft of the zero-padded series.
"""
import json
import os

import numpy as np
import pytest

import oracle
from fft_block_toeplitz_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _problem(Nm, Nd, Nt, seed=0):
    return (W.operator(Nm, Nd, Nt, seed), W.input_m(Nm, Nt, seed), W.input_d(Nd, Nt, seed))


@pytest.fixture(scope="module")
def small():
    F, m, d = W.problem(W.SMALL)
    return F, m, d, oracle.setup(F)


# ---------------------------------------------------------------- definition
@pytest.mark.parametrize("dims", [(8, 4, 16), (3, 5, 7), (1, 1, 1), (2, 3, 3), (6, 2, 10), (5, 4, 25)])
def test_five_stages_match_dense_product(dims):
    Nm, Nd, Nt = dims
    F, m, d = _problem(Nm, Nd, Nt, seed=sum(dims))
    Fh = oracle.setup(F)
    A = oracle.dense_operator(F)
    v = oracle.apply(Fh, m)
    w = oracle.apply_adjoint(Fh, d)
    assert v.shape == (Nt, Nd) and w.shape == (Nt, Nm)
    assert oracle.rel_l2(v.ravel(), A @ m.ravel()) <= 1e-14
    assert oracle.rel_l2(w.ravel(), A.T @ d.ravel()) <= 1e-14


def test_dense_operator_is_block_lower_triangular():
    F, _, _ = _problem(3, 2, 4)
    A = oracle.dense_operator(F)
    for i in range(4):
        for j in range(4):
            blk = A[i * 2:(i + 1) * 2, j * 3:(j + 1) * 3]
            if j > i:
                assert not blk.any()
            else:
                assert np.array_equal(blk, F[i - j])


def test_direct_matches_dense_product():
    F, m, d = _problem(8, 4, 16)
    A = oracle.dense_operator(F)
    assert oracle.rel_l2(oracle.direct(F, m).ravel(), A @ m.ravel()) <= 1e-15 * 8
    assert oracle.rel_l2(oracle.direct_adjoint(F, d).ravel(), A.T @ d.ravel()) <= 1e-15 * 8
    steps = np.array([7, 0, 15])
    full = oracle.direct(F, m)
    assert np.array_equal(oracle.direct(F, m, steps), full[steps])


def test_worked_examples():
    for ex in json.load(open(GOLDEN))["matvec"]:
        F = np.array(ex["F"], dtype=float)
        Fh = oracle.setup(F)
        m, d = np.array(ex["m"], float), np.array(ex["d"], float)
        assert np.max(np.abs(oracle.apply(Fh, m) - np.array(ex["v"]))) <= 1e-14, ex["name"]
        assert np.max(np.abs(oracle.apply_adjoint(Fh, d) - np.array(ex["w"]))) <= 1e-14, ex["name"]
        assert np.max(np.abs(oracle.direct(F, m) - np.array(ex["v"]))) == 0, ex["name"]
        assert np.max(np.abs(oracle.direct_adjoint(F, d) - np.array(ex["w"]))) == 0, ex["name"]


def test_small_matches_direct_sum(small):
    F, m, d, Fh = small
    assert oracle.rel_l2(oracle.apply(Fh, m), oracle.direct(F, m)) <= 1e-13
    assert oracle.rel_l2(oracle.apply_adjoint(Fh, d), oracle.direct_adjoint(F, d)) <= 1e-13


@pytest.mark.parametrize("shape", ["tiny", "small"])
def test_adjoint_identity(shape, small):
    if shape == "small":
        F, m, d, Fh = small
    else:
        F, m, d = W.problem(W.TINY)
        Fh = oracle.setup(F)
    v = oracle.apply(Fh, m)
    w = oracle.apply_adjoint(Fh, d)
    lhs, rhs = np.vdot(v, d), np.vdot(m, w)
    assert abs(lhs - rhs) <= 1e-14 * np.linalg.norm(v) * np.linalg.norm(d) * 10


# ------------------------------------------------------------ special inputs
def test_zero_input_gives_exact_zero(small):
    F, m, d, Fh = small
    v = oracle.apply(Fh, np.zeros_like(m))
    w = oracle.apply_adjoint(Fh, np.zeros_like(d))
    assert not v.any() and not w.any()
    assert np.isfinite(v).all() and np.isfinite(w).all()


@pytest.mark.parametrize("j0,c0", [(0, 0), (3, 5), (15, 7)])
def test_delta_input_picks_a_column(j0, c0):
    Nm, Nd, Nt = 8, 4, 16
    F, _, _ = _problem(Nm, Nd, Nt)
    Fh = oracle.setup(F)
    m = np.zeros((Nt, Nm))
    m[j0, c0] = 1.0
    v = oracle.apply(Fh, m)
    scale = np.abs(F).max()
    for i in range(Nt):
        ref = F[i - j0][:, c0] if i >= j0 else np.zeros(Nd)
        assert np.max(np.abs(v[i] - ref)) <= 1e-15 * 16 * scale


@pytest.mark.parametrize("i0,r0", [(0, 0), (9, 2), (15, 3)])
def test_delta_adjoint_picks_a_row(i0, r0):
    Nm, Nd, Nt = 8, 4, 16
    F, _, _ = _problem(Nm, Nd, Nt)
    Fh = oracle.setup(F)
    d = np.zeros((Nt, Nd))
    d[i0, r0] = 1.0
    w = oracle.apply_adjoint(Fh, d)
    scale = np.abs(F).max()
    for j in range(Nt):
        ref = F[i0 - j][r0, :] if j <= i0 else np.zeros(Nm)
        assert np.max(np.abs(w[j] - ref)) <= 1e-15 * 16 * scale


def test_single_step_is_a_gemv():
    F, m, d = _problem(37, 11, 1)
    Fh = oracle.setup(F)
    assert oracle.rel_l2(oracle.apply(Fh, m)[0], F[0] @ m[0]) <= 1e-15 * 8
    assert oracle.rel_l2(oracle.apply_adjoint(Fh, d)[0], F[0].T @ d[0]) <= 1e-15 * 8


@pytest.mark.parametrize("Nt", [1, 2, 5, 16, 100, 250])
def test_scalar_blocks_are_a_convolution(Nt):
    F, m, d = _problem(1, 1, Nt, seed=Nt)
    Fh = oracle.setup(F)
    f, x, y = F[:, 0, 0], m[:, 0], d[:, 0]
    assert oracle.rel_l2(oracle.apply(Fh, m)[:, 0], np.convolve(f, x)[:Nt]) <= 1e-14
    # the transpose is the correlation w_j = sum_{i>=j} f_{i-j} y_i
    corr = np.convolve(f[::-1], y)[Nt - 1:]
    assert oracle.rel_l2(oracle.apply_adjoint(Fh, d)[:, 0], corr) <= 1e-14


def test_block_diagonal_operator():
    Nm, Nd, Nt = 6, 3, 20
    F, m, d = _problem(Nm, Nd, Nt)
    F[1:] = 0.0
    Fh = oracle.setup(F)
    assert oracle.rel_l2(oracle.apply(Fh, m), m @ F[0].T) <= 1e-14
    assert oracle.rel_l2(oracle.apply_adjoint(Fh, d), d @ F[0]) <= 1e-14


@pytest.mark.parametrize("s", [1, 4, 19])
def test_pure_delay(s):
    Nm, Nd, Nt = 5, 3, 20
    F, m, d = _problem(Nm, Nd, Nt, seed=s)
    G = F[0].copy()
    F[:] = 0.0
    F[s] = G
    Fh = oracle.setup(F)
    v = oracle.apply(Fh, m)
    ref = np.zeros((Nt, Nd))
    ref[s:] = m[:Nt - s] @ G.T
    assert np.max(np.abs(v - ref)) <= 1e-14 * np.abs(ref).max()
    w = oracle.apply_adjoint(Fh, d)
    refw = np.zeros((Nt, Nm))
    refw[:Nt - s] = d[s:] @ G
    assert np.max(np.abs(w - refw)) <= 1e-14 * np.abs(refw).max()


def test_linearity(small):
    F, m, d, Fh = small
    m2 = np.random.default_rng(5).standard_normal(m.shape)
    a, b = 0.75, -2.5
    lhs = oracle.apply(Fh, a * m + b * m2)
    rhs = a * oracle.apply(Fh, m) + b * oracle.apply(Fh, m2)
    assert oracle.rel_l2(lhs, rhs) <= 1e-14


# --------------------------------------------------------- frequency blocks
def test_fhat_closed_forms(small):
    F, _, _, Fh = small
    Nt = F.shape[0]
    assert Fh.shape == (Nt + 1, F.shape[1], F.shape[2])
    sign = (-1.0) ** np.arange(Nt)
    assert oracle.rel_l2(Fh[0], F.sum(axis=0)) <= 1e-14
    assert oracle.rel_l2(Fh[Nt], np.tensordot(sign, F, axes=1)) <= 1e-14
    assert np.max(np.abs(Fh[0].imag)) <= 1e-14 and np.max(np.abs(Fh[Nt].imag)) <= 1e-13


def test_fhat_matches_numpy_rfft(small):
    F, _, _, Fh = small
    Nt = F.shape[0]
    ref = np.fft.rfft(F, n=2 * Nt, axis=0)
    assert oracle.rel_l2(Fh, ref) <= 1e-14


def test_fhat_worked_example():
    for ex in json.load(open(GOLDEN))["fhat"]:
        Fh = oracle.setup(np.array(ex["F"], float))
        ref = np.array(ex["Fhat_re"]) + 1j * np.array(ex["Fhat_im"])
        assert np.max(np.abs(Fh[:, 0, 0] - ref)) <= 1e-15 * 4, ex["name"]


def test_stage_dumps(small):
    F, m, d, Fh = small
    Nt = F.shape[0]
    v, mh, vh = oracle.apply(Fh, m, dumps=True)
    assert oracle.rel_l2(mh, np.fft.rfft(m, n=2 * Nt, axis=0)) <= 1e-14
    assert oracle.rel_l2(vh, np.einsum("krc,kc->kr", Fh, mh)) <= 1e-14
    assert oracle.rel_l2(v, np.fft.irfft(vh, n=2 * Nt, axis=0)[:Nt]) <= 1e-14
    w, dh, wh = oracle.apply_adjoint(Fh, d, dumps=True)
    assert oracle.rel_l2(dh, np.fft.rfft(d, n=2 * Nt, axis=0)) <= 1e-14
    assert oracle.rel_l2(wh, np.einsum("krc,kr->kc", Fh.conj(), dh)) <= 1e-14
    assert oracle.rel_l2(w, np.fft.irfft(wh, n=2 * Nt, axis=0)[:Nt]) <= 1e-14


def test_inverse_ignores_imaginary_dc_and_nyquist():
    """The inverse rebuilds a real signal: imaginary parts of bins 0 and Nt
    must not change the result (they are zero in exact arithmetic)."""
    Nm, Nd, Nt = 4, 3, 8
    F, m, _ = _problem(Nm, Nd, Nt)
    Fh = oracle.setup(F)
    Fh2 = Fh.copy()
    Fh2[0] += 1j * 0.5
    Fh2[Nt] += 1j * 0.25
    # Fhat_0 and Fhat_Nt multiply real spectra of m at those bins, so the
    # products gain imaginary parts only; v must not move.
    assert oracle.rel_l2(oracle.apply(Fh2, m), oracle.apply(Fh, m)) <= 1e-15 * 8


def test_rejects_bad_arguments():
    with pytest.raises(RuntimeError):
        oracle.direct(np.zeros((2, 1, 1)), np.zeros((2, 1)), steps=[2])


# ------------------------------------------------------------ full size
@pytest.mark.slow
def test_main_spot_steps_match_direct_sum():
    """Main shape (Nm=5000, Nd=100, Nt=1000): the five stages against the
    direct sum at spot time steps, and the adjoint identity."""
    F, m, d = W.problem(W.MAIN)
    Fh = oracle.setup(F)
    steps = np.array([0, 1, 500, 998, 999])
    v = oracle.apply(Fh, m)
    assert oracle.rel_l2(v[steps], oracle.direct(F, m, steps)) <= 1e-13
    wsteps = np.array([0, 1, 500, 999])
    w = oracle.apply_adjoint(Fh, d)
    assert oracle.rel_l2(w[wsteps], oracle.direct_adjoint(F, d, wsteps)) <= 1e-13
    lhs, rhs = np.vdot(v, d), np.vdot(m, w)
    assert abs(lhs - rhs) <= 1e-13 * np.linalg.norm(v) * np.linalg.norm(d)
