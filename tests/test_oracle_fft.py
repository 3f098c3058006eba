"""Pins for the oracle's own FFT (CPU only).

The oracle's recursive mixed-radix FFT is checked against things it does not
share code with: a textbook O(N^2) DFT with exact integer reduction of the
exponent, numpy.fft (a library routine), closed forms, Parseval's identity
and hand-worked values.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
SIZES = [1, 2, 3, 4, 5, 7, 8, 10, 16, 25, 32, 125, 512, 1000, 2000, 4000]


def _rand(n, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(n) + 1j * g.standard_normal(n)


def _textbook_dft(x, sign):
    n = x.size
    jk = np.outer(np.arange(n), np.arange(n)) % n  # exact integer reduction
    W = np.exp(sign * 2j * np.pi * jk / n)
    return W @ x


@pytest.mark.parametrize("n", [s for s in SIZES if s <= 1000])
@pytest.mark.parametrize("sign", [-1, 1])
def test_fft_matches_textbook_dft(n, sign):
    x = _rand(n, n)
    assert oracle.rel_l2(oracle.fft(x, sign), _textbook_dft(x, sign)) <= 1e-13


@pytest.mark.parametrize("n", SIZES)
def test_fft_matches_numpy(n):
    x = _rand(n, 100 + n)
    assert oracle.rel_l2(oracle.fft(x, -1), np.fft.fft(x)) <= 1e-14
    assert oracle.rel_l2(oracle.fft(x, +1), np.fft.ifft(x) * n) <= 1e-14


@pytest.mark.parametrize("n", [8, 10, 125, 2000])
def test_fft_closed_forms(n):
    k = np.arange(n)
    # unit impulse at p -> exp(-2 pi i k p / n)
    p = 3 % n
    x = np.zeros(n, complex)
    x[p] = 1
    assert np.max(np.abs(oracle.fft(x) - np.exp(-2j * np.pi * ((k * p) % n) / n))) <= 1e-14
    # constant -> n at k = 0
    X = oracle.fft(np.ones(n, complex))
    ref = np.zeros(n, complex)
    ref[0] = n
    assert np.max(np.abs(X - ref)) <= 1e-12
    # (-1)^n -> n at k = n/2 (even n only)
    if n % 2 == 0:
        X = oracle.fft((-1.0) ** k + 0j)
        ref = np.zeros(n, complex)
        ref[n // 2] = n
        assert np.max(np.abs(X - ref)) <= 1e-12
    # cos(2 pi k0 n / N) -> n/2 at k0 and N-k0
    k0 = 1
    X = oracle.fft(np.cos(2 * np.pi * k0 * k / n) + 0j)
    ref = np.zeros(n, complex)
    ref[k0] += n / 2
    ref[n - k0] += n / 2
    assert np.max(np.abs(X - ref)) <= 1e-11


@pytest.mark.parametrize("n", [5, 512, 2000])
def test_fft_parseval_and_round_trip(n):
    x = _rand(n, 7 * n)
    X = oracle.fft(x)
    assert abs(np.vdot(X, X).real / n - np.vdot(x, x).real) <= 1e-12 * np.vdot(x, x).real
    back = oracle.fft(X, +1) / n
    assert oracle.rel_l2(back, x) <= 1e-15 * 4


@pytest.mark.parametrize("n", [16, 1000])
def test_fft_hermitian_for_real_input(n):
    x = np.random.default_rng(n).standard_normal(n) + 0j
    X = oracle.fft(x)
    k = np.arange(1, n)
    assert np.max(np.abs(X[k] - np.conj(X[n - k]))) <= 1e-12
    assert abs(X[0].imag) <= 1e-13


def test_fft_worked_examples():
    for ex in json.load(open(GOLDEN))["dft"]:
        x = np.array(ex["x_re"]) + 1j * np.array(ex["x_im"])
        X = np.array(ex["X_re"]) + 1j * np.array(ex["X_im"])
        assert np.max(np.abs(oracle.fft(x) - X)) <= 1e-15 * 8, ex["name"]


def test_fft_rejects_bad_arguments():
    with pytest.raises(RuntimeError):
        oracle.fft(np.zeros(4, complex), sign=0)
