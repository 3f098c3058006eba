"""The index scheme of the setup transform's decimation-in-frequency kernel
(fft_block_toeplitz_amd/csrc/fft_setup.hip), restated in numpy and checked
against numpy's real FFT of the zero-padded series ("Mixed-precision
FFTMatvec performance optimization on AMD GPUs", section 1.1: the frequency
blocks are the transforms of every series padded to 2 Nt).

The kernel writes L = Nt = R1 * 125, packs z[n] = x[2n] + i x[2n+1], takes
one decimation-in-frequency step into R1 sub-transforms of 125 points, works
through the slots in mirror-closed groups {0, R1/2}, {g, R1 - g}, and emits
each bin k together with its mirror L - k. This test walks the same rounds,
items and indices and checks that every bin 0..L comes out exactly once and
equals the reference. No GPU, no library code."""
import numpy as np
import pytest

SUB = 125


def decomposed_rfft(x, L, NSL):
    R1 = L // SUB
    H, NG = R1 // 2, R1 // 2
    tw = np.exp(-2j * np.pi * np.arange(2 * L) / (2 * L))  # w_2L^t
    z = np.zeros(L, complex)
    z[: L // 2] = x[0::2] + 1j * x[1::2]
    n2 = np.arange(SUB)
    zz = np.stack([z[n2 + SUB * n1] for n1 in range(H)])  # only n1 < R1/2 are nonzero
    assert not z[SUB * H:].any()
    X = np.full(L + 1, np.nan + 0j)
    for r in range(NG // (NSL // 2)):
        slots = {}
        for gi in range(NSL // 2):
            g = r * (NSL // 2) + gi
            if g == 0:  # slots 0 and R1/2
                A = zz.sum(0)
                B = (zz * ((-1.0) ** np.arange(H))[:, None]).sum(0)
                ya, yb = A, B * tw[n2 * R1]
            else:  # slots g and R1 - g
                w = np.array([tw[(2 * L // R1) * ((n1 * g) % R1)] for n1 in range(H)])[:, None]
                ya = (zz * w).sum(0) * tw[2 * n2 * g]
                yb = (zz * np.conj(w)).sum(0) * tw[2 * n2 * (R1 - g)]
            slots[2 * gi], slots[2 * gi + 1] = np.fft.fft(ya), np.fft.fft(yb)
        nitems = (NSL // 2) * SUB + (1 if r == 0 else 0)
        for it in range(nitems):
            if r == 0 and it < 2 * 63:
                if it < 63:
                    sla = slb = 0
                    k2a, k2b, k = it, (0 if it == 0 else SUB - it), R1 * it
                else:
                    sla = slb = 1
                    k2a = it - 63
                    k2b, k = SUB - 1 - k2a, R1 // 2 + R1 * k2a
            else:
                it2 = it - 1 if r == 0 else it
                gi = it2 // SUB
                k2a = it2 - gi * SUB
                sla, slb = 2 * gi, 2 * gi + 1
                k2b, k = SUB - 1 - k2a, r * (NSL // 2) + gi + R1 * k2a
            za, zb = slots[sla][k2a], np.conj(slots[slb][k2b])
            ev, dd = (za + zb) * 0.5, za - zb
            t = (dd.imag * 0.5 - 1j * dd.real * 0.5) * tw[k]
            out = [(k, ev + t)] + ([(L - k, np.conj(ev - t))] if 2 * k != L else [])  # bin L/2 pairs with itself
            for kk, val in out:
                assert np.isnan(X[kk]), f"bin {kk} written twice"
                X[kk] = val
    assert not np.isnan(X).any(), "a bin was never written"
    return X


@pytest.mark.parametrize("L,NSL", [(1000, 2), (1000, 4), (1000, 8), (2000, 2), (2000, 4), (2000, 16)])
def test_decomposition_matches_rfft(L, NSL):
    rng = np.random.default_rng(L + NSL)
    for _ in range(3):
        x = rng.standard_normal(L)
        got = decomposed_rfft(x, L, NSL)
        ref = np.fft.rfft(x, 2 * L)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_decomposition_delta_and_constant():
    # closed forms: a unit impulse at t = 0 has every bin 1; a constant
    # series of length L has bin 0 equal to L
    L = 1000
    x = np.zeros(L)
    x[0] = 1.0
    assert np.allclose(decomposed_rfft(x, L, 2), np.ones(L + 1), atol=1e-13)
    got = decomposed_rfft(np.ones(L), L, 4)
    assert abs(got[0] - L) < 1e-10
