"""GPU parity of the precision-selection inputs ("Mixed-precision FFTMatvec
performance optimization on AMD GPUs", sections 1.1, 2.1, 2.2):

  - fftmv_condition (Lanczos on each frequency's Gram matrix, on the device)
    against the oracle's SVD of every Fhat_k, on random operators and on
    operators with singular values known in closed form;
  - the 32-configuration sweep: the errors it measures against the plan's
    own all-FP64 apply agree with the errors against the oracle, and its
    measured Pareto front is non-dominated.

Tolerances: with iters >= n the Lanczos values are the Gram matrix's up to
rounding, so s_min is resolved to about u * s_max^2 / s_min (u the unit
roundoff of the Fhat copy used): 1e-8 relative with complex128 at the
condition numbers here, 1e-4 with complex64 only.
"""
import sys

import numpy as np
import pytest

import oracle
from fft_block_toeplitz_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fft_block_toeplitz_amd as fm

    fm.lib()
    return fm


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


SHAPES = [(8, 4, 16), (37, 5, 20), (500, 20, 256), (2, 130, 40), (129, 65, 1000), (3, 3, 125)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mask,rtol", [(0x000, 1e-8), (0x186, 1e-4)])
def test_condition_matches_oracle_svd(fm, shape, mask, rtol):
    Nm, Nd, Nt = shape
    F = W.operator(Nm, Nd, Nt, 3)
    kappa_ref, smax_ref, smin_ref = oracle.condition(oracle.setup(F))
    note(f"condition shape={shape} mask={mask:#x}")
    plan = fm.Plan(dev(F), mask)
    kappa, smax, smin = plan.condition()
    plan.close()
    note(f"  kappa {kappa:.6g} (oracle {kappa_ref:.6g})")
    np.testing.assert_allclose(smax, smax_ref, rtol=rtol)
    np.testing.assert_allclose(smin, smin_ref, rtol=rtol)
    assert kappa == pytest.approx(kappa_ref, rel=rtol)


def _known(rows, cols, s, seed):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((rows, rows)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, cols)))
    S = np.zeros((rows, cols))
    S[np.arange(len(s)), np.arange(len(s))] = s
    return U @ S @ V.T


@pytest.mark.parametrize("rows,cols", [(6, 40), (40, 6)])
def test_condition_closed_form(fm, rows, cols):
    """F_n = a_n G with a = (1, r): kappa = (1 + r) s_max / ((1 - r) s_min)."""
    Nt, r = 20, 0.5
    s = np.array([50.0, 9.0, 4.0, 2.0, 1.5, 1.0])
    G = _known(rows, cols, s, seed=rows)
    F = np.zeros((Nt, rows, cols))
    F[0], F[1] = G, r * G
    plan = fm.Plan(dev(F), 0x000)
    kappa, smax, smin = plan.condition()
    plan.close()
    k = np.arange(Nt + 1)
    scale = np.abs(1.0 + r * np.exp(-1j * np.pi * k / Nt))
    np.testing.assert_allclose(smax, scale * 50.0, rtol=1e-9)
    np.testing.assert_allclose(smin, scale * 1.0, rtol=1e-8)
    assert kappa == pytest.approx(3.0 * 50.0, rel=1e-8)


def test_condition_with_few_steps_brackets_the_extremes(fm):
    Nm, Nd, Nt = 300, 60, 40
    F = W.operator(Nm, Nd, Nt, 4)
    kappa_ref, smax_ref, smin_ref = oracle.condition(oracle.setup(F))
    plan = fm.Plan(dev(F), 0x000)
    kappa, smax, smin = plan.condition(iters=12)
    plan.close()
    # Ritz values lie inside the spectrum
    assert np.all(np.asarray(smax) <= smax_ref * (1 + 1e-10))
    assert np.all(np.asarray(smin) >= smin_ref * (1 - 1e-10))
    assert kappa <= kappa_ref * (1 + 1e-10)
    # and the largest is already within a few percent after 12 steps (this
    # spectrum has no gap at its top edge, so convergence is slow)
    np.testing.assert_allclose(smax, smax_ref, rtol=5e-2)


def test_condition_singular_block(fm):
    G = _known(4, 6, np.array([2.0, 1.0, 1.0, 0.0]), seed=9)
    F = np.zeros((5, 4, 6))  # 2 Nt = 10
    F[0] = G
    plan = fm.Plan(dev(F), 0x000)
    kappa, _, smin = plan.condition()
    plan.close()
    # the zero singular value is resolved to about sqrt(u) s_max
    assert kappa > 1e6 and max(smin) < 1e-6


def test_sweep_errors_match_the_oracle(fm):
    from fft_block_toeplitz_amd import precision

    Nm, Nd, Nt = 37, 5, 1000
    F, m, d = W.operator(Nm, Nd, Nt, 0), W.input_m(Nm, Nt, 0), W.input_d(Nd, Nt, 0)
    Fh = oracle.setup(F)
    v_ref, w_ref = oracle.apply(Fh, m), oracle.apply_adjoint(Fh, d)
    records, kappa = precision.sweep(dev(F), dev(m), dev(d), reps=2, warmup=1)
    assert len(records) == 64
    plan = fm.Plan(dev(F), fm.FFTMV_FLAG_FHAT_BOTH)
    worst = 0.0
    for r in records:
        plan.set_mask(r["bits"] << (5 * r["direction"]))
        if r["direction"] == 0:
            got, ref = plan.apply(dev(m)), v_ref
        else:
            got, ref = plan.apply_adjoint(dev(d)), w_ref
        torch.cuda.synchronize()
        e = oracle.rel_l2(got.cpu().numpy(), ref)
        # against the oracle the all-FP64 apply is within 1e-11; the sweep's
        # FP64 reference shifts the others by at most that much
        assert abs(e - r["error"]) <= 1e-11 + 1e-6 * e, (r, e)
        worst = max(worst, e)
    plan.close()
    note(f"sweep at {Nm}x{Nd}x{Nt}: kappa {kappa:.4g}, worst FP32 error {worst:.3e}")
    for direction in (0, 1):
        front = precision.measured_front(records, direction)
        assert front and front[0]["ms"] == min(r["ms"] for r in records if r["direction"] == direction)
        for a in front:
            for b in records:
                if b["direction"] == direction:
                    assert not (b["ms"] <= a["ms"] and b["error"] <= a["error"]
                                and (b["ms"] < a["ms"] or b["error"] < a["error"]))
        params = precision.fit_params(records, Nm, Nd, Nt, kappa, direction)
        # the fitted bound covers every measured configuration
        for r in records:
            if r["direction"] == direction and r["bits"]:
                pred, _ = fm.fftmv_predict(Nm, Nd, Nt, direction, r["bits"], 0, kappa, params)
                assert pred >= r["error"] * (1 - 1e-12)
