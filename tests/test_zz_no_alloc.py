"""The allocation-free apply (fftmv_apply_scratch) against the applies it
mirrors (fftmv_apply / fftmv_apply_adjoint) and the FP64 oracle, through the
C ABI. Consecutive calls share the library's static device scratch, so the
cases run in sequence: a larger apply, then a smaller one; a scratch left
full of NaN by one plan, then a plan with an odd row width (the padding
entry after its last channel is read by the 16-byte GEMV loads); the
five-kernel form; and an apply too large for the scratch, which is rejected."""
import sys

import numpy as np
import pytest

import oracle
from fft_block_toeplitz_amd import workloads as W
from parity import within

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


def scratch_apply(fm, plan, direction, x):
    n_out = plan.Nd if direction == fm.FFTMV_DIR_F else plan.Nm
    out = torch.full((plan.Nt, n_out), float("nan"), dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    fm.fftmv_apply_scratch(plan.handle, direction, x.data_ptr(), out.data_ptr(), stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_case(fm, Nm, Nd, Nt, mask, tol, m=None, d=None, adjoint=True):
    F = W.operator(Nm, Nd, Nt, 0)
    m = W.input_m(Nm, Nt, 0) if m is None else m
    d = W.input_d(Nd, Nt, 0) if d is None else d
    note(f"no-alloc apply Nm={Nm} Nd={Nd} Nt={Nt} mask={mask:#x}")
    plan = fm.Plan(dev(F), mask)
    m_dev, d_dev = dev(m), dev(d)
    v_ref = plan.apply(m_dev).cpu().numpy()
    w_ref = plan.apply_adjoint(d_dev).cpu().numpy()
    v = scratch_apply(fm, plan, fm.FFTMV_DIR_F, m_dev)
    # same kernels in the same order: the same bits as the plan-workspace applies
    assert np.array_equal(v, v_ref, equal_nan=True)
    if adjoint:
        w = scratch_apply(fm, plan, fm.FFTMV_DIR_FADJ, d_dev)
        assert np.array_equal(w, w_ref, equal_nan=True)
    if adjoint and np.isfinite(m).all() and np.isfinite(d).all():
        Fh = oracle.setup(F)
        okv, ev, _ = within(v, oracle.apply(Fh, m), tol)
        okw, ew, _ = within(w, oracle.apply_adjoint(Fh, d), tol)
        note(f"  rel err vs oracle: F {ev:.2e}, F* {ew:.2e}")
        assert okv and okw
    plan.close()


def test_larger_then_smaller(fm):
    check_case(fm, 4103, 3, 1000, fm.FFTMV_MIXED, 1e-6)
    check_case(fm, 500, 20, 256, fm.FFTMV_ALL_FP64, 1e-11)
    check_case(fm, 37, 5, 20, fm.FFTMV_MIXED, 1e-6)


def test_stale_nan_scratch_then_odd_width(fm):
    """A NaN input fills the scratch spectra with NaN; the next plan (odd Nm,
    whose last 16-byte vector of each spectrum row covers the padding entry)
    must not see it."""
    m = np.full((1000, 700), np.nan)
    check_case(fm, 700, 3, 1000, fm.FFTMV_MIXED, 1e-6, m=m, adjoint=False)  # spectra all NaN
    check_case(fm, 129, 65, 1000, fm.FFTMV_MIXED, 1e-6)
    check_case(fm, 37, 5, 20, fm.FFTMV_MIXED, 1e-6)


def test_five_kernel_form(fm):
    check_case(fm, 129, 65, 1000, fm.FFTMV_MIXED | fm.FFTMV_FLAG_STAGED, 1e-6)
    check_case(fm, 37, 5, 20, fm.FFTMV_ALL_FP64 | fm.FFTMV_FLAG_STAGED, 1e-11)


def test_split_gemv_forms(fm):
    """Tall blocks and few-column rows: the GEMV partial sums live in the
    scratch too."""
    check_case(fm, 5, 4000, 8, fm.FFTMV_MIXED, 1e-6)
    check_case(fm, 20000, 4, 16, fm.FFTMV_MIXED, 1e-6)


def test_too_large_for_the_scratch_is_rejected(fm):
    Nm, Nd, Nt = 20000, 1, 1000  # (Nt+1) x Nm complex64 = 160 MB > 128 MiB
    F = dev(W.operator(Nm, Nd, Nt, 0))
    plan = fm.Plan(F, fm.FFTMV_MIXED)
    m = dev(W.input_m(Nm, Nt, 0))
    v = torch.zeros((Nt, Nd), dtype=torch.float64, device="cuda")
    st = fm.lib().fftmv_apply_scratch(plan.handle, fm.FFTMV_DIR_F, m.data_ptr(), v.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == fm.FFTMV_ERR_UNSUPPORTED_SIZE
    assert fm.lib().fftmv_apply_scratch(plan.handle, 2, m.data_ptr(), v.data_ptr(), None) == \
        fm.FFTMV_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert not v.any()  # nothing was launched
    plan.close()
    # and the library keeps working afterwards
    check_case(fm, 37, 5, 20, fm.FFTMV_MIXED, 1e-6)
