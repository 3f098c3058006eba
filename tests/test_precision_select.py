"""Host-side precision selection (no GPU): the error predictor, the
performance predictor and the Pareto search of "Mixed-precision FFTMatvec
performance optimization on AMD GPUs", sections 1.1, 2.1 and 2.2, through
the C ABI.

Pins: hand-worked predictor values, the byte model against bench.py's own
algorithmic byte count, the Pareto front against its definition by brute
force over all 32 configurations, and monotonicity in each stage's
precision.
"""
import itertools
import math

import pytest

import bench
import fft_block_toeplitz_amd as fm

U32, U64 = 2.0 ** -24, 2.0 ** -53
INF = math.inf
PARAMS = [1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 1e12, 1e13, 1e-6]
HBM_ONLY = PARAMS[:7] + [INF, 1e-6]  # LDS term switched off


def test_defaults_are_usable():
    for direction in (0, 1):
        p = fm.fftmv_model_defaults(direction)
        assert len(p) == fm.FFTMV_MODEL_PARAMS
        assert all(x >= 0 for x in p) and p[6] > 0 and p[7] > 0 and math.isfinite(p[8])


def test_error_predictor_hand_worked():
    # Nm=10, Nd=4, Nt=8 (log2 Nt = 3), F, only stage 3 in FP32, kappa = 2:
    # 2 * [1 u64 + (6 u64 + 2 u64 + 4 u64) * 3 + 3 u32 * 10 + 5 u64]
    #   = 2 * [42 u64 + 30 u32]
    err, _ = fm.fftmv_predict(10, 4, 8, 0, 0b00100, 0, 2.0, PARAMS)
    assert err == pytest.approx(2 * (42 * U64 + 30 * U32), rel=1e-14)
    # the same for F*: the inner length is Nd = 4 -> 3 u32 * 4
    err, _ = fm.fftmv_predict(10, 4, 8, 1, 0b00100, 0, 2.0, PARAMS)
    assert err == pytest.approx(2 * (42 * U64 + 12 * U32), rel=1e-14)
    # all FP32: 2 * [1 u32 + (6 u64 + 2 u32 + 4 u32) * 3 + 30 u32 + 5 u32]
    err, _ = fm.fftmv_predict(10, 4, 8, 0, 0b11111, 0, 2.0, PARAMS)
    assert err == pytest.approx(2 * (18 * U64 + 54 * U32), rel=1e-14)


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("bits", [0b00000, 0b00110, 0b01100, 0b11111, 0b10001])
def test_time_model_is_the_algorithmic_byte_count(direction, bits):
    Nm, Nd, Nt = 5000, 100, 1000
    _, sec = fm.fftmv_predict(Nm, Nd, Nt, direction, bits, 0, 1.0, HBM_ONLY)
    mask = bits << (5 * direction)
    want = bench.apply_bytes(Nm, Nd, Nt, mask, direction) / HBM_ONLY[6] + 3 * HBM_ONLY[8]
    assert sec == pytest.approx(want, rel=1e-12)


def test_lds_term_hand_worked():
    # Nt = 1000 = 2^3 5^3: radix passes 8, 5, 5, 5. Each writes and reads the
    # tile: 2 * 4 * 1000 * (5000 channels * 16 B + 100 * 16 B) = 652.8 MB for
    # F in FP64; an FP32 forward FFT halves the 5000-channel part.
    lds_only = PARAMS[:6] + [INF, 1.0, 0.0]
    _, b = fm.fftmv_predict(5000, 100, 1000, 0, 0b00000, 0, 1.0, lds_only)
    assert b == pytest.approx(652.8e6, rel=1e-14)
    _, b = fm.fftmv_predict(5000, 100, 1000, 0, 0b00010, 0, 1.0, lds_only)
    assert b == pytest.approx(332.8e6, rel=1e-14)
    # F*: the inverse FFT has the 5000 channels
    _, b = fm.fftmv_predict(5000, 100, 1000, 1, 0b01000, 0, 1.0, lds_only)
    assert b == pytest.approx(332.8e6, rel=1e-14)


def test_staged_model_adds_the_pad_and_unpad_passes():
    Nm, Nd, Nt = 5000, 100, 1000
    # F, all FP64: pad reads and writes Nt*Nm*8, the FFT reads that buffer
    # instead of m; unpad reads and writes Nt*Nd*8
    _, fused = fm.fftmv_predict(Nm, Nd, Nt, 0, 0, 0, 1.0, PARAMS)
    _, staged = fm.fftmv_predict(Nm, Nd, Nt, 0, 0, fm.FFTMV_FLAG_STAGED, 1.0, PARAMS)
    extra = (2 * Nt * Nm * 8 + 2 * Nt * Nd * 8) / PARAMS[6] + 2 * PARAMS[8]
    assert staged - fused == pytest.approx(extra, rel=1e-12)


def _all(Nm, Nd, Nt, direction, flags, kappa, params):
    return {b: fm.fftmv_predict(Nm, Nd, Nt, direction, b, flags, kappa, params) for b in range(32)}


def _front_by_definition(pred, tol):
    feas = {b: v for b, v in pred.items() if v[0] <= tol}
    front = set()
    for b, (e, t) in feas.items():
        dominated = any((t2 <= t and e2 <= e and (t2 < t or e2 < e)) for b2, (e2, t2) in feas.items() if b2 != b)
        if not dominated:
            front.add((e, t))
    return front


@pytest.mark.parametrize("direction,flags,kappa", [(0, 0, 1.0), (1, 0, 3.0), (0, fm.FFTMV_FLAG_STAGED, 10.0)])
@pytest.mark.parametrize("tol", [1e-14, 1e-10, 1e-7, 1e-6, 1e-4, 1.0])
def test_pareto_front_by_brute_force(direction, flags, kappa, tol):
    for params in (PARAMS, None):
        shape = (5000, 100, 1000)
        pred = _all(*shape, direction, flags, kappa, params)
        front = fm.fftmv_pareto_front(*shape, direction, flags, kappa, tol, params)
        # one representative per distinct (error, time) point of the front
        assert {pred[b] for b in front} == _front_by_definition(pred, tol)
        assert len(front) == len({pred[b] for b in front})
        times = [pred[b][1] for b in front]
        assert times == sorted(times)
        bits, err, sec, ok = fm.fftmv_select_precision(*shape, direction, flags, kappa, tol, params)
        if front:
            assert ok and bits == front[0]
            assert sec == min(t for e, t in pred.values() if e <= tol)
            assert (err, sec) == pred[bits]
        else:
            assert not ok and bits == 0 and (err, sec) == pred[0]


def test_ffts_next_to_an_fp32_sbgemv_save_only_lds_time():
    # buffers hold the narrower precision of their two stages: once stage 3
    # is FP32 both spectra are complex64 whatever stages 2 and 4 use; FP32
    # FFTs then save only their LDS traffic
    for params, want in ((HBM_ONLY, 0b00100), (PARAMS, 0b01110)):
        _, t3 = fm.fftmv_predict(5000, 100, 1000, 0, 0b00100, 0, 1.0, params)
        _, t234 = fm.fftmv_predict(5000, 100, 1000, 0, 0b01110, 0, 1.0, params)
        assert (t3 == t234) if params is HBM_ONLY else (t234 < t3)
        bits, _, _, ok = fm.fftmv_select_precision(5000, 100, 1000, 0, 0, 1.0, 1.0, params)
        assert ok and bits == want


def test_ties_prefer_fewer_fp32_stages():
    # with c1 = c5 = 0 stages 1 and 5 cost neither time (fused form) nor
    # error in FP32: equal candidates, and the one with fewer FP32 stages wins
    params = [0.0, 2.0, 3.0, 4.0, 0.0, 6.0, 1e12, INF, 1e-6]  # no LDS term
    e1, t1 = fm.fftmv_predict(5000, 100, 1000, 0, 0b00100, 0, 1.0, params)
    e2, t2 = fm.fftmv_predict(5000, 100, 1000, 0, 0b10101, 0, 1.0, params)
    assert (e1, t1) == (e2, t2)
    bits, _, _, ok = fm.fftmv_select_precision(5000, 100, 1000, 0, 0, 1.0, 1.0, params)
    assert ok and bits == 0b00100


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("flags", [0, fm.FFTMV_FLAG_STAGED])
def test_fp32_never_adds_time_or_removes_error(direction, flags):
    pred = _all(500, 20, 256, direction, flags, 2.0, PARAMS)
    for b, s in itertools.product(range(32), range(5)):
        if not b & (1 << s):
            e0, t0 = pred[b]
            e1, t1 = pred[b | (1 << s)]
            assert e1 > e0 and t1 <= t0


@pytest.mark.parametrize("args", [
    dict(Nm=0), dict(direction=2), dict(bits=32), dict(kappa=0.5), dict(kappa=float("nan")),
    dict(flags=1 << 20), dict(params=[1, 1, 1, 1, 1, 1, 0, 1, 0]), dict(params=[-1, 1, 1, 1, 1, 1, 1e12, 1, 0]),
    dict(params=[1, 1, 1, 1, 1, 1, 1e12, 1e13, INF]),
])
def test_invalid_arguments(args):
    a = dict(Nm=10, Nd=4, Nt=8, direction=0, bits=0, flags=0, kappa=1.0, params=None)
    a.update(args)
    with pytest.raises(fm.FftmvError) as e:
        fm.fftmv_predict(a["Nm"], a["Nd"], a["Nt"], a["direction"], a["bits"], a["flags"], a["kappa"],
                         a["params"])
    assert e.value.status == fm.FFTMV_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        fm.fftmv_predict(10, 4, 8, 0, 0, 0, 1.0, [1.0] * 8)


@pytest.mark.parametrize("Nt", [2053, 3001, 4093, 4097])
def test_unsupported_lengths(Nt):
    with pytest.raises(fm.FftmvError) as e:
        fm.fftmv_predict(10, 4, Nt, 0, 0, 0, 1.0)
    assert e.value.status == fm.FFTMV_ERR_UNSUPPORTED_SIZE
    with pytest.raises(fm.FftmvError):
        fm.fftmv_select_precision(10, 4, Nt, 0, 0, 1.0, 1e-6)


def test_every_smooth_length_up_to_4096_is_supported():
    """Nt = 2^a 3^b 5^c 7^d <= 4096 has a radix schedule that fits a
    workgroup (the longest radix-7 ones in 1024-thread workgroups), and a
    prime up to 2048 has a Bluestein tile."""
    def smooth(n):
        for p in (2, 3, 5, 7):
            while n % p == 0:
                n //= p
        return n == 1

    lengths = [n for n in range(1, 4097) if smooth(n)] + [2039, 2027, 1009, 11]
    for Nt in lengths:
        fm.fftmv_predict(10, 4, Nt, 0, 0, 0, 1.0)  # raises if unsupported
