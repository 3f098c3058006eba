"""Pareto analysis over the 32 stage configurations of each direction
("Mixed-precision FFTMatvec performance optimization on AMD GPUs", sections
1.2 and 2.2), and the fit of the model parameters that fftmv_select_precision
(section 2.1) predicts with.

For every configuration the sweep measures, on one plan holding Fhat in both
precisions, the apply time (HIP events, after warm-up) and the relative L2
error of the output against the same plan's all-FP64 apply. That reference
is itself within ~1e-14 of an FP64 definition of the operator, far below
any FP32 configuration's error, so the reference's own error does not enter
the sweep's figures.

The fit (`fit_params`) follows the bound of section 1.1 term by term: c_s
from the configuration with stage s alone in FP32 (its error above the
all-FP64 one, divided by kappa u32 times the stage's growth factor: 1,
log2 Nt, n, log2 Nt, 1), cF left at 1 (the all-FP64 configuration is the
sweep's reference, so its own error is not measured here; the FP64 terms
are ~1e-14 and do not decide any selection), then every constant scaled up by the largest measured / predicted ratio over the sweep so that
the model bounds every measured configuration. The bandwidths B (HBM) and
B_lds and the per-kernel time t0 are the non-negative least-squares fit of
the measured times to hbm_bytes / B + lds_bytes / B_lds + kernels * t0.

Run: python -m fft_block_toeplitz_amd.precision [--shape main] [--reps 20]
prints a markdown table, the measured Pareto fronts and the fitted
parameters (one GPU).
"""

from __future__ import annotations

import argparse
import json
import math
import sys

import numpy as np

import fft_block_toeplitz_amd as fm

U32, U64 = 2.0 ** -24, 2.0 ** -53
STAGES = ("pad", "fft", "sbgemv", "ifft", "unpad")


def describe(bits: int) -> str:
    """Stage precisions as a string, e.g. '64 32 32 64 64'."""
    return " ".join("32" if bits & (1 << s) else "64" for s in range(5))


def _rel(a, ref) -> float:
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def sweep(F_dev, m_dev, d_dev, reps: int = 20, warmup: int = 5, staged: bool = False,
          directions=(0, 1), iters: int = 0, log=None):
    """Time and error of all 32 configurations of each direction.

    Returns (records, kappa): records are dicts with direction, bits,
    error, ms (mean apply time)."""
    import torch

    flags = fm.FFTMV_FLAG_FHAT_BOTH | (fm.FFTMV_FLAG_STAGED if staged else 0)
    plan = fm.Plan(F_dev, fm.FFTMV_ALL_FP64 | flags)
    try:
        import time

        t0 = time.perf_counter()
        kappa, _, _ = plan.condition(iters)
        if log:
            log(f"kappa(Fhat) = {kappa:.6g} in {time.perf_counter() - t0:.3f} s")
        stream = torch.cuda.current_stream()
        records = []
        for direction in directions:
            x = m_dev if direction == 0 else d_dev
            run = plan.apply if direction == 0 else plan.apply_adjoint
            out = torch.empty((plan.Nt, plan.Nd if direction == 0 else plan.Nm), dtype=torch.float64,
                              device=x.device)
            ref = None
            for bits in range(32):
                plan.set_mask(bits << (5 * direction))
                run(x, out=out)
                torch.cuda.synchronize()
                got = out.cpu().numpy()
                if bits == 0:
                    ref = got.copy()
                for _ in range(warmup):
                    run(x, out=out)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    run(x, out=out)
                e1.record(stream)
                torch.cuda.synchronize()
                rec = {"direction": direction, "bits": bits, "stages": describe(bits),
                       "error": _rel(got, ref) if bits else 0.0, "ms": e0.elapsed_time(e1) / reps}
                records.append(rec)
                if log:
                    log(f"dir {direction} bits {bits:05b}: err {rec['error']:.3e}  {rec['ms']:.4f} ms")
        return records, kappa
    finally:
        plan.close()


def measured_front(records, direction: int, tol: float = math.inf):
    """Measured Pareto front (time, error) of one direction's configurations
    with error <= tol, fastest first."""
    rs = sorted((r for r in records if r["direction"] == direction and r["error"] <= tol),
                key=lambda r: (r["ms"], r["error"], bin(r["bits"]).count("1")))
    front, best = [], math.inf
    for r in rs:
        if r["error"] < best:
            front.append(r)
            best = r["error"]
    return front


def _growth(Nm, Nd, Nt, direction):
    lg = math.log2(Nt)
    n = Nm if direction == 0 else Nd
    return [1.0, lg, float(n), lg, 1.0]


def fit_params(records, Nm, Nd, Nt, kappa, direction, staged=False):
    """Model parameters [c1..c5, cF, B, B_lds, t0] fitted to one direction's sweep.
    The all-FP64 configuration's error is measured against itself (zero),
    so cF keeps the value 1 (the FP64 setup term is ~1e-14 here)."""
    rs = {r["bits"]: r for r in records if r["direction"] == direction}
    g = _growth(Nm, Nd, Nt, direction)
    base = rs[0]["error"]
    c = [max(rs[1 << s]["error"] - base, 0.0) / (kappa * U32 * g[s]) if g[s] > 0 else 0.0 for s in range(5)]
    c.append(1.0)
    flags = fm.FFTMV_FLAG_STAGED if staged else 0
    # HBM bytes, LDS bytes and kernel count of each configuration, read off
    # the library's own model with one term switched on at a time
    inf = math.inf
    X, y = [], []
    for b, r in rs.items():
        row = [fm.fftmv_predict(Nm, Nd, Nt, direction, b, flags, 1.0, c + unit)[1]
               for unit in ([1.0, inf, 0.0], [inf, 1.0, 0.0], [inf, inf, 1.0])]
        X.append(row)
        y.append(r["ms"] * 1e-3)
    X, y = np.array(X), np.array(y)
    # least squares with non-negative coefficients: drop a term whose
    # coefficient comes out negative and fit the rest again
    active = [0, 1, 2]
    while True:
        sol, *_ = np.linalg.lstsq(X[:, active], y, rcond=None)
        if all(v > 0 for v in sol) or len(active) == 1:
            break
        active.pop(int(np.argmin(sol)))
    coef = [0.0, 0.0, 0.0]
    for i, v in zip(active, sol):
        coef[i] = max(float(v), 0.0)
    params = c + [1.0 / coef[0] if coef[0] > 0 else inf, 1.0 / coef[1] if coef[1] > 0 else inf, coef[2]]
    # scale the error constants so that the model bounds every measurement
    worst = 0.0
    for b, r in rs.items():
        if b == 0:
            continue
        pred, _ = fm.fftmv_predict(Nm, Nd, Nt, direction, b, flags, kappa, params)
        worst = max(worst, r["error"] / pred)
    if worst > 1.0:
        params = [x * worst for x in params[:6]] + params[6:]
    return params


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shape", default="main", choices=None)
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--staged", action="store_true")
    ap.add_argument("--json", default=None, help="also write the records here")
    args = ap.parse_args(argv)

    import torch

    from fft_block_toeplitz_amd import workloads as W

    shape = W.SHAPES[args.shape]
    Nm, Nd, Nt = shape.Nm, shape.Nd, shape.Nt
    F, m, d = W.problem(shape)
    dev = torch.device("cuda:0")
    F_dev, m_dev, d_dev = (torch.from_numpy(a).to(dev) for a in (F, m, d))
    del F
    log = lambda s: print(s, file=sys.stderr, flush=True)  # noqa: E731
    records, kappa = sweep(F_dev, m_dev, d_dev, args.reps, args.warmup, args.staged, log=log)

    print(f"## 32-configuration sweep, Nm={Nm} Nd={Nd} Nt={Nt}" + (" (five-kernel form)" if args.staged else ""))
    print(f"\nkappa(Fhat) = {kappa:.6g} (Lanczos on the complex128 blocks)\n")
    params = {}
    for direction in (0, 1):
        name = "F" if direction == 0 else "F*"
        params[direction] = fit_params(records, Nm, Nd, Nt, kappa, direction, args.staged)
        flags = fm.FFTMV_FLAG_STAGED if args.staged else 0
        print(f"### {name}\n")
        print("| stages 1-5 (pad fft sbgemv ifft unpad) | bits | rel. error | ms | predicted error | predicted ms |")
        print("|---|---|---|---|---|---|")
        for r in (r for r in records if r["direction"] == direction):
            pe, pt = fm.fftmv_predict(Nm, Nd, Nt, direction, r["bits"], flags, kappa, params[direction])
            print(f"| {r['stages']} | {r['bits']:05b} | {r['error']:.3e} | {r['ms']:.4f} | {pe:.3e} | "
                  f"{pt * 1e3:.4f} |")
        front = measured_front(records, direction)
        print(f"\nMeasured Pareto front ({name}): " +
              ", ".join(f"{r['bits']:05b} ({r['error']:.2e}, {r['ms']:.4f} ms)" for r in front))
        p = params[direction]
        print(f"\nFitted parameters ({name}): c1..c5 = " + ", ".join(f"{x:.4g}" for x in p[:5]) +
              f", cF = {p[5]:.4g}, B = {p[6]:.4g} B/s, B_lds = {p[7]:.4g} B/s, t0 = {p[8]:.3g} s")
        print(f"\nAs C initialiser: {{{', '.join(repr(float(x)) for x in p)}}}")
        for tol in (1e-6, 1e-7):
            bits, pe, pt, ok = fm.fftmv_select_precision(Nm, Nd, Nt, direction, flags, kappa, tol, p)
            meas = next(r for r in records if r["direction"] == direction and r["bits"] == bits)
            print(f"\nselect_precision({tol:g}) -> {bits:05b} [{describe(bits)}]"
                  f"{'' if ok else ' (no configuration meets the tolerance)'}: predicted {pe:.2e} / "
                  f"{pt * 1e3:.4f} ms, measured {meas['error']:.2e} / {meas['ms']:.4f} ms")
        print()
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"shape": [Nm, Nd, Nt], "kappa": kappa, "staged": args.staged, "records": records,
                       "params": {str(k): v for k, v in params.items()}}, f, indent=1)


if __name__ == "__main__":
    main()
