#!/usr/bin/env python3
"""Benchmark of the block-Toeplitz FFT matvec on one MI355X.

One step = one F apply followed by one F* apply (all five stages of each,
"Mixed-precision FFTMatvec performance optimization on AMD GPUs", section
1.1) at Nm=5000, Nd=100, Nt=1000 in the page's mixed precision (section 2.2:
F with FFT + SBGEMV in FP32, F* with SBGEMV + IFFT in FP32), inputs resident
in HBM. Prints one JSON line.

value = algorithmic HBM bytes of the step / step time (GB/s). The bytes are
the fused minimum of each apply: read the FP64 input once, write and read
the stage-2 output once, read Fhat once, write and read the stage-3 output
once, write the FP64 output once (zero padding not counted).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "sbgemv_main_mixed_traffic.json")


def measured_traffic(Nm, Nd, Nt, mask, kernel):
    """HBM bytes per launch of a stage-3 kernel ("sbgemv_n" or "sbgemv_c")
    from the committed rocprofv3 counter record (FETCH_SIZE + WRITE_SIZE,
    calibrated on a plain copy), or None if the record is for another
    workload or the kernel sources changed since the counters were taken."""
    import hashlib

    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != f"Nm={Nm} Nd={Nd} Nt={Nt} mask {mask:#05x}":
        return None
    h = hashlib.sha256()
    for rel in rec.get("sources", []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return int(round(k["traffic_bytes"])) if k else None


def shape_of(name: str):
    """A named workload shape, or NmxNdxNt."""
    from fft_block_toeplitz_amd import workloads as W

    if name in W.SHAPES:
        return W.SHAPES[name]
    parts = name.lower().split("x")
    if len(parts) != 3 or not all(p.isdigit() and int(p) > 0 for p in parts):
        raise SystemExit(f"--shape {name!r}: expected one of {sorted(W.SHAPES)} or NmxNdxNt")
    Nm, Nd, Nt = (int(p) for p in parts)
    return W.Shape(name, Nm=Nm, Nd=Nd, Nt=Nt)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # ~0.65 s at Main: the input copy of F (gigabytes) is freed just before
    # the warm-up, and the HBM-bound kernels run slow for a few hundred
    # milliseconds after such a free
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--shape", default="main",
                    help="tiny, small, main, scale, or NmxNdxNt (e.g. 5000x100x1029) for any supported size")
    ap.add_argument("--mask", type=lambda s: int(s, 0), default=0x186)
    ap.add_argument("--staged", action="store_true", help="five-kernel form (pad/unpad materialised)")
    ap.add_argument("--kernel-reps", type=int, default=20, help="stage-3-only launches timed for the roofline")
    ap.add_argument("--setup-reps", type=int, default=3, help="extra plan setups timed after the first")
    ap.add_argument("--max-extra-warmup", type=int, default=3000,
                    help="further warm-up steps, in chunks of 50, while the step time still improves")
    ap.add_argument("--graph-steps", type=int, default=100, help="steps replayed from a HIP graph (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-cols", type=int, default=0,
                    help="oracle sample: input columns (0 = all Nm when the host's available memory holds twice "
                         "the oracle's complex128 Fhat and F, else Nm/5)")
    ap.add_argument("--no-check", action="store_true", help="skip the spot-step check against the oracle")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (reference for the HBM byte counters) and exit")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the memory ceilings (streaming read, copy, the setup transform's pattern) "
                         "and print them as one JSON line")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of known size: its FETCH_SIZE and
    WRITE_SIZE readings calibrate the counters taken on the kernels."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": n * 4, "copies": 3}), flush=True)


def memory_ceilings(setup_pattern: bool = False, reps: int = 10):
    """Memory-system ceilings of this GPU from the plain kernels of
    libfftmv_ceiling.so (built from fft_block_toeplitz_amd/csrc/ceiling.hip),
    timed with events on the stream they run on:
      read_GBs   4 GiB streamed, each workgroup one contiguous 16 or 64 KiB
                 chunk with all its 16-byte loads in flight (best of both)
      copy_GBs   2 GiB read and written elsewhere in the same chunks
                 (read + write bytes per second, best of both)
      setup_pattern_GBs (optional) the setup transform's memory pattern
                 without its arithmetic, at 8 and 16 FP64 channels per
                 workgroup: F [1000][5e5] read in runs of 8 C bytes, 1001
                 rows of C 8-byte values written (read + write bytes / s)."""
    import ctypes

    import torch

    from fft_block_toeplitz_amd import build as fbuild

    lib = ctypes.CDLL(fbuild.CEILING_LIB)
    P = ctypes.c_void_p
    lib.ceiling_read.argtypes = [P, ctypes.c_size_t, ctypes.c_int, P, P]
    lib.ceiling_copy.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int, P]
    lib.ceiling_tile_rw.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, P]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def timed(launch, nbytes):
        for _ in range(3):
            assert launch() == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    out = {}
    nbytes = 4 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    rd = {kib: timed(lambda kib=kib: lib.ceiling_read(buf.data_ptr(), nbytes, kib, sink.data_ptr(), sh), nbytes)
          for kib in (16, 64)}
    half = nbytes // 2
    src, dst = buf.data_ptr(), buf.data_ptr() + half
    cp = {kib: timed(lambda kib=kib: lib.ceiling_copy(src, dst, half, kib, sh), 2 * half) for kib in (16, 64)}
    out["read_ceiling_GBs"] = max(rd.values())
    out["copy_ceiling_GBs"] = max(cp.values())
    out["read_GBs_by_chunk_kib"] = rd
    out["copy_GBs_by_chunk_kib"] = cp
    del buf
    if setup_pattern:
        nchan = 500000
        F = torch.zeros(1000 * nchan, dtype=torch.float64, device="cuda")
        G = torch.zeros(1001 * nchan, dtype=torch.float64, device="cuda")
        rw = 8 * nchan * (1000 + 1001)
        out["setup_pattern_GBs_by_channels"] = {
            C: timed(lambda C=C: lib.ceiling_tile_rw(F.data_ptr(), G.data_ptr(), nchan, C, sh), rw) for C in (8, 16)}
        del F, G
    torch.cuda.empty_cache()
    return out


def elem(mask, direction, s1, s2, cplx):
    f32 = bool(mask & (1 << (5 * direction + s1 - 1))) or bool(mask & (1 << (5 * direction + s2 - 1)))
    return (8 if f32 else 16) if cplx else (4 if f32 else 8)


def apply_bytes(Nm, Nd, Nt, mask, direction):
    """Fused-minimum algorithmic bytes of one apply."""
    K = Nt + 1
    nin, nout = (Nm, Nd) if direction == 0 else (Nd, Nm)
    fhat = K * Nd * Nm * (8 if mask & (1 << (5 * direction + 2)) else 16)
    hin = K * nin * elem(mask, direction, 2, 3, True)
    hout = K * nout * elem(mask, direction, 3, 4, True)
    return Nt * nin * 8 + 2 * hin + fhat + 2 * hout + Nt * nout * 8


def sbgemv_bytes(Nm, Nd, Nt, mask, direction):
    """Algorithmic bytes of one stage-3 launch: Fhat + its input + its output."""
    K = Nt + 1
    nin, nout = (Nm, Nd) if direction == 0 else (Nd, Nm)
    fhat = K * Nd * Nm * (8 if mask & (1 << (5 * direction + 2)) else 16)
    return fhat + K * nin * elem(mask, direction, 2, 3, True) + K * nout * elem(mask, direction, 3, 4, True)


def host_mem_bytes():
    """(MemTotal, MemAvailable) of the host in bytes, or (None, None)."""
    tot = avail = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    tot = int(line.split()[1]) * 1024
                elif line.startswith("MemAvailable:"):
                    avail = int(line.split()[1]) * 1024
    except OSError:
        pass
    return tot, avail


def host_info():
    """Host CPU model, memory and the thread settings the oracle runs under."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    tot, avail = host_mem_bytes()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "mem_total_GB": tot and round(tot / 1e9, 1),
            "mem_available_GB": avail and round(avail / 1e9, 1),
            "sched_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(shape, mask, F, m, d, cols):
    """The FP64 CPU oracle (as it stands) on the same workload, or on a
    column sample of it (Nm reduced to `cols`, everything else unchanged)
    when cols < Nm. One F and one F* apply with Fhat precomputed, median of
    5 on all the threads the oracle uses and of 3 on one thread; a sample is
    scaled to the full step by the byte model."""
    import oracle

    Nm, Nd, Nt = shape.Nm, shape.Nd, shape.Nt
    Fs = F if cols >= Nm else np.ascontiguousarray(F[:, :, :cols])
    ms = m if cols >= Nm else np.ascontiguousarray(m[:, :cols])
    cols = min(cols, Nm)
    Fh = oracle.setup(Fs)
    sample_bytes = apply_bytes(cols, Nd, Nt, mask, 0) + apply_bytes(cols, Nd, Nt, mask, 1)

    def timed(reps):
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.apply(Fh, ms)
            oracle.apply_adjoint(Fh, d)
            times.append(time.perf_counter() - t0)
        return float(np.median(times))

    threads = oracle.num_threads()
    t = timed(5)
    oracle.set_num_threads(1)
    try:
        t1 = timed(3)
    finally:
        oracle.set_num_threads(threads)
    gbs = sample_bytes / t / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"F and F* apply at Nm={cols} (of {Nm}), Nd={Nd}, Nt={Nt}, FP64 oracle, Fhat precomputed, "
                       f"median of 5: {t * 1e3:.1f} ms; GB/s on the step's byte model at that Nm"
                       + (" (the whole workload)" if cols == Nm else
                          " (a column sample: the host's available memory is below twice the oracle's Fhat + F)")),
            "ms_per_step_full_equiv": round(t * 1e3 * Nm / cols, 1),
            "one_thread": {"value": round(sample_bytes / t1 / 1e9, 3), "unit": "GB/s",
                           "ms_per_step_full_equiv": round(t1 * 1e3 * Nm / cols, 1)},
            "host": host_info()}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.read_ceiling:
        import torch

        torch.cuda.set_device(0)
        print(json.dumps({"memory_ceilings": memory_ceilings(setup_pattern=True), "peak_GBs": PEAK_HBM_GBS}),
              flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import fft_block_toeplitz_amd as fm
    from fft_block_toeplitz_amd import workloads as W

    shape = shape_of(args.shape)
    Nm, Nd, Nt, mask = shape.Nm, shape.Nd, shape.Nt, args.mask
    t0 = time.perf_counter()
    F, m, d = W.problem(shape)
    gen_s = time.perf_counter() - t0
    print(f"[bench] inputs {args.shape} Nm={Nm} Nd={Nd} Nt={Nt} generated in {gen_s:.1f}s", file=sys.stderr,
          flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    F_dev = torch.from_numpy(F).to(dev)
    m_dev = torch.from_numpy(m).to(dev)
    d_dev = torch.from_numpy(d).to(dev)
    flags = fm.FFTMV_FLAG_STAGED if args.staged else 0
    t0 = time.perf_counter()
    plan = fm.Plan(F_dev, mask | flags)
    setup_s = time.perf_counter() - t0
    del F_dev
    torch.cuda.empty_cache()
    v_dev = torch.empty((Nt, Nd), dtype=torch.float64, device=dev)
    w_dev = torch.empty((Nt, Nm), dtype=torch.float64, device=dev)
    print(f"[bench] setup {setup_s:.2f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.apply(m_dev, out=v_dev)
        plan.apply_adjoint(d_dev, out=w_dev)
    torch.cuda.synchronize()
    # then keep warming in chunks while the step time still improves: memory
    # freed just before (here or by an earlier process) slows HBM-bound
    # kernels for a while after the free
    warm_run = args.warmup
    prev = None
    for _ in range(args.max_extra_warmup // 50):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(50):
            plan.apply(m_dev, out=v_dev)
            plan.apply_adjoint(d_dev, out=w_dev)
        c1.record(stream)
        torch.cuda.synchronize()
        warm_run += 50
        chunk = c0.elapsed_time(c1)
        if prev is not None and chunk > prev * 0.995:
            break
        prev = chunk

    # whole steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        plan.apply(m_dev, out=v_dev)
        ev[3 * i + 1].record(stream)
        plan.apply_adjoint(d_dev, out=w_dev)
        ev[3 * i + 2].record(stream)
        ev[3 * i + 3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = ev[0].elapsed_time(ev[3 * args.steps])
    f_ms = [ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)]
    a_ms = [ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)]
    ms_step = total_ms / args.steps
    print(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (wall {wall:.3f}s)", file=sys.stderr, flush=True)

    # the same step replayed from a HIP graph (context: launch overhead)
    graph_ms = None
    if args.graph_steps:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            plan.apply(m_dev, out=v_dev)
            plan.apply_adjoint(d_dev, out=w_dev)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            plan.apply(m_dev, out=v_dev)
            plan.apply_adjoint(d_dev, out=w_dev)
        for _ in range(10):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.graph_steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.graph_steps
        del graph

    bF, bA = apply_bytes(Nm, Nd, Nt, mask, 0), apply_bytes(Nm, Nd, Nt, mask, 1)
    value = (bF + bA) / (ms_step * 1e-3) / 1e9

    # the stage-3 kernels alone (same kernels and launches as in the applies),
    # timed with events on the stream they are launched on; the roofline
    # reports the one that takes longer (the step's dominant kernel)
    kernel = {}
    for direction, name in ((0, "sbgemv_n"), (1, "sbgemv_c")):
        plan.run_stages(direction, 3, 3)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.kernel_reps):
            plan.run_stages(direction, 3, 3)
        e1.record(stream)
        torch.cuda.synchronize()
        kms = e0.elapsed_time(e1) / args.kernel_reps
        kb = sbgemv_bytes(Nm, Nd, Nt, mask, direction)
        kernel[name] = {"avg_ms": round(kms, 5), "bytes": kb, "GB/s": round(kb / (kms * 1e-3) / 1e9, 1)}
    print(f"[bench] kernels {kernel}", file=sys.stderr, flush=True)

    # context: the streaming read and copy ceilings of this GPU, measured
    # before the extra setups below, whose frees of gigabytes slow HBM-bound
    # kernels for a while
    ceilings = memory_ceilings()
    print(f"[bench] memory ceilings {ceilings}", file=sys.stderr, flush=True)

    # correctness spot check against the oracle (direct sum at a few steps)
    check = None
    if not args.no_check:
        import oracle

        steps = np.array([0, 1, Nt // 2, Nt - 1])
        plan.apply(m_dev, out=v_dev)
        plan.apply_adjoint(d_dev, out=w_dev)
        torch.cuda.synchronize()
        v, w = v_dev.cpu().numpy(), w_dev.cpu().numpy()
        check = {"steps": steps.tolist(),
                 "rel_err_F": float(oracle.rel_l2(v[steps], oracle.direct(F, m, steps))),
                 "rel_err_Fadj": float(oracle.rel_l2(w[steps], oracle.direct_adjoint(F, d, steps)))}
        print(f"[bench] spot check {check}", file=sys.stderr, flush=True)

    # setup again on a warm allocator: the time of fftmv_setup itself
    # (allocation, zero fills, the FP64 transform of F, synchronisation).
    # Done after the timed region: freeing gigabytes of device memory slows
    # the HBM-bound kernels that follow for a few hundred milliseconds.
    setup_ms = []
    if args.setup_reps:
        F_dev = torch.from_numpy(F).to(dev)
        for _ in range(args.setup_reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            extra = fm.Plan(F_dev, mask | flags)
            setup_ms.append((time.perf_counter() - t0) * 1e3)
            extra.close()
        del F_dev
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cols = args.cpu_sample_cols
        if not cols:
            need = (Nt + 1) * Nd * Nm * 16 + Nt * Nd * Nm * 8  # the oracle's Fhat and F
            avail = host_mem_bytes()[1]
            cols = Nm if avail is not None and avail >= 2 * need else max(1, Nm // 5)
        t0 = time.perf_counter()
        cpu = cpu_baseline(shape, mask, F, m, d, cols)
        print(f"[bench] cpu baseline {cpu} ({time.perf_counter() - t0:.1f}s)", file=sys.stderr, flush=True)

    dom = max(kernel, key=lambda name: kernel[name]["avg_ms"])
    kn = kernel[dom]
    achieved = kn["bytes"] / (kn["avg_ms"] * 1e-3) / 1e9
    fmed, amed = float(np.median(f_ms)), float(np.median(a_ms))
    headline = (Nm, Nd, Nt, mask, args.staged) == (5000, 100, 1000, 0x186, False)
    out = {
        "metric": ("F / F* apply ms + HBM GB/s (% of peak) at Nm=5000 Nd=100 Nt=1000, mixed" if headline else
                   f"F / F* apply ms + HBM GB/s (% of peak) at Nm={Nm} Nd={Nd} Nt={Nt}, mask {mask:#05x}"),
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_run,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+f64",
        "data": "synthetic",
        "config": {"workload": f"FFT block-Toeplitz matvec, F + F* apply, Nm={Nm} Nd={Nd} Nt={Nt}, "
                               f"precision mask {mask:#05x}" + (" (five-kernel form)" if args.staged else ""),
                   "Nm": Nm, "Nd": Nd, "Nt": Nt, "mask": hex(mask), "staged": args.staged, "seed": 0},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 1),
        "f_apply_ms": round(fmed, 4),
        "fadj_apply_ms": round(amed, 4),
        "f_apply_ms_min": round(float(np.min(f_ms)), 4),
        "fadj_apply_ms_min": round(float(np.min(a_ms)), 4),
        "f_apply_GBs": round(bF / (fmed * 1e-3) / 1e9, 1),
        "fadj_apply_GBs": round(bA / (amed * 1e-3) / 1e9, 1),
        "bytes_per_step": bF + bA,
        "kernels": kernel,
        "roofline": {"bound": "hbm",
                     "kernel": dom + (" (stage 3, F)" if dom == "sbgemv_n" else " (stage 3, F*)"),
                     "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(Nm, Nd, Nt, mask, dom),
                     "algorithmic_bytes": kn["bytes"]},
        "cpu_baseline": cpu,
        "check": check,
        "context": {"page_mi355x_f_apply_ms": {"fp64": 1.9, "mixed": 1.3},
                    "read_ceiling_GBs": ceilings["read_ceiling_GBs"],
                    "copy_ceiling_GBs": ceilings["copy_ceiling_GBs"],
                    "dominant_kernel_frac_of_read_ceiling": round(achieved / ceilings["read_ceiling_GBs"], 4)},
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms else None,
        "setup_s": round(setup_s, 3),
        "setup_ms": {"first": round(setup_s * 1e3, 2), "repeats": [round(x, 2) for x in setup_ms]},
    }
    print(json.dumps(out), flush=True)
    plan.close()


if __name__ == "__main__":
    main()
