"""CPU oracle for the block-Toeplitz FFT matvec -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library neither imports nor
links it, and the two share no code.

Thin ctypes wrapper around ``oracle.c`` (plain binary64 C with its own
recursive mixed-radix FFT), plus ``dense_operator``, the brute-force
(Nd*Nt) x (Nm*Nt) matrix for tiny cases.

Source: "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
sections 1 (block triangular Toeplitz operator), 1.1 (five stages) and 1.2
(conjugate transpose for the adjoint).

Parity pins (tests/test_oracle_*.py): the FFT against a textbook O(N^2) DFT,
numpy.fft and closed forms; the five stages against the dense product and
the direct double sum; the adjoint identity; zero, delta, delay, block
diagonal, Nt = 1 and scalar-convolution special cases; the condition number
of Fhat against operators built with known singular values (closed forms).
No function here is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        # compiling starts gcc as a child process; a process that has already
        # initialised a GPU must not do that (build first, before the GPU)
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_initialized():
            raise RuntimeError("oracle/liboracle.so is missing or older than oracle.c: run "
                               "__graft_entry__.build() (or oracle.build()) before using the GPU")
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_fft.argtypes = [I64, P, P, ctypes.c_int]
    lib.oracle_setup.argtypes = [P, I64, I64, I64, P]
    lib.oracle_apply.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.oracle_apply_adjoint.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.oracle_direct.argtypes = [P, I64, I64, I64, P, P, I64, P]
    lib.oracle_direct_adjoint.argtypes = [P, I64, I64, I64, P, P, I64, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def fft(x, sign: int = -1) -> np.ndarray:
    """Unnormalised DFT of a complex vector: sum_j x[j] exp(sign 2 pi i j k / n)."""
    x = np.ascontiguousarray(x, dtype=np.complex128)
    out = np.empty_like(x)
    _check(_load().oracle_fft(x.size, _ptr(x), _ptr(out), int(sign)), "oracle_fft")
    return out


def setup(F) -> np.ndarray:
    """Fhat [Nt+1][Nd][Nm] complex128 from F [Nt][Nd][Nm]."""
    F = _f64(F)
    Nt, Nd, Nm = F.shape
    Fhat = np.empty((Nt + 1, Nd, Nm), dtype=np.complex128)
    _check(_load().oracle_setup(_ptr(F), Nm, Nd, Nt, _ptr(Fhat)), "oracle_setup")
    return Fhat


def apply(Fhat, m, dumps: bool = False):
    """v = F m, v [Nt][Nd]. With dumps=True returns (v, mhat, vhat)."""
    K, Nd, Nm = Fhat.shape
    Nt = K - 1
    m = _f64(m)
    assert m.shape == (Nt, Nm)
    v = np.empty((Nt, Nd))
    mh = np.empty((K, Nm), np.complex128) if dumps else None
    vh = np.empty((K, Nd), np.complex128) if dumps else None
    _check(_load().oracle_apply(_ptr(Fhat), Nm, Nd, Nt, _ptr(m), _ptr(v), _ptr(mh), _ptr(vh)),
           "oracle_apply")
    return (v, mh, vh) if dumps else v


def apply_adjoint(Fhat, d, dumps: bool = False):
    """w = F* d, w [Nt][Nm]. With dumps=True returns (w, dhat, what)."""
    K, Nd, Nm = Fhat.shape
    Nt = K - 1
    d = _f64(d)
    assert d.shape == (Nt, Nd)
    w = np.empty((Nt, Nm))
    dh = np.empty((K, Nd), np.complex128) if dumps else None
    wh = np.empty((K, Nm), np.complex128) if dumps else None
    _check(_load().oracle_apply_adjoint(_ptr(Fhat), Nm, Nd, Nt, _ptr(d), _ptr(w), _ptr(dh), _ptr(wh)),
           "oracle_apply_adjoint")
    return (w, dh, wh) if dumps else w


def direct(F, m, steps=None) -> np.ndarray:
    """v_i = sum_{j<=i} F_{i-j} m_j for the listed steps i (all by default)."""
    F, m = _f64(F), _f64(m)
    Nt, Nd, Nm = F.shape
    steps = np.arange(Nt, dtype=np.int64) if steps is None else np.ascontiguousarray(steps, dtype=np.int64)
    v = np.empty((steps.size, Nd))
    _check(_load().oracle_direct(_ptr(F), Nm, Nd, Nt, _ptr(m), _ptr(steps), steps.size, _ptr(v)),
           "oracle_direct")
    return v


def direct_adjoint(F, d, steps=None) -> np.ndarray:
    """w_j = sum_{i>=j} F_{i-j}^T d_i for the listed steps j (all by default)."""
    F, d = _f64(F), _f64(d)
    Nt, Nd, Nm = F.shape
    steps = np.arange(Nt, dtype=np.int64) if steps is None else np.ascontiguousarray(steps, dtype=np.int64)
    w = np.empty((steps.size, Nm))
    _check(_load().oracle_direct_adjoint(_ptr(F), Nm, Nd, Nt, _ptr(d), _ptr(steps), steps.size, _ptr(w)),
           "oracle_direct_adjoint")
    return w


def dense_operator(F) -> np.ndarray:
    """The block lower-triangular Toeplitz matrix itself, built block by
    block: A[i*Nd + r, j*Nm + c] = F[i-j][r][c] for i >= j, 0 above.
    For tiny cases only (size (Nd*Nt) x (Nm*Nt))."""
    F = _f64(F)
    Nt, Nd, Nm = F.shape
    A = np.zeros((Nt * Nd, Nt * Nm))
    for i in range(Nt):
        for j in range(i + 1):
            A[i * Nd:(i + 1) * Nd, j * Nm:(j + 1) * Nm] = F[i - j]
    return A


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole array."""
    x = np.asarray(x).ravel()
    ref = np.asarray(ref).ravel()
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def condition(Fhat):
    """(kappa, s_max per frequency, s_min per frequency) of Fhat [K][Nd][Nm].

    Section 1.1 scales the error bound by the condition number of Fhat.
    Fhat is block diagonal with one Nd x Nm block per frequency, so its
    singular values are those of all the blocks together:
    kappa = max_k s_max(Fhat_k) / min_k s_min(Fhat_k), each block having
    min(Nd, Nm) singular values; +inf when a block is singular. numpy's SVD
    is the step."""
    Fh = np.asarray(Fhat, dtype=np.complex128)
    s = np.linalg.svd(Fh, compute_uv=False)
    smax, smin = s[:, 0], s[:, -1]
    lo = float(smin.min())
    kappa = float(smax.max()) / lo if lo > 0 else float("inf")
    return kappa, smax, smin
