"""fft_block_toeplitz_amd -- block lower-triangular Toeplitz matvec through the
FFT on an AMD Instinct MI355X.

Thin ctypes binding of ``libfftmv.so`` (C ABI declared in
``include/fftmv.h``). The ``fftmv_*`` functions here carry the same names
and arguments as the C entry points and only marshal arguments: every stage
of the computation runs in the library's HIP kernels. ``Plan`` wraps them
for torch tensors (torch only provides device memory and streams).

Operation: "Mixed-precision FFTMatvec performance optimization on AMD
GPUs", sections 1 (block triangular Toeplitz operator), 1.1 (five stages),
1.2 (conjugate-transpose product for F*) and 2.2 (per-stage FP32/FP64).

There is no fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfftmv.so")

# ---- constants mirrored from include/fftmv.h
FFTMV_SUCCESS = 0
FFTMV_ERR_INVALID_ARG = -1
FFTMV_ERR_UNSUPPORTED_SIZE = -2
FFTMV_ERR_OUT_OF_MEMORY = -3
FFTMV_ERR_HIP = -4
FFTMV_ERR_INTERNAL = -5
FFTMV_ERR_NO_CONFIG = -6

FFTMV_DIR_F = 0
FFTMV_DIR_FADJ = 1
FFTMV_ALL_FP64 = 0x000
FFTMV_MIXED_F = 0x006
FFTMV_MIXED_FADJ = 0x180
FFTMV_MIXED = 0x186
FFTMV_PREC_BITS = 0x3FF
FFTMV_FLAG_STAGED = 1 << 16
FFTMV_FLAG_FHAT_BOTH = 1 << 17
FFTMV_MODEL_PARAMS = 9

FFTMV_SCRATCH_BYTES = 128 << 20

EXPORTS = ("fftmv_setup", "fftmv_apply", "fftmv_apply_adjoint", "fftmv_apply_scratch", "fftmv_destroy",
           "fftmv_status_string",
           "fftmv_query", "fftmv_set_mask", "fftmv_run_stages", "fftmv_buffer", "fftmv_model_defaults",
           "fftmv_predict", "fftmv_pareto_front", "fftmv_select_precision", "fftmv_condition", "fftmv_version")


def FFTMV_FP32(direction: int, stage: int) -> int:
    """Mask bit that puts stage (1..5) of direction (0 = F, 1 = F*) in FP32."""
    return 1 << (5 * direction + stage - 1)


def stage_is_fp32(mask: int, direction: int, stage: int) -> bool:
    return bool(mask & FFTMV_FP32(direction, stage))


class FftmvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fftmv_status_string(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m fft_block_toeplitz_amd.build "
                           "or __graft_entry__.build()); there is no CPU fallback")
    # torch ships its own HIP runtime under the same soname; load it first so
    # that the library binds to that one runtime (one set of streams and
    # allocations per process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, I64, U32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int
    L.fftmv_setup.argtypes = [ctypes.POINTER(P), P, I64, I64, I64, U32, P]
    L.fftmv_apply.argtypes = [P, P, P, P]
    L.fftmv_apply_adjoint.argtypes = [P, P, P, P]
    L.fftmv_apply_scratch.argtypes = [P, I, P, P, P]
    L.fftmv_destroy.argtypes = [P]
    L.fftmv_status_string.argtypes = [I]
    L.fftmv_status_string.restype = ctypes.c_char_p
    L.fftmv_query.argtypes = [P, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.fftmv_set_mask.argtypes = [P, U32]
    L.fftmv_run_stages.argtypes = [P, I, I, I, P, P, P]
    L.fftmv_buffer.argtypes = [P, I, ctypes.POINTER(P), ctypes.POINTER(I64), ctypes.POINTER(I)]
    D, DP = ctypes.c_double, ctypes.POINTER(ctypes.c_double)
    L.fftmv_model_defaults.argtypes = [I, DP]
    L.fftmv_predict.argtypes = [I64, I64, I64, I, U32, U32, D, DP, DP, DP]
    L.fftmv_pareto_front.argtypes = [I64, I64, I64, I, U32, D, D, DP, ctypes.POINTER(U32), ctypes.POINTER(I)]
    L.fftmv_select_precision.argtypes = [I64, I64, I64, I, U32, D, D, DP, ctypes.POINTER(U32), DP, DP]
    L.fftmv_condition.argtypes = [P, I, DP, DP, DP, P]
    L.fftmv_version.argtypes = []
    for name in EXPORTS:
        if name != "fftmv_status_string":
            getattr(L, name).restype = I
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != FFTMV_SUCCESS:
        raise FftmvError(status, what)


# ---- same-name wrappers of the C entry points (pointers and streams as ints)
def fftmv_setup(F_dev: int, Nm: int, Nd: int, Nt: int, mask: int, stream: int = 0) -> int:
    plan = ctypes.c_void_p()
    _check(lib().fftmv_setup(ctypes.byref(plan), F_dev, Nm, Nd, Nt, mask, stream), "fftmv_setup")
    return plan.value


def fftmv_apply(plan: int, m_dev: int, v_dev: int, stream: int = 0) -> None:
    _check(lib().fftmv_apply(plan, m_dev, v_dev, stream), "fftmv_apply")


def fftmv_apply_adjoint(plan: int, d_dev: int, w_dev: int, stream: int = 0) -> None:
    _check(lib().fftmv_apply_adjoint(plan, d_dev, w_dev, stream), "fftmv_apply_adjoint")


def fftmv_apply_scratch(plan: int, direction: int, in_dev: int, out_dev: int, stream: int = 0) -> None:
    _check(lib().fftmv_apply_scratch(plan, direction, in_dev, out_dev, stream), "fftmv_apply_scratch")


def fftmv_destroy(plan: int) -> None:
    _check(lib().fftmv_destroy(plan), "fftmv_destroy")


def fftmv_status_string(status: int) -> str:
    return lib().fftmv_status_string(status).decode()


def fftmv_query(plan: int) -> tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().fftmv_query(plan, ctypes.byref(a), ctypes.byref(b)), "fftmv_query")
    return a.value, b.value


def fftmv_set_mask(plan: int, mask: int) -> None:
    _check(lib().fftmv_set_mask(plan, mask), "fftmv_set_mask")


def fftmv_run_stages(plan: int, direction: int, first: int, last: int, in_dev: int | None,
                     out_dev: int | None, stream: int = 0) -> None:
    _check(lib().fftmv_run_stages(plan, direction, first, last, in_dev, out_dev, stream), "fftmv_run_stages")


def fftmv_buffer(plan: int, which: int) -> tuple[int, int, int]:
    p, ld, eb = ctypes.c_void_p(), ctypes.c_int64(), ctypes.c_int()
    _check(lib().fftmv_buffer(plan, which, ctypes.byref(p), ctypes.byref(ld), ctypes.byref(eb)), "fftmv_buffer")
    return p.value or 0, ld.value, eb.value


def _params(params):
    if params is None:
        return None
    vals = [float(x) for x in params]
    if len(vals) != FFTMV_MODEL_PARAMS:
        raise ValueError(f"model parameters: expected {FFTMV_MODEL_PARAMS} values, got {len(vals)}")
    return (ctypes.c_double * FFTMV_MODEL_PARAMS)(*vals)


def fftmv_model_defaults(direction: int) -> list[float]:
    """[c1, c2, c3, c4, c5, cF, HBM bytes/s, LDS bytes/s, seconds per kernel]."""
    out = (ctypes.c_double * FFTMV_MODEL_PARAMS)()
    _check(lib().fftmv_model_defaults(direction, out), "fftmv_model_defaults")
    return list(out)


def fftmv_predict(Nm: int, Nd: int, Nt: int, direction: int, stage_bits: int, flags: int, kappa: float,
                  params=None) -> tuple[float, float]:
    """(predicted relative error, predicted apply seconds) of one configuration."""
    e, t = ctypes.c_double(), ctypes.c_double()
    _check(lib().fftmv_predict(Nm, Nd, Nt, direction, stage_bits, flags, kappa, _params(params), ctypes.byref(e),
                               ctypes.byref(t)), "fftmv_predict")
    return e.value, t.value


def fftmv_pareto_front(Nm: int, Nd: int, Nt: int, direction: int, flags: int, kappa: float, error_tol: float,
                       params=None) -> list[int]:
    """Stage-bit configurations on the feasible Pareto front, fastest first."""
    front, n = (ctypes.c_uint32 * 32)(), ctypes.c_int()
    _check(lib().fftmv_pareto_front(Nm, Nd, Nt, direction, flags, kappa, error_tol, _params(params), front,
                                    ctypes.byref(n)), "fftmv_pareto_front")
    return list(front[:n.value])


def fftmv_select_precision(Nm: int, Nd: int, Nt: int, direction: int, flags: int, kappa: float,
                           error_tol: float, params=None) -> tuple[int, float, float, bool]:
    """(stage bits, predicted error, predicted seconds, feasible). When no
    configuration meets the tolerance, feasible is False and the all-FP64
    configuration is reported."""
    b, e, t = ctypes.c_uint32(), ctypes.c_double(), ctypes.c_double()
    st = lib().fftmv_select_precision(Nm, Nd, Nt, direction, flags, kappa, error_tol, _params(params),
                                      ctypes.byref(b), ctypes.byref(e), ctypes.byref(t))
    if st not in (FFTMV_SUCCESS, FFTMV_ERR_NO_CONFIG):
        _check(st, "fftmv_select_precision")
    return b.value, e.value, t.value, st == FFTMV_SUCCESS


def fftmv_condition(plan: int, iters: int, K: int, stream: int = 0):
    """(kappa, sigma_max[K], sigma_min[K]) of the plan's frequency blocks;
    K = Nt + 1. Synchronises the stream."""
    kappa = ctypes.c_double()
    smax, smin = (ctypes.c_double * K)(), (ctypes.c_double * K)()
    _check(lib().fftmv_condition(plan, iters, ctypes.byref(kappa), smax, smin, stream), "fftmv_condition")
    return kappa.value, list(smax), list(smin)


def fftmv_version() -> int:
    return lib().fftmv_version()


# ---- torch convenience layer
def _stream_handle(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _require(t, shape, name):
    import torch

    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float64 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float64 CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class Plan:
    """A setup plan on torch tensors. ``F`` is a contiguous float64 device
    tensor [Nt][Nd][Nm]; it may be freed once the constructor returns."""

    def __init__(self, F, mask: int = FFTMV_MIXED, stream=None):
        Nt, Nd, Nm = (int(s) for s in F.shape)
        _require(F, (Nt, Nd, Nm), "F")
        self.Nm, self.Nd, self.Nt, self.mask = Nm, Nd, Nt, mask
        self.device = F.device
        self.handle = fftmv_setup(F.data_ptr(), Nm, Nd, Nt, mask, _stream_handle(stream))

    def apply(self, m, out=None, stream=None):
        """v = F m on the given (default: current) stream; returns v [Nt][Nd]."""
        import torch

        _require(m, (self.Nt, self.Nm), "m")
        v = torch.empty((self.Nt, self.Nd), dtype=torch.float64, device=m.device) if out is None else out
        _require(v, (self.Nt, self.Nd), "out")
        fftmv_apply(self.handle, m.data_ptr(), v.data_ptr(), _stream_handle(stream))
        return v

    def apply_adjoint(self, d, out=None, stream=None):
        """w = F* d on the given (default: current) stream; returns w [Nt][Nm]."""
        import torch

        _require(d, (self.Nt, self.Nd), "d")
        w = torch.empty((self.Nt, self.Nm), dtype=torch.float64, device=d.device) if out is None else out
        _require(w, (self.Nt, self.Nm), "out")
        fftmv_apply_adjoint(self.handle, d.data_ptr(), w.data_ptr(), _stream_handle(stream))
        return w

    def set_mask(self, mask: int) -> None:
        fftmv_set_mask(self.handle, mask)
        self.mask = mask

    def run_stages(self, direction: int, first: int, last: int, x=None, out=None, stream=None) -> None:
        """Stages first..last of one direction: x (the FP64 input, needed when
        first == 1) and out (the FP64 output, when last == 5) are checked
        against the direction's shapes."""
        n_in, n_out = (self.Nm, self.Nd) if direction == FFTMV_DIR_F else (self.Nd, self.Nm)
        if first == 1:
            _require(x, (self.Nt, n_in), "x")
        if last == 5:
            _require(out, (self.Nt, n_out), "out")
        fftmv_run_stages(self.handle, direction, first, last, None if x is None else x.data_ptr(),
                         None if out is None else out.data_ptr(), _stream_handle(stream))

    def condition(self, iters: int = 0, stream=None):
        """(kappa, sigma_max per frequency, sigma_min per frequency) of Fhat."""
        return fftmv_condition(self.handle, iters, self.Nt + 1, _stream_handle(stream))

    def query(self) -> tuple[int, int]:
        return fftmv_query(self.handle)

    def buffer_info(self, which: int):
        """(rows, ld, elem_bytes, is_complex, device pointer) of a plan buffer."""
        ptr, ld, eb = fftmv_buffer(self.handle, which)
        if which in (0, 1):
            rows, cplx = (self.Nt + 1) * self.Nd, True
        else:
            st = (which - 10) % 10
            rows, cplx = (self.Nt if st in (1, 4) else self.Nt + 1), st in (2, 3)
        return rows, ld, eb, cplx, ptr

    def _dtype(self, which: int):
        import torch

        rows, ld, eb, cplx, ptr = self.buffer_info(which)
        dtype = {(4, False): torch.float32, (8, False): torch.float64,
                 (8, True): torch.complex64, (16, True): torch.complex128}[(eb, cplx)]
        return rows, ld, eb, dtype, ptr

    def read_buffer(self, which: int):
        """Copy of a plan buffer (rows x ld) as a torch tensor on the device.
        Synchronises the device first."""
        import torch

        rows, ld, eb, dtype, ptr = self._dtype(which)
        if not ptr:
            raise ValueError(f"plan buffer {which} is not allocated")
        t = torch.empty((rows, ld), dtype=dtype, device=self.device)
        torch.cuda.synchronize(self.device)
        _hip_memcpy_d2d(t.data_ptr(), ptr, rows * ld * eb)
        return t

    def write_buffer(self, which: int, values) -> None:
        """Overwrite a plan buffer (rows x ld) from a device tensor, for
        stage-by-stage checks. Synchronises the device first."""
        import torch

        rows, ld, eb, dtype, ptr = self._dtype(which)
        src = values.to(device=self.device, dtype=dtype).contiguous()
        if tuple(src.shape) != (rows, ld):
            raise ValueError(f"buffer {which} is {(rows, ld)}, got {tuple(src.shape)}")
        torch.cuda.synchronize(self.device)
        _hip_memcpy_d2d(ptr, src.data_ptr(), rows * ld * eb)

    def close(self) -> None:
        if getattr(self, "handle", None):
            fftmv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_hip = None


def _hip_memcpy_d2d(dst: int, src: int, nbytes: int) -> None:
    """Blocking device-to-device copy through the HIP runtime."""
    global _hip
    if _hip is None:
        lib()
        # the HIP runtime already mapped into this process (torch's)
        paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
        _hip = ctypes.CDLL(paths[0] if paths else "libamdhip64.so.7")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    rc = _hip.hipMemcpy(dst, src, nbytes, 3)  # hipMemcpyDeviceToDevice
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed with {rc}")
