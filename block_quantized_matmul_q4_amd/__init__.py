"""Python binding of libqmm: block-quantized (GGUF Q4_0 / Q8_0, and Q4_K
super-blocks) weight matmul on AMD Instinct MI355X.

Argument marshalling only: every step of the computation runs in the
library's gfx950 kernels; PyTorch supplies device memory and the stream.

Two layers:
* ``qmm_gemv_q4_0``, ``qmm_gemv_q8_0``, ``qmm_gemm_q4_0``, ``qmm_gemm_q8_0``,
  ``qmm_ffn_gate_up_q4_0``, ``qmm_gemv_q4_k``, ``qmm_gemm_q4_k`` -- the C-ABI
  entry points of ``include/qmm.h``
  with the same names and arguments (device addresses as integers, a HIP
  stream handle); they return the status code.
* ``gemv_q4_0``, ``gemv_q8_0``, ``gemm_q4_0``, ``gemm_q8_0``,
  ``ffn_gate_up_q4_0``, ``gemv_q4_k``, ``gemm_q4_k`` -- tensor front ends that check dtypes, shapes and
  devices, allocate ``y`` with torch, launch on the current stream and raise
  ``QmmError`` on a non-OK status.

There is no fallback: if ``libqmm.so`` is missing, every call raises.
Build it with ``python -m block_quantized_matmul_q4_amd._build``.
"""

from __future__ import annotations

import ctypes
import pathlib

HERE = pathlib.Path(__file__).resolve().parent
LIBRARY = HERE / "libqmm.so"

QMM_OK, QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED, QMM_EHIP = range(5)
GEMV_MAX_M = 16
MAX_K = 65536
# format -> (weights per block, bytes per block)
BLOCKS = {"q4_0": (32, 18), "q8_0": (32, 34), "q4_k": (256, 144)}

# Every symbol include/qmm.h declares.
EXPORTS = ("qmm_gemv_q4_0", "qmm_gemv_q8_0", "qmm_gemm_q4_0", "qmm_gemm_q8_0",
           "qmm_ffn_gate_up_q4_0", "qmm_gemv_q4_k", "qmm_gemm_q4_k", "qmm_status_string",
           "qmm_last_error", "qmm_version")


class QmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded ``libqmm.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # PyTorch owns the device memory and streams we are handed, so the
        # library must bind to the same HIP runtime instance: load torch's
        # first (the loader then resolves libqmm's libamdhip64.so.7 to it).
        import torch  # noqa: F401
        if not LIBRARY.exists():
            raise QmmError(QMM_EHIP, f"{LIBRARY} is not built; run "
                           "`python -m block_quantized_matmul_q4_amd._build`")
        lib = ctypes.CDLL(str(LIBRARY))
        args = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        for name in ("qmm_gemv_q4_0", "qmm_gemv_q8_0", "qmm_gemm_q4_0", "qmm_gemm_q8_0",
                     "qmm_gemv_q4_k", "qmm_gemm_q4_k"):
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.qmm_ffn_gate_up_q4_0.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [
            ctypes.c_void_p]
        lib.qmm_ffn_gate_up_q4_0.restype = ctypes.c_int
        lib.qmm_status_string.argtypes = [ctypes.c_int]
        lib.qmm_status_string.restype = ctypes.c_char_p
        lib.qmm_last_error.argtypes = []
        lib.qmm_last_error.restype = ctypes.c_char_p
        lib.qmm_version.argtypes = []
        lib.qmm_version.restype = ctypes.c_int
        _lib = lib
    return _lib


# ---------------------------------------------------------------------------
# C-ABI mirror
# ---------------------------------------------------------------------------

def qmm_gemv_q4_0(x: int, w: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return library().qmm_gemv_q4_0(x, w, y, M, N, K, stream)


def qmm_gemv_q8_0(x: int, w: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return library().qmm_gemv_q8_0(x, w, y, M, N, K, stream)


def qmm_gemm_q4_0(x: int, w: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return library().qmm_gemm_q4_0(x, w, y, M, N, K, stream)


def qmm_gemm_q8_0(x: int, w: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return library().qmm_gemm_q8_0(x, w, y, M, N, K, stream)


def qmm_ffn_gate_up_q4_0(x: int, w_gate: int, w_up: int, h: int, M: int, N: int, K: int,
                         stream: int = 0) -> int:
    return library().qmm_ffn_gate_up_q4_0(x, w_gate, w_up, h, M, N, K, stream)


def qmm_gemv_q4_k(x: int, w: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return library().qmm_gemv_q4_k(x, w, y, M, N, K, stream)


def qmm_gemm_q4_k(x: int, w: int, y: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return library().qmm_gemm_q4_k(x, w, y, M, N, K, stream)


def qmm_status_string(status: int) -> str:
    return library().qmm_status_string(status).decode()


def qmm_last_error() -> str:
    return library().qmm_last_error().decode()


def qmm_version() -> int:
    return library().qmm_version()


def status_string(status: int) -> str:
    try:
        return qmm_status_string(status)
    except Exception:  # library missing: still name the status
        return {0: "QMM_OK", 1: "QMM_EINVAL", 2: "QMM_EALIGN",
                3: "QMM_EUNSUPPORTED", 4: "QMM_EHIP"}.get(status, str(status))


def check(status: int) -> None:
    if status != QMM_OK:
        raise QmmError(status, qmm_last_error())


# ---------------------------------------------------------------------------
# Tensor front ends
# ---------------------------------------------------------------------------

def _call(fn, fmt, x, w, n, k, out):
    import torch

    if not (isinstance(x, torch.Tensor) and isinstance(w, torch.Tensor)):
        raise TypeError("x and w must be torch tensors")
    if x.device.type != "cuda" or w.device != x.device:
        raise ValueError("x and w must be on the same GPU")
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 [M, K] tensor")
    if w.dtype != torch.uint8 or not w.is_contiguous():
        raise ValueError("w must be a contiguous uint8 tensor of packed blocks")
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x has {x.shape[1]} columns, K={k}")
    per, nbytes = BLOCKS[fmt]
    if k % per or w.numel() != n * (k // per) * nbytes:
        raise ValueError(f"w has {w.numel()} bytes; {fmt} N={n} K={k} needs "
                         f"{n * (k // per) * nbytes} (K a multiple of {per})")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    elif (out.dtype != torch.float32 or out.shape != (m, n) or not out.is_contiguous()
          or out.device != x.device):
        raise ValueError("out must be a contiguous float32 [M, N] tensor on x's device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        check(fn(x.data_ptr(), w.data_ptr(), out.data_ptr(), m, n, k, stream))
    return out


def gemv_q4_0(x, w, n: int, k: int, out=None):
    """y[M, N] = x[M, K] @ W^T for Q4_0 W (1 <= M <= 16)."""
    return _call(qmm_gemv_q4_0, "q4_0", x, w, n, k, out)


def gemv_q8_0(x, w, n: int, k: int, out=None):
    """y[M, N] = x[M, K] @ W^T for Q8_0 W (1 <= M <= 16)."""
    return _call(qmm_gemv_q8_0, "q8_0", x, w, n, k, out)


def gemm_q4_0(x, w, n: int, k: int, out=None):
    """y[M, N] = bf16(x) @ bf16(W)^T with f32 accumulation, Q4_0 W, any M
    (M <= 4, and M <= 16 with N <= 4096: the GEMV result, bit for bit)."""
    return _call(qmm_gemm_q4_0, "q4_0", x, w, n, k, out)


def gemm_q8_0(x, w, n: int, k: int, out=None):
    """y[M, N] = bf16(x) @ bf16(W)^T with f32 accumulation, Q8_0 W, any M
    (M <= 4, and M <= 16 with N <= 4096: the GEMV result, bit for bit)."""
    return _call(qmm_gemm_q8_0, "q8_0", x, w, n, k, out)


def gemv_q4_k(x, w, n: int, k: int, out=None):
    """y[M, N] = x[M, K] @ W^T for Q4_K W (super-blocks of 256; 1 <= M <= 16)."""
    return _call(qmm_gemv_q4_k, "q4_k", x, w, n, k, out)


def gemm_q4_k(x, w, n: int, k: int, out=None):
    """y[M, N] = bf16(x) @ bf16(W)^T with f32 accumulation, Q4_K W, any M
    (M <= 4, and M <= 16 with N <= 4096: the GEMV result, bit for bit)."""
    return _call(qmm_gemm_q4_k, "q4_k", x, w, n, k, out)


def ffn_gate_up_q4_0(x, w_gate, w_up, n: int, k: int, out=None):
    """h[M, N] = gelu_tanh(x @ W_gate^T) * (x @ W_up^T) for Q4_0 W_gate, W_up (1 <= M <= 16)."""
    import torch

    if not isinstance(w_up, torch.Tensor):
        raise TypeError("w_up must be a torch tensor")
    if w_up.device != w_gate.device or w_up.dtype != torch.uint8 or not w_up.is_contiguous():
        raise ValueError("w_up must be a contiguous uint8 tensor on w_gate's device")
    if w_up.numel() != w_gate.numel():
        raise ValueError("w_up and w_gate must have the same size")

    def fn(xp, wp, yp, m, n_, k_, stream):
        return qmm_ffn_gate_up_q4_0(xp, wp, w_up.data_ptr(), yp, m, n_, k_, stream)

    return _call(fn, "q4_0", x, w_gate, n, k, out)
