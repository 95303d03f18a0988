"""CPU oracle for the block-quantized matmul -- TEST INFRASTRUCTURE ONLY.

Plain f64 reference (``qmm_oracle.c``) for y = x * W^T over GGUF Q4_0 / Q8_0
weight blocks and Q4_K super-blocks, plus the error-bound scale
s = sum_k |x_k * w_k|. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the product path (the HIP library and its binding) never does, and
the two share no code.

Build: ``python -m oracle.build`` (gcc, OpenMP), also run by the package
build entry point.
"""

from __future__ import annotations

import ctypes
import os
import pathlib

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
SOURCE = HERE / "qmm_oracle.c"
LIBRARY = HERE / "libqmm_oracle.so"

# format -> (weights per block, bytes per block)
_FMT_BLOCK = {"q4_0": (32, 18), "q8_0": (32, 34), "q4_k": (256, 144)}


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: os.PathLike | str = LIBRARY):
        path = pathlib.Path(path)
        if not path.exists():
            raise FileNotFoundError(
                f"oracle library {path} is not built; run `python -m oracle.build`")
        self.path = path
        lib = ctypes.CDLL(str(path))
        i64, f32p, u8p, f64p, i64p = (ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p)
        lib.qmm_oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.qmm_oracle_half_to_double.restype = ctypes.c_double
        for name in ("qmm_oracle_q4_0", "qmm_oracle_q8_0", "qmm_oracle_q4_k"):
            fn = getattr(lib, name)
            fn.argtypes = [f32p, u8p, i64, i64, i64, f64p, f64p]
            fn.restype = None
        for name in ("qmm_oracle_q4_0_at", "qmm_oracle_q8_0_at", "qmm_oracle_q4_k_at"):
            fn = getattr(lib, name)
            fn.argtypes = [f32p, u8p, i64, i64p, i64p, i64, f64p, f64p]
            fn.restype = None
        lib.qmm_oracle_threads.argtypes = []
        lib.qmm_oracle_threads.restype = ctypes.c_int
        lib.qmm_oracle_gelu_tanh.argtypes = [ctypes.c_double]
        lib.qmm_oracle_gelu_tanh.restype = ctypes.c_double
        lib.qmm_oracle_ffn_gate_up_q4_0.argtypes = [f32p, u8p, u8p, i64, i64, i64,
                                                    f64p, f64p, f64p, f64p, f64p]
        lib.qmm_oracle_ffn_gate_up_q4_0.restype = None
        self._lib = lib

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _operands(fmt, x, w, n, k):
        x = np.ascontiguousarray(x, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        if x.ndim != 2 or x.shape[1] != k:
            raise ValueError(f"x shape {x.shape} does not match K={k}")
        per, nbytes = _FMT_BLOCK[fmt]
        if k % per:
            raise ValueError(f"K must be a multiple of {per} for {fmt}")
        row = k // per * nbytes
        if w.size != n * row:
            raise ValueError(f"w has {w.size} bytes, expected {n * row}")
        return x, w

    def half_to_double(self, bits: int) -> float:
        return self._lib.qmm_oracle_half_to_double(bits)

    def threads(self) -> int:
        return self._lib.qmm_oracle_threads()

    def matmul(self, fmt: str, x: np.ndarray, w: np.ndarray, n: int, k: int):
        """Full ``(y, s)``, both ``float64[M, N]``."""
        x, w = self._operands(fmt, x, w, n, k)
        m = x.shape[0]
        y = np.empty((m, n), dtype=np.float64)
        s = np.empty((m, n), dtype=np.float64)
        if m and n:
            fn = getattr(self._lib, f"qmm_oracle_{fmt}")
            fn(x.ctypes.data, w.ctypes.data, m, n, k, y.ctypes.data, s.ctypes.data)
        return y, s

    def gelu_tanh(self, g: float) -> float:
        return self._lib.qmm_oracle_gelu_tanh(g)

    def ffn_gate_up(self, x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, n: int,
                    k: int):
        """Gated FFN front half over Q4_0 weights: ``(h, g, u, s_g, s_u)``,
        each ``float64[M, N]``, with h = gelu_tanh(g) * u."""
        x, wg = self._operands("q4_0", x, w_gate, n, k)
        _, wu = self._operands("q4_0", x, w_up, n, k)
        m = x.shape[0]
        out = [np.empty((m, n), dtype=np.float64) for _ in range(5)]
        if m and n:
            self._lib.qmm_oracle_ffn_gate_up_q4_0(
                x.ctypes.data, wg.ctypes.data, wu.ctypes.data, m, n, k,
                *(a.ctypes.data for a in out))
        return tuple(out)

    def matmul_at(self, fmt: str, x: np.ndarray, w: np.ndarray, n: int, k: int,
                  ms, ns):
        """``(y, s)`` at the sampled output positions ``(ms[i], ns[i])``."""
        x, w = self._operands(fmt, x, w, n, k)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        if ms.shape != ns.shape or ms.ndim != 1:
            raise ValueError("ms and ns must be 1-D and of equal length")
        if ms.size and (ms.min() < 0 or ms.max() >= x.shape[0] or ns.min() < 0
                        or ns.max() >= n):
            raise ValueError("sample index out of range")
        y = np.empty(ms.size, dtype=np.float64)
        s = np.empty(ms.size, dtype=np.float64)
        if ms.size:
            fn = getattr(self._lib, f"qmm_oracle_{fmt}_at")
            fn(x.ctypes.data, w.ctypes.data, k, ms.ctypes.data, ns.ctypes.data,
               ms.size, y.ctypes.data, s.ctypes.data)
        return y, s


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from ``qmm_oracle.c`` in this directory."""
    global _default
    if _default is None:
        _default = Oracle(LIBRARY)
    return _default


def q4_0(x, w, n, k):
    return load().matmul("q4_0", x, w, n, k)


def q8_0(x, w, n, k):
    return load().matmul("q8_0", x, w, n, k)


def q4_k(x, w, n, k):
    return load().matmul("q4_k", x, w, n, k)
