"""Seeded synthetic inputs for the block-quantized matmul (GGUF Q4_0 / Q8_0).

This module is shared by the tests, the benchmark and the smoke check. It
draws random numbers and places block fields into bytes; it holds none of
the arithmetic of the method itself (no dequantization, no products, no
sums), so the CPU oracle and the GPU path can both consume its output
without sharing any computation.

Storage layout (GGUF block formats, as named by the quant-kernel pages
"Add generated quant-kernel JIT and accelerate Gemma4, BGE-M3, and GLiNER2",
section Validation, which counts Q4_0 and Q8_0 quant dispatches):

* Q4_0 block, 18 bytes: fp16 scale ``d`` (little-endian) followed by 16
  bytes ``qs``; element ``j`` (j < 16) is the low nibble of ``qs[j]`` and
  element ``j + 16`` is its high nibble. Nibble values are 0..15.
* Q8_0 block, 34 bytes: fp16 scale ``d`` followed by 32 signed bytes,
  element ``j`` is ``qs[j]``.
* A weight matrix with N output rows and K inputs is ``N x (K/32)`` blocks,
  rows contiguous, no padding.
* Q4_K super-block (the k-quant 4-bit format the pages keep for their
  CLIP/CLAP path, section Summary, without a layout; GGUF's is taken), 144
  bytes per 256 weights: fp16 ``d``, fp16 ``dmin``, 12 bytes holding eight
  6-bit sub-block scales ``sc`` and minimums ``mn``, then 128 nibble bytes.
  Weight ``64c + i`` (i < 32) is the low nibble of nibble byte ``32c + i``
  and weight ``64c + 32 + i`` its high nibble; weight ``e`` belongs to
  sub-block ``e // 32``. Scale bytes: ``b[j] = sc[j] | (sc[j+4] >> 4) << 6``
  and ``b[4+j] = mn[j] | (mn[j+4] >> 4) << 6`` for j < 4, and
  ``b[8+j] = (sc[j+4] & 15) | (mn[j+4] & 15) << 4``.

Distributions (the workloads of the quant-kernel pages stand-in, see the
design notes): nibbles uniform over 0..15, Q8_0 integers uniform over
-127..127, scales ``|N(0, sigma)|`` rounded to fp16 (sigma 0.02 for Q4_0,
0.005 for Q8_0), activations f32 standard normal. Q4_K (no distribution is
given for it): nibbles uniform over 0..15, sub-block scales and minimums
uniform over 0..63, ``d`` and ``dmin`` ``|N(0, 0.002)|`` rounded to fp16.
"""

from __future__ import annotations

import hashlib

import numpy as np

Q4_0_BLOCK_BYTES = 18
Q8_0_BLOCK_BYTES = 34
BLOCK = 32

# Stream tags: one independent random stream per field, so that equal
# shapes share bytes across configurations.
TAG_Q4_NIBBLES = 1
TAG_Q4_SCALES = 2
TAG_Q8_INTS = 3
TAG_Q8_SCALES = 4
TAG_X = 5
TAG_QK_NIBBLES = 6
TAG_QK_SCALES = 7
TAG_QK_SUB = 8

Q4_K_SUPER = 256
Q4_K_BYTES = 144


def _rng(seed: int, tag: int, dim0: int, k: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tag, dim0, k]))


def _check_k(k: int) -> None:
    if k <= 0 or k % BLOCK:
        raise ValueError(f"K must be a positive multiple of {BLOCK}, got {k}")


# ----------------------------------------------------------------------------
# Byte placement (encoders). Inputs are the logical field values.
# ----------------------------------------------------------------------------

def pack_q4_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Place fp16 scales ``d[N, K/32]`` and nibbles ``q[N, K]`` (0..15) into
    Q4_0 blocks. Returns ``uint8[N, K/32*18]``."""
    d = np.ascontiguousarray(d, dtype=np.float16)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, k = q.shape
    _check_k(k)
    nb = k // BLOCK
    if d.shape != (n, nb):
        raise ValueError(f"scale shape {d.shape} != {(n, nb)}")
    if q.size and int(q.max()) > 15:
        raise ValueError("Q4_0 nibble values must lie in 0..15")
    qb = q.reshape(n, nb, BLOCK)
    out = np.empty((n, nb, Q4_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = qb[:, :, :16] | (qb[:, :, 16:] << 4)
    return out.reshape(n, nb * Q4_0_BLOCK_BYTES)


def pack_q8_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Place fp16 scales ``d[N, K/32]`` and int8 values ``q[N, K]`` into Q8_0
    blocks. Returns ``uint8[N, K/32*34]``."""
    d = np.ascontiguousarray(d, dtype=np.float16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    _check_k(k)
    nb = k // BLOCK
    if d.shape != (n, nb):
        raise ValueError(f"scale shape {d.shape} != {(n, nb)}")
    out = np.empty((n, nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = q.reshape(n, nb, BLOCK).view(np.uint8)
    return out.reshape(n, nb * Q8_0_BLOCK_BYTES)


def pack_q4_k(d: np.ndarray, dmin: np.ndarray, sc: np.ndarray, mn: np.ndarray,
              q: np.ndarray) -> np.ndarray:
    """Place fp16 ``d[N, K/256]`` and ``dmin[N, K/256]``, 6-bit sub-block
    scales ``sc[N, K/256, 8]`` and minimums ``mn[N, K/256, 8]`` (0..63) and
    nibbles ``q[N, K]`` (0..15) into Q4_K super-blocks. Returns
    ``uint8[N, K/256*144]``."""
    d = np.ascontiguousarray(d, dtype=np.float16)
    dmin = np.ascontiguousarray(dmin, dtype=np.float16)
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, k = q.shape
    if k <= 0 or k % Q4_K_SUPER:
        raise ValueError(f"K must be a positive multiple of {Q4_K_SUPER}, got {k}")
    ns = k // Q4_K_SUPER
    if d.shape != (n, ns) or dmin.shape != (n, ns):
        raise ValueError(f"scale shapes {d.shape}, {dmin.shape} != {(n, ns)}")
    if sc.shape != (n, ns, 8) or mn.shape != (n, ns, 8):
        raise ValueError(f"sub-block shapes {sc.shape}, {mn.shape} != {(n, ns, 8)}")
    if (sc.size and int(sc.max()) > 63) or (mn.size and int(mn.max()) > 63):
        raise ValueError("Q4_K sub-block scales and minimums must lie in 0..63")
    if q.size and int(q.max()) > 15:
        raise ValueError("Q4_K nibble values must lie in 0..15")
    out = np.empty((n, ns, Q4_K_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(n, ns, 2)
    out[:, :, 2:4] = dmin.astype("<f2").view(np.uint8).reshape(n, ns, 2)
    out[:, :, 4:8] = sc[:, :, 0:4] | ((sc[:, :, 4:8] >> 4) << 6)
    out[:, :, 8:12] = mn[:, :, 0:4] | ((mn[:, :, 4:8] >> 4) << 6)
    out[:, :, 12:16] = (sc[:, :, 4:8] & 15) | ((mn[:, :, 4:8] & 15) << 4)
    qc = q.reshape(n, ns, 4, 64)
    out[:, :, 16:] = (qc[:, :, :, :32] | (qc[:, :, :, 32:] << 4)).reshape(n, ns, 128)
    return out.reshape(n, ns * Q4_K_BYTES)


# ----------------------------------------------------------------------------
# Seeded draws
# ----------------------------------------------------------------------------

def q4_0_fields(n: int, k: int, seed: int = 0, sigma: float = 0.02):
    """Logical Q4_0 fields: ``(d fp16[N, K/32], q uint8[N, K])``."""
    _check_k(k)
    q = _rng(seed, TAG_Q4_NIBBLES, n, k).integers(0, 16, (n, k), dtype=np.uint8)
    d = np.abs(_rng(seed, TAG_Q4_SCALES, n, k).normal(0.0, sigma, (n, k // BLOCK)))
    return d.astype(np.float16), q


def q8_0_fields(n: int, k: int, seed: int = 0, sigma: float = 0.005):
    """Logical Q8_0 fields: ``(d fp16[N, K/32], q int8[N, K])``."""
    _check_k(k)
    q = _rng(seed, TAG_Q8_INTS, n, k).integers(-127, 128, (n, k), dtype=np.int8)
    d = np.abs(_rng(seed, TAG_Q8_SCALES, n, k).normal(0.0, sigma, (n, k // BLOCK)))
    return d.astype(np.float16), q


def q4_0_weights(n: int, k: int, seed: int = 0, sigma: float = 0.02) -> np.ndarray:
    """Packed Q4_0 weights ``uint8[N, K/32*18]`` for the seeded draw."""
    return pack_q4_0(*q4_0_fields(n, k, seed, sigma))


def q8_0_weights(n: int, k: int, seed: int = 0, sigma: float = 0.005) -> np.ndarray:
    """Packed Q8_0 weights ``uint8[N, K/32*34]`` for the seeded draw."""
    return pack_q8_0(*q8_0_fields(n, k, seed, sigma))


def q4_k_fields(n: int, k: int, seed: int = 0, sigma: float = 0.002):
    """Logical Q4_K fields ``(d, dmin, sc, mn, q)``: fp16 ``d`` and ``dmin``
    ``[N, K/256]``, uint8 ``sc`` and ``mn`` ``[N, K/256, 8]`` (0..63), uint8
    ``q[N, K]`` (0..15)."""
    if k <= 0 or k % Q4_K_SUPER:
        raise ValueError(f"K must be a positive multiple of {Q4_K_SUPER}, got {k}")
    ns = k // Q4_K_SUPER
    q = _rng(seed, TAG_QK_NIBBLES, n, k).integers(0, 16, (n, k), dtype=np.uint8)
    dd = np.abs(_rng(seed, TAG_QK_SCALES, n, k).normal(0.0, sigma, (2, n, ns)))
    sub = _rng(seed, TAG_QK_SUB, n, k).integers(0, 64, (2, n, ns, 8), dtype=np.uint8)
    return (dd[0].astype(np.float16), dd[1].astype(np.float16), sub[0], sub[1], q)


def q4_k_weights(n: int, k: int, seed: int = 0, sigma: float = 0.002) -> np.ndarray:
    """Packed Q4_K weights ``uint8[N, K/256*144]`` for the seeded draw."""
    return pack_q4_k(*q4_k_fields(n, k, seed, sigma))


def activations(m: int, k: int, seed: int = 0) -> np.ndarray:
    """Activations ``float32[M, K]``, standard normal."""
    if m < 0 or k < 0:
        raise ValueError("negative shape")
    return _rng(seed, TAG_X, m, k).standard_normal((m, k)).astype(np.float32)


def sha256(a: np.ndarray) -> str:
    """Hex digest of an array's bytes (C order), for reports."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# ----------------------------------------------------------------------------
# Workloads (shapes of the decode/prefill matmuls the pages count)
# ----------------------------------------------------------------------------

WORKLOADS = {
    "q4_0_gemv_tiny": dict(fmt="q4_0", M=1, K=512, N=256),
    "q4_0_gemv_ffn_up": dict(fmt="q4_0", M=1, K=2048, N=8192),
    "q4_0_gemv_ffn_down": dict(fmt="q4_0", M=1, K=8192, N=2048),
    "q4_0_gemv_small_m2": dict(fmt="q4_0", M=2, K=2048, N=8192),
    "q4_0_gemv_small_m4": dict(fmt="q4_0", M=4, K=2048, N=8192),
    "q4_0_gemv_small_m8": dict(fmt="q4_0", M=8, K=2048, N=8192),
    "q4_0_gemv_small_m16": dict(fmt="q4_0", M=16, K=2048, N=8192),
    "q4_0_gemm_prefill": dict(fmt="q4_0", M=2048, K=2048, N=8192),
    "q8_0_gemv_vocab": dict(fmt="q8_0", M=1, K=2048, N=262144),
    "q4_k_gemv_ffn_up": dict(fmt="q4_k", M=1, K=2048, N=8192),
    "q4_k_gemv_ffn_down": dict(fmt="q4_k", M=1, K=8192, N=2048),
}


def workload_inputs(name: str, seed: int = 0):
    """``(x f32[M,K], w uint8[N, K/32*bs])`` for a named workload."""
    cfg = WORKLOADS[name]
    m, k, n = cfg["M"], cfg["K"], cfg["N"]
    if cfg["fmt"] == "q4_0":
        w = q4_0_weights(n, k, seed)
    elif cfg["fmt"] == "q4_k":
        w = q4_k_weights(n, k, seed)
    else:
        w = q8_0_weights(n, k, seed)
    return activations(m, k, seed), w
