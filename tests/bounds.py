"""Accuracy scales that some kernels' bounds are stated in and that the
oracle's own s = sum_k |x_k w_k| does not give directly."""

import numpy as np


def q4_k_term_abs_sum(d, dmin, sc, mn, q, x):
    """sum_k (|d sc q| + |dmin mn|) |x_k| for every output (m, n), in f64.

    Takes the logical Q4_K fields (fp16 d, dmin [N, K/256]; 6-bit sc, mn
    [N, K/256, 8]; nibbles q [N, K]) and x [M, K]; returns [M, N]. This is
    the scale of the bound of a Q4_K GEMV that rounds each sub-block's
    scale part d*sc*sum(q x) and minimum part dmin*mn*sum(x) apart: it is
    at least sum_k |x w| (triangle inequality) and equals it where every
    minimum is zero."""
    n, k = q.shape
    col = np.arange(k)
    dd = np.abs(np.asarray(d, dtype=np.float64))[:, col // 256]
    dm = np.abs(np.asarray(dmin, dtype=np.float64))[:, col // 256]
    s = np.asarray(sc, dtype=np.float64).reshape(n, -1)[:, col // 32]
    m = np.asarray(mn, dtype=np.float64).reshape(n, -1)[:, col // 32]
    per_weight = dd * s * np.asarray(q, dtype=np.float64) + dm * m
    return np.abs(np.asarray(x, dtype=np.float64)) @ per_weight.T
