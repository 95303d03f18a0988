"""The test-side bound scale of tests/bounds.py against the oracle's s and a
hand-worked case (CPU)."""

import numpy as np

import bounds
import oracle
import synth


def test_q4_k_term_abs_sum_hand_case():
    # one super-block, one row: d = dmin = 1, sc[j] = j + 1, mn[j] = 2 j,
    # every nibble 1, x = 1: sum over the 8 sub-blocks of 32 (sc + mn)
    # = 32 * sum_j (3 j + 1) = 32 * 92
    d = dmin = np.ones((1, 1), np.float16)
    sc = (np.arange(8, dtype=np.uint8) + 1).reshape(1, 1, 8)
    mn = (2 * np.arange(8, dtype=np.uint8)).reshape(1, 1, 8)
    q = np.ones((1, 256), np.uint8)
    x = np.ones((1, 256), np.float32)
    assert bounds.q4_k_term_abs_sum(d, dmin, sc, mn, q, x)[0, 0] == 32 * 92
    # a single activation picks its own weight's two terms: column 200 is in
    # sub-block 6 (sc 7, mn 12), nibble 1, x = -3
    x = np.zeros((1, 256), np.float32)
    x[0, 200] = -3.0
    assert bounds.q4_k_term_abs_sum(d, dmin, sc, mn, q, x)[0, 0] == 3 * (7 + 12)


def test_q4_k_term_abs_sum_against_oracle():
    o = oracle.load()
    n, k, m = 37, 768, 3
    d, dmin, sc, mn, q = synth.q4_k_fields(n, k, seed=5)
    x = synth.activations(m, k, seed=5)
    _, s = o.matmul("q4_k", x, synth.pack_q4_k(d, dmin, sc, mn, q), n, k)
    t = bounds.q4_k_term_abs_sum(d, dmin, sc, mn, q, x)
    assert np.all(t >= s * (1 - 1e-12)), "triangle inequality"
    assert np.any(t > s * 1.01), "the minimums must count where they cancel"
    # no minimums: w = d sc q, and the scale is the oracle's sum |x w|
    zero = np.zeros_like(mn)
    _, s0 = o.matmul("q4_k", x, synth.pack_q4_k(d, dmin, sc, zero, q), n, k)
    t0 = bounds.q4_k_term_abs_sum(d, dmin, sc, zero, q, x)
    assert np.allclose(t0, s0, rtol=1e-12, atol=0)
    # negative scales count by magnitude
    t1 = bounds.q4_k_term_abs_sum(-d.astype(np.float32), -dmin.astype(np.float32), sc, mn, q, x)
    assert np.array_equal(t1, t)
