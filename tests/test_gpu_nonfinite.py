"""Non-finite scales through every kernel (GPU against the f64 oracle).

The stated behaviour (include/qmm.h): for finite x, y[m][n] is non-finite
(NaN, +Inf or -Inf; which of them is not specified) exactly where weight
row n holds a block whose fp16 scale is +Inf, -Inf or NaN (Q4_K: d or
dmin), and every other output keeps its accuracy bound. The kind may differ
from the definition's: the f64 definition forms each weight d * (q - 8)
first, so an infinite scale over a zero code gives Inf * 0 = NaN there,
while the GEMV paths apply d to a block's partial sum and give +-Inf.

Each case plants +Inf, -Inf and NaN scales into a few rows of seeded
weights, runs one launch shape of one kernel, and checks (a) that the
oracle's non-finite outputs are exactly the planted rows (the statement
above, on the oracle side; the oracle's IEEE propagation is pinned by
``pins.special_values``), (b) that the GPU's non-finite outputs are the
same positions, and (c) the usual bound on all other outputs.
"""

import numpy as np
import pytest
import torch

import block_quantized_matmul_q4_amd as qmm
import bounds
import oracle
import synth

pytestmark = pytest.mark.gpu

TAU_GEMV = 1e-4
TAU_GEMM = 8e-3
SPECIALS = (0x7C00, 0xFC00, 0x7E00)      # +Inf, -Inf, NaN as fp16 bits


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def weights(fmt, n, k, seed):
    if fmt == "q4_k":
        return synth.q4_k_weights(n, k, seed)
    return synth.q4_0_weights(n, k, seed) if fmt == "q4_0" else synth.q8_0_weights(n, k, seed)


def plant(fmt, w, n, k, seed, rows=6):
    """Copy of w with non-finite scales in `rows` random rows; returns (w, rows)."""
    w = np.array(w, dtype=np.uint8).reshape(n, -1).copy()
    rng = np.random.default_rng(seed)
    picked = sorted(set(int(r) for r in rng.choice(n, size=min(rows, n), replace=False)))
    for i, r in enumerate(picked):
        bits = SPECIALS[i % 3]
        if fmt == "q4_k":
            sb = int(rng.integers(0, k // 256))
            off = 144 * sb + (2 if i % 2 else 0)        # d or dmin
        else:
            bs = 18 if fmt == "q4_0" else 34
            off = bs * int(rng.integers(0, k // 32))
        w[r, off] = bits & 0xFF
        w[r, off + 1] = bits >> 8
    return w.reshape(-1), picked


def expect_nonfinite(y, yref, s, tau, planted, what):
    m, n = yref.shape
    want = np.zeros((m, n), dtype=bool)
    want[:, planted] = True
    assert np.array_equal(~np.isfinite(yref), want), f"{what}: oracle non-finite positions"
    bad = ~np.isfinite(y)
    assert np.array_equal(bad, want), (
        f"{what}: GPU non-finite at {np.argwhere(bad & ~want)[:4].tolist()} (unexpected) / "
        f"finite at {np.argwhere(want & ~bad)[:4].tolist()} (expected non-finite)")
    ok = ~want
    err = np.abs(y[ok].astype(np.float64) - yref[ok])
    assert np.all(err <= tau * s[ok]), f"{what}: finite outputs out of bound"


def run(fn, x, w, n, k):
    y = fn(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), n, k)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# (entry, fmt, M, N, K): one case per kernel and launch-table branch the
# entry points route to
CASES = [
    # one-row GEMV: wave-local T = 8, shared staging T = 32, 64, 128
    ("gemv", "q4_0", 1, 300, 512), ("gemv", "q4_0", 1, 300, 2048),
    ("gemv", "q4_0", 1, 300, 4096), ("gemv", "q4_0", 1, 300, 8192),
    ("gemv", "q8_0", 1, 300, 2048), ("gemv", "q8_0", 1, 300, 8192),
    # 2-4 rows (f32 FMA kernel; M = 3 runs four rows)
    ("gemv", "q4_0", 2, 300, 2048), ("gemv", "q4_0", 3, 300, 8192),
    ("gemv", "q8_0", 4, 300, 2048),
    # 5-16 rows: the small-M matrix-core kernel and the weight-slice kernel
    ("gemv", "q4_0", 6, 300, 1024), ("gemv", "q4_0", 12, 300, 1024),
    ("gemv", "q8_0", 8, 300, 1024), ("gemv", "q8_0", 12, 8200, 256),
    # GEMM: medium M (32- and 64-row bands), 128 x 128 and 256 x 256 tiles
    ("gemm", "q4_0", 20, 300, 1024), ("gemm", "q4_0", 100, 4100, 256),
    ("gemm", "q4_0", 300, 300, 512), ("gemm", "q4_0", 2048, 8192, 64),
    ("gemm", "q8_0", 20, 300, 1024), ("gemm", "q8_0", 300, 300, 512),
    # medium M with 64-column slices (8 and 4 waves)
    ("gemm", "q4_0", 80, 8150, 256), ("gemm", "q8_0", 100, 8193, 256),
    # Q4_K: GEMV (1 and 3 rows; 8 and 12 rows on the small-M kernel, 12 on the
    # weight slices from N = 8192), medium M and tiles
    ("gemv", "q4_k", 1, 300, 2048), ("gemv", "q4_k", 3, 300, 1024),
    ("gemv", "q4_k", 8, 300, 1024), ("gemv", "q4_k", 12, 8200, 512),
    ("gemv", "q4_k", 12, 4000, 512), ("gemv", "q4_k", 4, 8200, 1280),
    ("gemm", "q4_k", 20, 300, 1024), ("gemm", "q4_k", 300, 300, 512),
    ("gemm", "q4_k", 80, 8150, 512),
    # wide-matrix branches: one row with 64 threads per row past 64 pairs,
    # two rows with two weight rows per thread, three and four rows on the
    # matrix cores, 5-8 rows in 4- and 2-wave workgroups, 9-16 rows on the
    # 16x16 kernel below N = 8192
    ("gemv", "q4_0", 1, 4100, 8192), ("gemv", "q8_0", 2, 8200, 8448),
    ("gemv", "q4_0", 4, 4100, 4352), ("gemv", "q8_0", 3, 4100, 4352),
    ("gemv", "q4_0", 6, 10000, 1024), ("gemv", "q4_0", 7, 20000, 1024),
    ("gemv", "q8_0", 6, 10000, 1024), ("gemv", "q4_0", 12, 4096, 2048),
    # Q4_K: one and two rows with T = 32 past 64 / 32 chunks, four rows with
    # two weight rows per thread (T = 16, 32, 64)
    ("gemv", "q4_k", 1, 4100, 4352), ("gemv", "q4_k", 2, 4100, 2304),
    ("gemv", "q4_k", 4, 12300, 2304), ("gemv", "q4_k", 4, 8200, 4352),
    ("gemv", "q4_k", 4, 4096, 4352),
    # GEMM: more than 128 rows over few tiles below N = 4096 (medium-M
    # kernel), 256 x 256 tiles short of one per compute unit
    ("gemm", "q4_0", 512, 1000, 1024), ("gemm", "q8_0", 1000, 14000, 128),
]


@pytest.mark.parametrize("entry,fmt,m,n,k", CASES)
def test_nonfinite_scales(orc, entry, fmt, m, n, k):
    what = f"{entry}_{fmt} M={m} N={n} K={k} with +-Inf/NaN scales"
    print(f"[nonfinite] {what}", flush=True)
    seed = m * 31 + n + k
    x = synth.activations(m, k, seed)
    w, planted = plant(fmt, weights(fmt, n, k, seed), n, k, seed)
    fn = getattr(qmm, f"{entry}_{fmt}")
    with np.errstate(invalid="ignore"):
        y = run(fn, x, w, n, k)
        yref, s = orc.matmul(fmt, x, w, n, k)
        if entry == "gemv" and fmt == "q4_k" and m > 4:
            # the matrix-core Q4_K GEMV's bound scale (the planted rows,
            # whose scales changed, are not checked against it)
            s = bounds.q4_k_term_abs_sum(*synth.q4_k_fields(n, k, seed), x)
        expect_nonfinite(y, yref, s, TAU_GEMM if entry == "gemm" else TAU_GEMV, planted, what)


@pytest.mark.parametrize("m", [1, 3, 6, 12])
@pytest.mark.parametrize("k", [1024, 2048, 8192])
@pytest.mark.parametrize("which", ["gate", "up"])
def test_nonfinite_scales_ffn_gate_up(orc, k, which, m):
    n = 4100 if k == 8192 else 300     # past 32 pairs from N = 4096: T = 32 loops over K
    what = f"ffn_gate_up_q4_0 M={m} N={n} K={k} with +-Inf/NaN scales in {which}"
    print(f"[nonfinite] {what}", flush=True)
    x = synth.activations(m, k, seed=k)
    wg, wu = synth.q4_0_weights(n, k, seed=k + 1), synth.q4_0_weights(n, k, seed=k + 2)
    if which == "gate":
        wg, planted = plant("q4_0", wg, n, k, seed=k)
    else:
        wu, planted = plant("q4_0", wu, n, k, seed=k)
    wg, wu = np.ascontiguousarray(wg).reshape(-1), np.ascontiguousarray(wu).reshape(-1)
    with np.errstate(invalid="ignore", over="ignore"):
        h = qmm.ffn_gate_up_q4_0(torch.from_numpy(x).cuda(), torch.from_numpy(wg).cuda(),
                                 torch.from_numpy(wu).cuda(), n, k)
        torch.cuda.synchronize()
        h = h.cpu().numpy()
        href = orc.ffn_gate_up(x, wg, wu, n, k)[0]
    want = np.zeros((m, n), dtype=bool)
    want[:, planted] = True
    assert np.array_equal(~np.isfinite(href), want), f"{what}: oracle non-finite positions"
    assert np.array_equal(~np.isfinite(h), want), f"{what}: GPU non-finite positions"
