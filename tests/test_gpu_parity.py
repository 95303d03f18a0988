"""GPU parity: the HIP kernels (through the C-ABI binding) against the f64
CPU oracle, element by element, on seeded inputs.

Acceptance per output, with s = sum_k |x_k w_k| from the oracle:
    |y - y_ref| <= tau * s,   tau = 1e-4 (GEMV paths) or 8e-3 (bf16 GEMM);
no NaN/Inf where y_ref is finite; exact cases must match bitwise.
"""

import sys

import numpy as np
import pytest
import torch

import block_quantized_matmul_q4_amd as qmm
import bounds
import oracle
import pins
import synth

pytestmark = pytest.mark.gpu

TAU_GEMV = 1e-4
TAU_GEMM = 8e-3
BYTES = {"q4_0": 18, "q8_0": 34}      # per 32 weights (Q4_K: 144 per 256, the same rate)


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def weights(fmt, n, k, seed=0):
    if fmt == "q4_k":
        return synth.q4_k_weights(n, k, seed)
    return synth.q4_0_weights(n, k, seed) if fmt == "q4_0" else synth.q8_0_weights(n, k, seed)


def run(entry, fmt, x, w, n, k):
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(w).reshape(-1)).cuda()
    fn = {"gemv_q4_0": qmm.gemv_q4_0, "gemv_q8_0": qmm.gemv_q8_0,
          "gemm_q4_0": qmm.gemm_q4_0, "gemm_q8_0": qmm.gemm_q8_0,
          "gemv_q4_k": qmm.gemv_q4_k, "gemm_q4_k": qmm.gemm_q4_k}[f"{entry}_{fmt}"]
    y = fn(xt, wt, n, k)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_parity(y, yref, s, tau, what):
    assert y.shape == yref.shape, what
    finite = np.isfinite(yref)
    assert np.all(np.isfinite(y[finite])), f"{what}: non-finite output"
    err = np.abs(y.astype(np.float64) - yref)
    bound = tau * s
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)), y.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of bound; worst at {i}: "
                             f"y={y[i]!r} ref={yref[i]!r} err={err[i]:.3e} bound={bound[i]:.3e}")
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0


def check(orc, entry, fmt, m, n, k, seed=0, x=None, w=None):
    tau = TAU_GEMM if entry == "gemm" else TAU_GEMV
    what = f"{entry}_{fmt} M={m} N={n} K={k} seed={seed}"
    note(f"[parity] {what}")
    if x is None:
        x = synth.activations(m, k, seed)
    if w is None:
        w = weights(fmt, n, k, seed)
    y = run(entry, fmt, x, w, n, k)
    yref, s = orc.matmul(fmt, x, w, n, k)
    return assert_parity(y, yref, s, tau, what)


# ---------------------------------------------------------------------------
# The workloads at full size
# ---------------------------------------------------------------------------

def test_gemv_tiny(orc):
    check(orc, "gemv", "q4_0", 1, 256, 512)


@pytest.mark.parametrize("n,k", [(8192, 2048), (2048, 8192)], ids=["ffn_up", "ffn_down"])
def test_gemv_decode_pair(orc, n, k):
    check(orc, "gemv", "q4_0", 1, n, k)


@pytest.mark.parametrize("m", [2, 4, 8, 16])
def test_gemv_small_m(orc, m):
    check(orc, "gemv", "q4_0", m, 8192, 2048)


def test_gemv_q8_vocab(orc):
    check(orc, "gemv", "q8_0", 1, 262144, 2048)


@pytest.mark.parametrize("m", [2, 4])
def test_gemv_q8_vocab_multi_token(orc, m):
    # k + 1 tokens through the vocabulary head (multi-token prediction
    # verification with k = 1, 3)
    check(orc, "gemv", "q8_0", m, 262144, 2048)


def test_gemm_prefill(orc):
    check(orc, "gemm", "q4_0", 2048, 8192, 2048)


def test_gemm_prefill_q8_0(orc):
    # the prefill shape over Q8_0 weights (a Q8_0 projection over many tokens)
    check(orc, "gemm", "q8_0", 2048, 8192, 2048)


# ---------------------------------------------------------------------------
# Ragged and odd shapes (several tiles plus a tail)
# ---------------------------------------------------------------------------

GEMV_SHAPES = [
    (1, 1, 256), (1, 3, 512), (1, 17, 768), (1, 257, 2304), (1, 1000, 8192),
    (1, 333, 4096), (1, 65, 16384), (1, 50, 65536), (1, 4097, 1280),
    (2, 1, 256), (3, 257, 768), (5, 1000, 2048), (7, 17, 2304), (11, 130, 512),
    (16, 33, 8192), (16, 1, 256), (13, 4100, 1024),
    (1, 65539, 1280), (1, 4100, 8192), (1, 4099, 8448), (1, 2049, 4352),
    # 2-4 rows on the f32 FMA kernel: every K branch, ragged N and K, a
    # clamped third row (M = 3 runs four), N >= 65536; 3-4 rows on the
    # matrix cores (large matrices, 2048 < N < 4096, N <= 2048 past K = 8192)
    (2, 100, 1024), (4, 17, 512), (2, 1000, 2048), (4, 1000, 2048), (3, 333, 4096),
    (2, 2049, 8192), (4, 65, 16384), (3, 4099, 8448), (2, 65539, 1280), (3, 65537, 2048),
    (4, 4096, 4096), (3, 9000, 5120), (4, 4100, 4160), (4, 2560, 6912), (3, 3000, 3072),
    (4, 2049, 2816), (4, 1536, 8960), (3, 2048, 10240), (4, 16400, 1536), (3, 40000, 2048),
    # 5-16 rows with N < 8192 (16-row matrix-core workgroups)
    (5, 2048, 8192), (12, 2049, 8448),
    # K at its maximum on the multi-row kernels
    (2, 40, 65536), (8, 65, 65536), (16, 33, 65536),
    # one row, wide N, K <= 4096 (32 lanes x 2 chunks per row, ragged K)
    (1, 32769, 3328),
    # 9-16 rows on the 32-row weight slices (8 waves from N = 8192, 16
    # below; above N = 4096, and from N = 3072 at K <= 2048): ragged M and
    # N, K steps not a multiple of the waves, wide N
    (9, 8193, 1024), (12, 8192, 8448), (16, 65537, 512), (13, 9000, 256),
    (12, 5000, 8192), (16, 3072, 2048), (10, 7000, 4352), (14, 4097, 14336), (9, 3100, 1280),
    # K > 4096 from N = 4096 (64 threads per row looping over K; two weight
    # rows per thread at M = 4, and at M = 2 from N = 8192, K = 8192): ragged
    # N and a last chunk of 1-8 pairs
    (1, 8193, 4160), (2, 8200, 8448), (2, 9000, 5120), (4, 4097, 4160), (3, 8193, 8704),
    # 5-16 rows on the 16x16 kernel with next-slice prefetch: 2-wave
    # workgroups from N = 65536 (several slices per wave), 32 weight rows at
    # K = 2048 (ragged N) and without prefetch over two slices per wave, and
    # 9-16 rows up to N = 4096 over a ragged number of slices per wave
    (6, 65537, 1024), (7, 65536, 2560), (8, 8200, 2048), (6, 8192, 4096), (10, 4096, 14336),
    (16, 2048, 8448), (16, 4096, 8192), (12, 3071, 2048),
    # 5-8 rows between N = 4096 and 8192: 32-row workgroups (Q8_0: 16 rows
    # in 4 waves), ragged N, with and without prefetch; 9-16 rows there on
    # the weight slices
    (6, 5000, 2048), (7, 6000, 4352), (12, 6000, 1024), (16, 4097, 2304),
    # 5-8 rows over wide matrices: 16 rows in 4 waves up to N = 12288, 32
    # rows in 4 waves up to 16384, then 2 waves (Q8_0: 16 rows in 4 waves)
    (6, 10000, 2304), (8, 12289, 2304), (5, 14336, 4096), (7, 20000, 4096),
    # K a multiple of 64 but not of 256 (pair counts 1, 5, 14, 17, 47)
    (1, 300, 64), (1, 4097, 896), (2, 1000, 320), (3, 2049, 1088), (4, 65537, 896),
    (6, 500, 896), (8, 8192, 3008), (12, 700, 320), (16, 9000, 1088),
]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("m,n,k", GEMV_SHAPES)
def test_gemv_shapes(orc, fmt, m, n, k):
    check(orc, "gemv", fmt, m, n, k, seed=m * 7 + n)


# Up to 4 rows run the f32 FMA kernel with each pair decoded once for all
# rows, in the same order of operations as a one-row call: where both use
# the same threads per row (every K branch, N < 65536), each row of a
# multi-row result equals the one-row result bit for bit. Three and four
# rows at some shapes (K % 256 == 0 and K, N >= 4096; K > 2048 with
# 2048 < N < 4096; 1024 <= N <= 2048 just past K = 8192) take the matrix
# cores instead; there only two rows are compared.
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("n,k", [(1000, 1024), (8192, 2048), (333, 4096), (4099, 8448),
                                 (8200, 8448), (2049, 8192), (4100, 8256), (4095, 8448),
                                 (3000, 3072), (2048, 8192), (3000, 2048),
                                 (1536, 8960), (1024, 9728), (2048, 11520), (16384, 2048),
                                 (20000, 1536)])
def test_gemv_rows_match_single_row_bitwise(fmt, n, k):
    note(f"[bitwise] gemv_{fmt} rows vs single-row calls N={n} K={k}")
    x = synth.activations(4, k, seed=n)
    w = weights(fmt, n, k, seed=n + 1)
    single = np.stack([run("gemv", fmt, x[m:m + 1], w, n, k)[0] for m in range(4)])
    large = (n >= 4096 and k >= 4096) or (2048 < n < 4096 and k > 2048) or \
        (1024 <= n <= 2048 and 8192 < k <= (11264 if fmt == "q4_0" else 9216)) or \
        (fmt == "q4_0" and n >= 16384 and k >= 1536)
    matrix_cores = large and k % 256 == 0
    for m in ((2,) if matrix_cores else (2, 3, 4)):
        y = run("gemv", fmt, x[:m], w, n, k)
        assert np.array_equal(y.view(np.uint32), single[:m].view(np.uint32)), \
            f"M={m}: {int((y != single[:m]).sum())} outputs differ from one-row calls"


# The GEMM entry points hand M <= 4, and M <= 16 with N <= 4096, to the
# GEMV's kernels: the same launches, so the same bits.
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("m,n,k", [(1, 1000, 2048), (2, 257, 1024), (3, 333, 4096),
                                   (4, 2049, 8192), (4, 4096, 4096), (3, 8192, 8448),
                                   (5, 2048, 8192), (12, 4096, 2048), (16, 300, 320)])
def test_gemm_small_m_is_gemv(fmt, m, n, k):
    note(f"[bitwise] gemm_{fmt} vs gemv_{fmt} M={m} N={n} K={k}")
    x = synth.activations(m, k, seed=n)
    w = weights(fmt, n, k, seed=n + 2)
    yg = run("gemm", fmt, x, w, n, k)
    yv = run("gemv", fmt, x, w, n, k)
    assert np.array_equal(yg.view(np.uint32), yv.view(np.uint32))


GEMM_SHAPES = [(1, 1, 256), (5, 100, 768), (127, 129, 256), (129, 300, 2048),
               (300, 17, 512), (256, 256, 4096), (1000, 520, 1280), (17, 2049, 256),
               # medium M: 64-row bands (N >= 4096), 32-row bands, more waves
               # than K steps (K = 256), K steps not a multiple of the waves
               (64, 4100, 1024), (100, 8193, 2048), (33, 2048, 8448), (128, 300, 256),
               (6, 64, 256), (128, 4096, 512),
               # K a multiple of 64 but not of 256: odd step counts on the
               # tile kernels (15, 17, 1), medium M, GEMV routing
               (300, 300, 960), (1000, 520, 1088), (2100, 4100, 1088), (129, 257, 64),
               (40, 8192, 896), (3, 100, 320),
               # medium M from N = 4096, one shape per launch choice: 32 x 32,
               # 64 x 32, 32 x 64 and 64 x 64 (8 waves) and 64 x 64 with 4
               # waves (more than 256 workgroups in every shape), ragged edges
               (20, 5000, 512), (70, 4090, 512), (64, 4100, 1024), (80, 8150, 512),
               (100, 8193, 2048),
               # more than 128 rows over at most 128 tiles of 128 x 128 (the
               # medium-M kernel's 64 x 64 tiles, 8 and 4 waves)
               (160, 4096, 1024), (200, 8150, 512), (300, 4100, 1024),
               # below N = 4096: fewer than 128 such tiles (the medium-M
               # kernel's shape rule: 32 x 32 and 64 x 64 tiles) and more
               # (the 128 x 128 tile kernel)
               (160, 1000, 4096), (300, 3000, 1024), (2100, 1030, 512)]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_shapes(orc, fmt, m, n, k):
    check(orc, "gemm", fmt, m, n, k, seed=m + n)


# Shapes with at least 192 tiles of 256 x 256 (the large-tile kernel; the
# shapes above use the 128 x 128 one), with ragged M and N edges; 220 tiles
# (fewer than compute units) in the last.
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("m,n,k", [(4097, 4100, 256), (4000, 4353, 512), (4097, 4100, 320),
                                   (1000, 14000, 256)])
def test_gemm_large_tile_shapes(orc, fmt, m, n, k):
    check(orc, "gemm", fmt, m, n, k, seed=m + n)


# K at its maximum (65536) on each GEMM kernel: the medium-M bands and the
# 128 x 128 tile against the full oracle result, the 256 x 256 tile at the
# prefill workload's M and N on sampled outputs (corners included).
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q4_k"])
@pytest.mark.parametrize("m,n", [(40, 257), (130, 257)])
def test_gemm_max_k(orc, fmt, m, n):
    check(orc, "gemm", fmt, m, n, 65536, seed=m + n)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q4_k"])
def test_gemm_max_k_large_tiles_sampled(orc, fmt):
    m, n, k = 2048, 8192, 65536
    what = f"gemm_{fmt} M={m} N={n} K={k} seed=5 (sampled)"
    note(f"[parity] {what}")
    x = synth.activations(m, k, seed=5)
    w = weights(fmt, n, k, seed=5)
    y = run("gemm", fmt, x, w, n, k)
    assert np.all(np.isfinite(y)), what
    rng = np.random.default_rng(5)
    ms = np.concatenate([[0, m - 1, 0, m - 1, 255, 256], rng.integers(0, m, 58)])
    ns = np.concatenate([[0, n - 1, n - 1, 0, 256, 255], rng.integers(0, n, 58)])
    yref, s = orc.matmul_at(fmt, x, w, n, k, ms, ns)
    assert_parity(y[ms, ns], yref, s, TAU_GEMM, what)


# the medium-M kernel's 64-column slices (8 and 4 waves) at the largest K,
# on sampled outputs (corners included)
@pytest.mark.parametrize("fmt", ["q4_0", "q4_k"])
@pytest.mark.parametrize("m,n", [(80, 8150), (100, 8193)])
def test_gemm_mid_max_k_sampled(orc, fmt, m, n):
    k = 65536
    what = f"gemm_{fmt} M={m} N={n} K={k} seed=6 (sampled)"
    note(f"[parity] {what}")
    x = synth.activations(m, k, seed=6)
    w = weights(fmt, n, k, seed=6)
    y = run("gemm", fmt, x, w, n, k)
    assert np.all(np.isfinite(y)), what
    rng = np.random.default_rng(6)
    ms = np.concatenate([[0, m - 1, 0, m - 1, 63, 64], rng.integers(0, m, 58)])
    ns = np.concatenate([[0, n - 1, n - 1, 0, 63, 64], rng.integers(0, n, 58)])
    yref, s = orc.matmul_at(fmt, x, w, n, k, ms, ns)
    assert_parity(y[ms, ns], yref, s, TAU_GEMM, what)


@pytest.mark.parametrize("m,n,k", [(2048, 2048, 8192), (255, 8191, 1024)])
def test_gemm_small_tile_full_k(orc, m, n, k):
    # fewer than 256 large tiles: 128 x 128 tiles, long K and a ragged edge
    check(orc, "gemm", "q4_0", m, n, k, seed=m + n)


def test_q4_0_vs_q8_0_scale_distributions(orc):
    # the Q4_0 scale recipe on Q8_0 bytes and vice versa (wider/narrower d)
    w = synth.q8_0_weights(512, 2048, seed=5, sigma=0.02)
    check(orc, "gemv", "q8_0", 1, 512, 2048, w=w)
    w = synth.q4_0_weights(512, 2048, seed=5, sigma=0.005)
    check(orc, "gemv", "q4_0", 3, 512, 2048, w=w)


# ---------------------------------------------------------------------------
# Exact cases: the GPU must reproduce the oracle bitwise
# ---------------------------------------------------------------------------

def pad_golden(g, k=256):
    """Embed a golden case in K=256 (zero blocks, zero activations)."""
    bs = BYTES["q4_0" if g["fmt"] == "q4_k" else g["fmt"]]
    n, k0 = g["N"], g["K"]
    w = np.zeros((n, k // 32 * bs), np.uint8)
    w[:, : k0 // 32 * bs] = g["w"].reshape(n, -1)
    x = np.zeros((g["M"], k), np.float32)
    x[:, :k0] = g["x"]
    return x, w


GOLDEN_RUNS = [(path, entry) for path in pins.golden_cases() for entry in ("gemv", "gemm")]


@pytest.mark.parametrize("path,entry", GOLDEN_RUNS, ids=lambda v: getattr(v, "name", v))
def test_golden_on_gpu(orc, path, entry):
    """Hand-derived blocks (embedded in K=256 with zero padding) against their
    exact values: within the contract bound, and bitwise where the exact value
    is an integer (every partial sum is then exact in f32) and, for the GEMM,
    every weight is exact in bf16."""
    g = pins.load_golden(path)
    x, w = pad_golden(g)
    note(f"[golden] {path.name} {entry}")
    if g["fmt"] == "q4_k" and entry == "gemv":   # one activation row per call
        y = np.concatenate([run(entry, "q4_k", x[i:i + 1], w, g["N"], 256)
                            for i in range(g["M"])]).reshape(1, -1)
    else:
        y = run(entry, g["fmt"], x, w, g["N"], 256).reshape(1, -1)
    exact = np.array([[float(v) for v in g["y"]]])
    _, s = orc.matmul(g["fmt"], x, w, g["N"], 256)
    s = s.reshape(y.shape)
    assert_parity(y, exact, s, TAU_GEMM if entry == "gemm" else TAU_GEMV, path.name)
    if entry == "gemm" and g["fmt"] == "q4_k":
        return  # weights like 63 * 13 - 1 = 818 need 9 bits: not exact in bf16
    integral = np.array([v.denominator == 1 for v in g["y"]])
    assert np.array_equal(y[0][integral], exact[0][integral])


@pytest.mark.parametrize("entry,fmt,m", [("gemv", "q4_0", 1), ("gemv", "q4_0", 4),
                                         ("gemv", "q8_0", 1), ("gemv", "q8_0", 16),
                                         ("gemm", "q4_0", 64), ("gemm", "q8_0", 70)])
def test_one_hot_exact(orc, entry, fmt, m):
    n, k = 96, 512
    rng = np.random.default_rng(11)
    d = pins.random_fp16(rng, (n, k // 32))
    d = np.clip(d.astype(np.float32), -60000, 60000).astype(np.float16)
    q = (rng.integers(0, 16, (n, k), dtype=np.uint8) if fmt == "q4_0"
         else rng.integers(-128, 128, (n, k), dtype=np.int8))
    w = pins.pack(fmt, d, q)
    ks = rng.integers(0, k, m)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), ks] = 1.0
    note(f"[exact] one-hot {entry} {fmt} M={m}")
    y = run(entry, fmt, x, w, n, k).astype(np.float64)
    yref, _ = orc.matmul(fmt, x, w, n, k)
    if entry == "gemv":
        assert np.array_equal(y, yref.astype(np.float32).astype(np.float64))
    else:  # bf16(d * (q - 8)) or bf16(d * q) exactly
        want = torch.from_numpy(yref.astype(np.float32)).to(torch.bfloat16).float().numpy()
        assert np.array_equal(y, want.astype(np.float64))


@pytest.mark.parametrize("entry,fmt,m", [("gemv", "q4_0", 1), ("gemv", "q4_0", 9),
                                         ("gemv", "q8_0", 1), ("gemv", "q8_0", 5),
                                         ("gemm", "q4_0", 33), ("gemm", "q8_0", 33)])
def test_integer_exact(orc, entry, fmt, m):
    n, k = 200, 2048
    rng = np.random.default_rng(12)
    d = np.ones((n, k // 32), np.float16)
    q = (rng.integers(0, 16, (n, k), dtype=np.uint8) if fmt == "q4_0"
         else rng.integers(-128, 128, (n, k), dtype=np.int8))
    x = rng.integers(-8, 9, (m, k)).astype(np.float32)
    w = pins.pack(fmt, d, q)
    note(f"[exact] integer {entry} {fmt} M={m}")
    y = run(entry, fmt, x, w, n, k)
    yref, _ = orc.matmul(fmt, x, w, n, k)
    assert np.array_equal(y.astype(np.float64), yref)


@pytest.mark.parametrize("entry,m", [("gemv", 1), ("gemv", 6), ("gemm", 40)])
def test_zero_point_exact(entry, m):
    n, k = 100, 1024
    rng = np.random.default_rng(13)
    d = pins.random_fp16(rng, (n, k // 32))
    w = synth.pack_q4_0(d, np.full((n, k), 8, np.uint8))
    x = (rng.standard_normal((m, k)) * 100).astype(np.float32)
    note(f"[exact] all-8 nibbles {entry} M={m}")
    y = run(entry, "q4_0", x, w, n, k)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("entry,m", [("gemv", 1), ("gemv", 2), ("gemm", 17)])
def test_subnormal_scale_exact(entry, m):
    n, k = 4, 256
    bits = np.array([0x0001, 0x03FF, 0x8001, 0x0200], np.uint16)
    d = np.repeat(bits[:, None], k // 32, axis=1).view(np.float16)
    w = synth.pack_q4_0(d, np.full((n, k), 15, np.uint8))
    x = np.ones((m, k), np.float32)
    note(f"[exact] subnormal d {entry} M={m}")
    y = run(entry, "q4_0", x, w, n, k)
    f = (bits & 0x3FF).astype(np.float64) * np.where(bits & 0x8000, -1, 1)
    want = 7 * k * f * 2.0 ** -24
    if entry == "gemm":
        want = torch.from_numpy((7 * f * 2.0 ** -24).astype(np.float32)).to(
            torch.bfloat16).double().numpy() * k
    assert np.array_equal(y, np.broadcast_to(want, (m, n)).astype(np.float32))


def test_linear_in_d_bitwise():
    n, k = 300, 2048
    d, q = synth.q4_0_fields(n, k, seed=3)
    d2 = (d.astype(np.float64) * 2).astype(np.float16)
    x = synth.activations(4, k, seed=3)
    for m in (1, 4):
        note(f"[exact] linear in d M={m}")
        y1 = run("gemv", "q4_0", x[:m], synth.pack_q4_0(d, q), n, k)
        y2 = run("gemv", "q4_0", x[:m], synth.pack_q4_0(d2, q), n, k)
        assert np.array_equal(y2, 2 * y1)


# ---------------------------------------------------------------------------
# Gated FFN front half (M = 1)
# ---------------------------------------------------------------------------

GELU_SLOPE = 1.13    # max |d gelu_tanh / dg| over the reals (about 1.129)


def ffn_bound(g, u, sg, su, h):
    """|h - h_exact| bound: g and u within the GEMV contract (1e-4 of their
    abs-sums), propagated through gelu(g) * u with gelu's slope <= 1.13, plus
    f32 evaluation of the activation: 1 + tanh carries about one f32 ulp of
    1 (times |g| / 2), and a few ulps relative to h."""
    act = np.abs(0.5 * g * (1 + np.tanh(np.sqrt(2 / np.pi) * (g + 0.044715 * g ** 3))))
    prop = TAU_GEMV * (GELU_SLOPE * np.abs(u) * sg + (act + TAU_GEMV * GELU_SLOPE * sg) * su)
    return prop + 2.0 ** -20 * (np.abs(g) + 1) * np.abs(u) + 1e-5 * np.abs(h)


def run_ffn(x, wg, wu, n, k):
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    gt = torch.from_numpy(np.ascontiguousarray(wg).reshape(-1)).cuda()
    ut = torch.from_numpy(np.ascontiguousarray(wu).reshape(-1)).cuda()
    h = qmm.ffn_gate_up_q4_0(xt, gt, ut, n, k)
    torch.cuda.synchronize()
    return h.cpu().numpy()


@pytest.mark.parametrize("n,k", [(8192, 2048), (1, 256), (1000, 256), (333, 512), (257, 1024),
                                 (4097, 1280), (100, 4096), (2048, 8192), (65, 16384),
                                 (8200, 4352), (1000, 896), (300, 64), (4099, 5120),
                                 (4096, 14336)])
def test_ffn_gate_up(orc, n, k):
    note(f"[parity] ffn_gate_up_q4_0 N={n} K={k}")
    x = synth.activations(1, k, seed=n)
    wg, wu = synth.q4_0_weights(n, k, seed=n), synth.q4_0_weights(n, k, seed=n + 1)
    h = run_ffn(x, wg, wu, n, k)
    href, g, u, sg, su = orc.ffn_gate_up(x, wg, wu, n, k)
    err = np.abs(h.astype(np.float64) - href)
    bound = ffn_bound(g, u, sg, su, href)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{int(bad.sum())} outputs out of bound; worst err/bound "
                           f"{float(np.max(err / bound)):.3g}")


# Two to four tokens: every launch branch of the gated table (K = 64 to
# 16384, N >= 4096 with K = 8192), ragged N, M = 3 (four rows run, three
# stored); 5-16 tokens, and 3-4 from K = 4096 and N = 3072 outside
# 4096 < N < 8192, on the matrix cores (hi and lo terms packed up to 8 rows,
# apart above; each launch shape of the gated table; the weight slices),
# ragged N, N = 1, deep K
FFN_ROWS_SHAPES = [(2, 8192, 2048), (4, 8192, 2048), (4, 2048, 8192), (3, 1000, 256),
                   (2, 333, 512), (3, 257, 1024), (4, 100, 4096), (3, 65, 16384),
                   (2, 8200, 4352), (4, 300, 64), (3, 1, 256), (4, 9000, 8192),
                   (5, 8192, 2048), (8, 8192, 2048), (9, 8192, 2048), (16, 8192, 2048),
                   (6, 333, 512), (12, 1000, 1024), (7, 8200, 4352), (16, 65, 16384),
                   (9, 1, 256), (8, 4100, 8192), (4, 6000, 8192), (3, 3072, 4096),
                   (6, 12000, 2048), (5, 21000, 1024), (10, 5000, 1024),
                   # the gated weight slices (9-16 rows where the GEMV takes
                   # them, 5-16 rows for K not a multiple of 256)
                   (12, 8192, 2048), (16, 3072, 2048), (13, 4097, 8192), (10, 20000, 4096),
                   (5, 300, 320), (12, 5000, 1088), (16, 8193, 64),
                   # 3-4 tokens on either kernel at K = 1024-2048
                   (4, 6144, 2048), (3, 3072, 1024), (4, 11008, 1024), (3, 20000, 2048)]


@pytest.mark.parametrize("m,n,k", FFN_ROWS_SHAPES)
def test_ffn_gate_up_rows(orc, m, n, k):
    note(f"[parity] ffn_gate_up_q4_0 M={m} N={n} K={k}")
    x = synth.activations(m, k, seed=m + n)
    wg, wu = synth.q4_0_weights(n, k, seed=n + 2), synth.q4_0_weights(n, k, seed=n + 3)
    h = run_ffn(x, wg, wu, n, k)
    href, g, u, sg, su = orc.ffn_gate_up(x, wg, wu, n, k)
    err = np.abs(h.astype(np.float64) - href)
    bound = ffn_bound(g, u, sg, su, href)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{int(bad.sum())} outputs out of bound; worst err/bound "
                           f"{float(np.max(err / bound)):.3g}")


@pytest.mark.parametrize("m,n,k", [(2, 1000, 256), (3, 6144, 2048), (4, 2048, 8192),
                                   (4, 65, 16384), (4, 4100, 5120), (2, 8192, 2048),
                                   (4, 28672, 2048), (3, 8192, 768)])
def test_ffn_gate_up_rows_match_single_row_bitwise(m, n, k):
    x = synth.activations(m, k, seed=39)
    wg, wu = synth.q4_0_weights(n, k, seed=39), synth.q4_0_weights(n, k, seed=40)
    note(f"[bitwise] ffn_gate_up_q4_0 M={m} N={n} K={k} rows against M=1")
    h = run_ffn(x, wg, wu, n, k)
    for r in range(m):
        assert np.array_equal(h[r], run_ffn(x[r:r + 1], wg, wu, n, k)[0]), r


def test_ffn_gate_up_exact_cases(orc):
    n, k = 300, 1024
    rng = np.random.default_rng(17)
    x = synth.activations(3, k, seed=17)
    d = pins.random_fp16(rng, (n, k // 32))
    wu = synth.pack_q4_0(d, rng.integers(0, 16, (n, k), dtype=np.uint8))
    note("[exact] ffn gate all-8 nibbles")
    zero_gate = synth.pack_q4_0(d, np.full((n, k), 8, np.uint8))
    assert np.all(run_ffn(x, zero_gate, wu, n, k) == 0.0)      # gelu(0) * u
    note("[exact] ffn up all-8 nibbles")
    wg = synth.pack_q4_0(d, rng.integers(0, 16, (n, k), dtype=np.uint8))
    assert np.all(run_ffn(x, wg, zero_gate, n, k) == 0.0)      # gelu(g) * 0


# ---------------------------------------------------------------------------
# Determinism, streams, errors
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("entry,fmt,m,n,k", [("gemv", "q4_0", 1, 8192, 2048),
                                             ("gemv", "q4_0", 8, 8192, 2048),
                                             ("gemv", "q8_0", 1, 4096, 2048),
                                             ("gemm", "q4_0", 512, 1024, 2048),
                                             ("gemm", "q8_0", 300, 700, 1024),
                                             ("gemm", "q4_0", 80, 8150, 512),
                                             ("gemm", "q4_0", 100, 8193, 512),
                                             ("gemv", "q4_0", 4, 4096, 4096),
                                             ("gemv", "q8_0", 7, 20000, 1024),
                                             ("gemv", "q4_0", 12, 4096, 2048),
                                             ("gemv", "q4_k", 4, 12300, 2304),
                                             ("gemv", "q4_k", 4, 8200, 4352),
                                             ("gemm", "q8_0", 1000, 14000, 128)])
def test_bitwise_repeatable(entry, fmt, m, n, k):
    x = synth.activations(m, k, seed=21)
    w = weights(fmt, n, k, seed=21)
    note(f"[determinism] {entry}_{fmt} M={m}")
    ys = [run(entry, fmt, x, w, n, k) for _ in range(3)]
    assert all(np.array_equal(ys[0], yy) for yy in ys[1:])


def test_side_stream(orc):
    n, k = 1000, 2048
    x = synth.activations(2, k, seed=4)
    w = synth.q4_0_weights(n, k, seed=4)
    xt = torch.from_numpy(x).cuda()
    wt = torch.from_numpy(w.reshape(-1)).cuda()
    s = torch.cuda.Stream()
    note("[stream] side stream")
    with torch.cuda.stream(s):
        y1 = qmm.gemv_q4_0(xt[:1], wt, n, k)
        y2 = qmm.gemv_q4_0(xt, wt, n, k)
        y3 = qmm.gemm_q4_0(xt, wt, n, k)
    s.synchronize()
    yref, sref = orc.matmul("q4_0", x, w, n, k)
    assert_parity(y1.cpu().numpy(), yref[:1], sref[:1], TAU_GEMV, "side stream M=1")
    assert_parity(y2.cpu().numpy(), yref, sref, TAU_GEMV, "side stream M=2")
    assert_parity(y3.cpu().numpy(), yref, sref, TAU_GEMM, "side stream gemm")


def test_out_argument_overwrites():
    n, k = 64, 256
    x = torch.from_numpy(synth.activations(1, k)).cuda()
    w = torch.from_numpy(synth.q4_0_weights(n, k).reshape(-1)).cuda()
    out = torch.full((1, n), float("nan"), device="cuda")
    y = qmm.gemv_q4_0(x, w, n, k, out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr() and torch.isfinite(out).all()


def test_errors_raise_on_gpu():
    x = torch.zeros(1, 96, device="cuda")
    w = torch.zeros(8 * 3 * 18, dtype=torch.uint8, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.gemv_q4_0(x, w, 8, 96)
    assert e.value.status == qmm.QMM_EUNSUPPORTED
    x = torch.zeros(17, 256, device="cuda")
    w = torch.zeros(8 * 8 * 18, dtype=torch.uint8, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.gemv_q4_0(x, w, 8, 256)
    assert e.value.status == qmm.QMM_EINVAL


def test_randomized_wide_shapes(orc):
    """Seeded randomized differential test with wide N (4000-9000): the launch
    shapes that only wide matrices select (64-row medium-M bands, Q8_0 weight
    slices, ...), at ragged sizes."""
    rng = np.random.default_rng(77)
    for case in range(24):
        entry = "gemv" if case % 3 else "gemm"
        fmt = "q8_0" if case % 2 else "q4_0"
        m = int(rng.integers(1, 17)) if entry == "gemv" else int(rng.integers(5, 129))
        n = int(rng.integers(4000, 9001))
        k = 64 * int(rng.integers(1, 33 if entry == "gemv" else 17))
        check(orc, entry, fmt, m, n, k, seed=5000 + case)


def test_randomized_small_shapes(orc):
    """Seeded randomized differential test over many small shapes."""
    rng = np.random.default_rng(2024)
    for case in range(120):
        entry = ["gemv", "gemv", "gemm"][case % 3]
        fmt = "q8_0" if case % 2 else "q4_0"
        m = int(rng.integers(1, 17)) if entry == "gemv" else int(rng.integers(1, 200))
        n = int(rng.integers(1, 600))
        k = 256 * int(rng.integers(1, 13))
        check(orc, entry, fmt, m, n, k, seed=1000 + case)


# ---------------------------------------------------------------------------
# Q4_K super-blocks (one activation row)
# ---------------------------------------------------------------------------

Q4_K_SHAPES = [
    (8192, 2048), (2048, 8192),                      # the FFN decode pair
    (1, 256), (3, 512), (17, 768), (300, 512), (9000, 1024), (4097, 1280),
    (257, 2304), (333, 4096), (2049, 4352), (1000, 8192), (4099, 8448),
    (65, 16384), (50, 65536), (65539, 1280), (8193, 4352),
]


@pytest.mark.parametrize("n,k", Q4_K_SHAPES)
def test_gemv_q4_k_shapes(orc, n, k):
    check(orc, "gemv", "q4_k", 1, n, k, seed=n + k)


def q4_k_case(rng, n, k, d_one=False):
    ns = k // 256
    if d_one:
        d = dmin = np.ones((n, ns), np.float16)
    else:
        d = np.clip(pins.random_fp16(rng, (n, ns)).astype(np.float32), -60000, 60000)
        dmin = np.clip(pins.random_fp16(rng, (n, ns)).astype(np.float32), -60000, 60000)
        d, dmin = d.astype(np.float16), dmin.astype(np.float16)
    sc = rng.integers(0, 64, (n, ns, 8), dtype=np.uint8)
    mn = rng.integers(0, 64, (n, ns, 8), dtype=np.uint8)
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    return d, dmin, sc, mn, q


def test_gemv_q4_k_one_hot_exact(orc):
    """x = e_k selects w[n][k] = d sc q - dmin mn, rounded once to f32."""
    n, k = 96, 1024
    rng = np.random.default_rng(31)
    w = synth.pack_q4_k(*q4_k_case(rng, n, k))
    for k0 in [0, 31, 32, 63, 64, 100, 127, 128, 191, 200, 255, 256, 511, 700, 1023]:
        x = np.zeros((1, k), np.float32)
        x[0, k0] = 1.0
        note(f"[exact] q4_k one-hot k={k0}")
        y = run("gemv", "q4_k", x, w, n, k).astype(np.float64)
        yref, _ = orc.matmul("q4_k", x, w, n, k)
        assert np.array_equal(y, yref.astype(np.float32).astype(np.float64)), k0


def test_gemv_q4_k_integer_exact(orc):
    """d = dmin = 1 and integer x: every partial sum is an integer below 2^24."""
    n, k = 300, 2048
    rng = np.random.default_rng(32)
    w = synth.pack_q4_k(*q4_k_case(rng, n, k, d_one=True))
    x = rng.integers(-8, 9, (1, k)).astype(np.float32)
    note("[exact] q4_k integer")
    y = run("gemv", "q4_k", x, w, n, k)
    yref, _ = orc.matmul("q4_k", x, w, n, k)
    assert np.array_equal(y.astype(np.float64), yref)


def test_gemv_q4_k_zero_exact():
    n, k = 100, 1024
    rng = np.random.default_rng(33)
    d, dmin, sc, mn, q = q4_k_case(rng, n, k)
    w = synth.pack_q4_k(d, dmin, sc, np.zeros_like(mn), np.zeros_like(q))
    x = (rng.standard_normal((1, k)) * 100).astype(np.float32)
    note("[exact] q4_k zero nibbles and minimums")
    assert np.all(run("gemv", "q4_k", x, w, n, k) == 0.0)


def test_gemv_q4_k_repeatable_and_errors():
    n, k = 4096, 2048
    x = synth.activations(1, k, seed=34)
    w = synth.q4_k_weights(n, k, seed=34)
    note("[determinism] gemv_q4_k")
    ys = [run("gemv", "q4_k", x, w, n, k) for _ in range(3)]
    assert all(np.array_equal(ys[0], yy) for yy in ys[1:])
    xt = torch.zeros(5, 256, device="cuda")
    wt = torch.zeros(8 * 144, dtype=torch.uint8, device="cuda")
    xt = torch.zeros(17, 256, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.gemv_q4_k(xt, wt, 8, 256)
    assert e.value.status == qmm.QMM_EINVAL
    with pytest.raises(ValueError):
        qmm.gemv_q4_k(torch.zeros(1, 384, device="cuda"), wt, 8, 384)


# Two to four activation rows: every launch shape (one and several passes),
# ragged N, M = 3 (four rows run, the fourth not stored)
Q4_K_ROWS_SHAPES = [(2, 300, 512), (3, 1000, 2048), (4, 8192, 2048), (4, 2048, 8192),
                    (2, 17, 256), (3, 4099, 8448), (4, 65, 16384), (2, 50, 65536),
                    (4, 2049, 2048), (3, 9000, 1024), (4, 1000, 3840),
                    # four rows over 17-32 chunks at N = 8192: T = 16, one row per
                    # thread
                    (4, 8193, 1280),
                    # four rows, two weight rows per thread: T = 16 above N = 8192
                    # (17-128 chunks), T = 32 past 32 chunks above N = 4096, T = 64
                    # at N = 4096; ragged N
                    (3, 40000, 2048), (4, 12289, 2304), (3, 12300, 5120), (4, 16385, 2048),
                    (4, 6000, 8448), (3, 9000, 3072), (4, 11008, 2048), (4, 4100, 4608),
                    (4, 4096, 3072), (3, 4096, 7936),
                    # three and four rows on the matrix cores: 2048 < N < 4096
                    # above K = 2048, N = 4096 from K = 8192, 8192 < N <= 12288
                    # from K = 4096, any N > 2048 from K = 14336
                    (4, 2049, 4352), (3, 3000, 2304), (3, 3000, 8192), (3, 4096, 8448), (4, 8200, 8448),
                    (3, 9000, 5120), (4, 12288, 4096), (4, 6000, 14336), (3, 2050, 14336),
                    # two rows past 32 chunks above N = 4096: T = 32; at N = 4096: T = 64
                    (2, 4097, 2304), (2, 8192, 8448), (2, 4096, 4352)]


@pytest.mark.parametrize("m,n,k", Q4_K_ROWS_SHAPES)
def test_gemv_q4_k_rows(orc, m, n, k):
    check(orc, "gemv", "q4_k", m, n, k, seed=m + n + k)


# Up to 64 chunks per row (K <= 4096) the multi-row launch uses the one-row
# launch's threads per row (except four rows over 17-32 chunks from N = 8192,
# which take 16): each row then equals the one-row result bit for bit.
@pytest.mark.parametrize("m,n,k", [(2, 1000, 1024), (2, 8192, 2048), (4, 4096, 2048),
                                   (3, 333, 4096), (4, 300, 256)])
def test_gemv_q4_k_rows_match_single_row_bitwise(m, n, k):
    x = synth.activations(m, k, seed=38)
    w = synth.q4_k_weights(n, k, seed=38)
    note(f"[bitwise] gemv_q4_k M={m} N={n} K={k} rows against M=1")
    y = run("gemv", "q4_k", x, w, n, k)
    for r in range(m):
        assert np.array_equal(y[r], run("gemv", "q4_k", x[r:r + 1], w, n, k)[0]), r


# Five to sixteen activation rows (matrix-core kernels): every launch branch
# of the small-M kernel (N >= 65536 with M <= 8; N < 8192 with hi/lo packed
# (M <= 8) and apart) and the 32-row weight slices (9-16 rows from N =
# 8192), ragged N, one pass (K = 256) and the largest K. The contract's
# bound scale is sum_k (|d sc q| + |dmin mn|) |x|; on these seeded weights
# the error also stays within 1e-4 sum_k |x w|.
Q4_K_MANY_ROWS_SHAPES = [
    (5, 300, 1024), (6, 8192, 2048), (8, 2048, 8192), (7, 65539, 512), (8, 65536, 256),
    (9, 8192, 2048), (12, 2049, 4352), (16, 8192, 2048), (16, 2048, 8192), (13, 17, 256),
    (16, 50, 65536), (11, 4099, 8448), (5, 1, 256), (10, 9000, 1024), (14, 65537, 256),
    (16, 8200, 65536), (9, 8193, 256), (12, 12000, 1280), (6, 65536, 2048), (8, 8192, 4096),
    (7, 12300, 2048), (8, 10000, 1024), (6, 5000, 2048), (13, 6000, 1024), (6, 14000, 4096),
]


@pytest.mark.parametrize("m,n,k", Q4_K_MANY_ROWS_SHAPES)
def test_gemv_q4_k_many_rows(orc, m, n, k):
    seed = m + n + k
    what = f"gemv_q4_k M={m} N={n} K={k} seed={seed}"
    note(f"[parity] {what}")
    f = synth.q4_k_fields(n, k, seed)
    x = synth.activations(m, k, seed)
    w = synth.pack_q4_k(*f)
    y = run("gemv", "q4_k", x, w, n, k)
    yref, s = orc.matmul("q4_k", x, w, n, k)
    r = assert_parity(y, yref, bounds.q4_k_term_abs_sum(*f, x), TAU_GEMV, what)
    r1 = assert_parity(y, yref, s, TAU_GEMV, what + " (scale sum |x w|)")
    note(f"  max err / bound {r:.3g} (two-part scale), {r1:.3g} (sum |x w|)")


@pytest.mark.parametrize("m,n", [(5, 300), (8, 300), (9, 300), (16, 300), (8, 8192),
                                 (16, 8192), (9, 8192)])
def test_gemv_q4_k_many_rows_exact(orc, m, n):
    """5-16 rows. One-hot x: each output is the weight rounded once to f32
    (d sc and dmin mn are exact in f32, and the last step is one fused
    multiply-add). d = dmin = 1 with integer x: every partial sum is an
    integer below 2^24, so the result is exact. Zero nibbles and minimums
    give zeros. Three calls agree bit for bit."""
    k = 1024
    rng = np.random.default_rng(40 + m + n)
    w = synth.pack_q4_k(*q4_k_case(rng, n, k))
    x = np.zeros((m, k), np.float32)
    ks = rng.integers(0, k, m)
    x[np.arange(m), ks] = 1.0
    note(f"[exact] gemv_q4_k one-hot M={m} N={n}")
    y = run("gemv", "q4_k", x, w, n, k).astype(np.float64)
    yref, _ = orc.matmul("q4_k", x, w, n, k)
    assert np.array_equal(y, yref.astype(np.float32).astype(np.float64))

    d, dmin, sc, mn, q = q4_k_case(rng, n, k, d_one=True)
    w = synth.pack_q4_k(d, dmin, sc, mn, q)
    x = rng.integers(-4, 5, (m, k)).astype(np.float32)
    note(f"[exact] gemv_q4_k integer M={m} N={n}")
    ys = [run("gemv", "q4_k", x, w, n, k) for _ in range(3)]
    yref, _ = orc.matmul("q4_k", x, w, n, k)
    assert np.array_equal(ys[0].astype(np.float64), yref)
    assert all(np.array_equal(ys[0], yy) for yy in ys[1:])

    w = synth.pack_q4_k(d, dmin, sc, np.zeros_like(mn), np.zeros_like(q))
    x = (rng.standard_normal((m, k)) * 100).astype(np.float32)
    note(f"[exact] gemv_q4_k zero nibbles and minimums M={m} N={n}")
    assert np.all(run("gemv", "q4_k", x, w, n, k) == 0.0)


# Q4_K through the prefill GEMM: M <= 4, and M <= 16 with N <= 4096, take the
# GEMV (bitwise), other rows up to 128 the medium-M kernel, more the tiles
# (small and large)
Q4_K_GEMM_SHAPES = [
    (2048, 8192, 2048),                              # the prefill workload's shape
    (2, 300, 512), (4, 1000, 2048), (5, 257, 768), (33, 4097, 1024), (64, 8192, 2048),
    (128, 2049, 8192), (130, 257, 512), (300, 700, 1280), (1000, 2048, 8192),
    (512, 1024, 2048), (257, 8193, 256), (12, 5000, 1024), (16, 4096, 1024), (17, 1000, 2048),
    # the medium-M launch choices from N = 4096 (as for Q4_0)
    (20, 5000, 512), (70, 4090, 512), (80, 8150, 512), (100, 8193, 1024), (200, 8150, 512),
]


@pytest.mark.parametrize("m,n,k", Q4_K_GEMM_SHAPES)
def test_gemm_q4_k_shapes(orc, m, n, k):
    check(orc, "gemm", "q4_k", m, n, k, seed=m + n + k)


@pytest.mark.parametrize("m,n", [(1, 3000), (2, 3000), (3, 3000), (4, 3000), (5, 3000),
                                 (8, 4096), (16, 1000), (12, 2048)])
def test_gemm_q4_k_few_rows_is_gemv(m, n):
    k = 2048
    x = synth.activations(m, k, seed=35)
    w = synth.q4_k_weights(n, k, seed=35)
    note(f"[exact] gemm_q4_k M={m} is the GEMV")
    assert np.array_equal(run("gemm", "q4_k", x, w, n, k), run("gemv", "q4_k", x, w, n, k))


def test_gemm_q4_k_integer_exact(orc):
    """Weights sc q - mn with sc in {0, 1}, mn <= 15 and integer x are exact in
    bf16 and every partial sum is an integer below 2^24: the GEMM is exact."""
    n, k = 200, 2048
    rng = np.random.default_rng(36)
    ones = np.ones((n, k // 256), np.float16)
    sc = rng.integers(0, 2, (n, k // 256, 8), dtype=np.uint8)
    mn = rng.integers(0, 16, (n, k // 256, 8), dtype=np.uint8)
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    w = synth.pack_q4_k(ones, ones, sc, mn, q)
    for m in (3, 40, 300):
        x = rng.integers(-8, 9, (m, k)).astype(np.float32)
        note(f"[exact] gemm_q4_k integer M={m}")
        y = run("gemm", "q4_k", x, w, n, k)
        yref, _ = orc.matmul("q4_k", x, w, n, k)
        assert np.array_equal(y.astype(np.float64), yref), m


def test_gemm_q4_k_one_hot_is_bf16_of_weight(orc):
    n, k = 96, 1024
    rng = np.random.default_rng(37)
    w = synth.pack_q4_k(*q4_k_case(rng, n, k))
    ks = rng.integers(0, k, 40)
    x = np.zeros((40, k), np.float32)
    x[np.arange(40), ks] = 1.0
    note("[exact] gemm_q4_k one-hot")
    y = run("gemm", "q4_k", x, w, n, k).astype(np.float64)
    yref, _ = orc.matmul("q4_k", x, w, n, k)
    want = torch.from_numpy(yref.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(y, want.astype(np.float64))
