"""Seeded randomized differential test: 1,000 small random problems through
every entry point, each compared element by element with the f64 oracle.

Case i draws, from numpy's generator seeded with i, an entry point and a
shape: M from the entry point's range (GEMVs 1-16, GEMM 1-300, gated front
half 1-16), N in 1..1200, K a multiple of 64 (Q4_K: of 256) up to
4096, redrawn while M N K exceeds 2^24 so that the oracle stays fast; the
weights and activations come from the seeded generators with seed i. The
bound is the entry point's contract: 1e-4 sum_k |w x| for the GEMVs, 8e-3
for the GEMMs, and for the gated front half the GEMV bound on g and u
carried through the activation (slope <= 1.13) plus the f32 rounding of the
activation. The cases run in ten groups of 100 so that a failure names its
group and the first failing case.

A second set of 200 cases draws GEMMs over wide matrices (N 4000-9000, M
5-600, K up to 1024, M N K <= 2^29), the range where the GEMM's launch
choice between its medium-M shapes and its two tile sizes changes with the
shape; `route_wide` restates that choice so that the draw can be checked to
reach every branch.
"""

import numpy as np
import pytest
import torch

import block_quantized_matmul_q4_amd as qmm
import bounds
import oracle
import synth

pytestmark = pytest.mark.gpu

CASES = 1000
GROUPS = 10
ENTRIES = ("gemv_q4_0", "gemv_q8_0", "gemm_q4_0", "gemm_q8_0", "gemv_q4_k", "gemm_q4_k",
           "ffn_gate_up_q4_0")


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def draw(i):
    rng = np.random.default_rng(i)
    entry = ENTRIES[int(rng.integers(0, len(ENTRIES)))]
    fmt = entry.split("_", 1)[1] if entry != "ffn_gate_up_q4_0" else "q4_0"
    while True:
        if entry.startswith("gemv"):
            m = int(rng.integers(1, 17))
        elif entry.startswith("gemm"):
            m = int(rng.integers(1, 301))
        else:
            m = int(rng.integers(1, 17))
        n = int(rng.integers(1, 1201))
        step = 256 if fmt == "q4_k" else 64     # Q4_K super-blocks
        k = step * int(rng.integers(1, 4096 // step + 1))
        if m * n * k <= 1 << 24:
            return entry, fmt, m, n, k


def weights(fmt, n, k, seed):
    if fmt == "q4_k":
        return synth.q4_k_weights(n, k, seed)
    return synth.q4_0_weights(n, k, seed) if fmt == "q4_0" else synth.q8_0_weights(n, k, seed)


def one_case(o, i):
    entry, fmt, m, n, k = draw(i)
    x = synth.activations(m, k, seed=i)
    w = weights(fmt, n, k, seed=i)
    xt = torch.from_numpy(x).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(w).reshape(-1)).cuda()
    if entry == "ffn_gate_up_q4_0":
        wu = synth.q4_0_weights(n, k, seed=i + 100000)
        h = qmm.ffn_gate_up_q4_0(xt, wt, torch.from_numpy(wu.reshape(-1)).cuda(), n, k)
        torch.cuda.synchronize()
        href, g, u, sg, su = o.ffn_gate_up(x, w, wu, n, k)
        act = np.abs(np.array([o.gelu_tanh(v) for v in g.reshape(-1)])).reshape(g.shape)
        bound = (1e-4 * (1.13 * np.abs(u) * sg + (act + 1.13e-4 * sg) * su)
                 + 2.0 ** -20 * (np.abs(g) + 1) * np.abs(u) + 1e-5 * np.abs(href))
        y, yref = h.cpu().numpy().astype(np.float64), href
    else:
        y = getattr(qmm, entry)(xt, wt, n, k)
        torch.cuda.synchronize()
        yref, s = o.matmul(fmt, x, w, n, k)
        if entry == "gemv_q4_k" and m > 4:
            s = bounds.q4_k_term_abs_sum(*synth.q4_k_fields(n, k, seed=i), x)
        bound = (8e-3 if entry.startswith("gemm") else 1e-4) * s
        y = y.cpu().numpy().astype(np.float64)
    err = np.abs(y - yref)
    ok = bool(np.all(np.isfinite(y)) and np.all(err <= bound))
    return ok, f"case {i}: {entry} M={m} N={n} K={k}, max err/bound " \
               f"{float(np.max(err / np.maximum(bound, 1e-300))):.3g}"


@pytest.mark.parametrize("group", range(GROUPS))
def test_random_differential(orc, group):
    per = CASES // GROUPS
    print(f"[random] cases {group * per}..{group * per + per - 1}", flush=True)
    for i in range(group * per, (group + 1) * per):
        ok, what = one_case(orc, i)
        assert ok, what



WIDE_CASES = 200
WIDE_GROUPS = 4
WIDE_ENTRIES = ("gemm_q4_0", "gemm_q8_0", "gemm_q4_k")


def draw_wide(i):
    rng = np.random.default_rng(1_000_000 + i)
    entry = WIDE_ENTRIES[int(rng.integers(0, len(WIDE_ENTRIES)))]
    fmt = entry.split("_", 1)[1]
    while True:
        m = int(rng.integers(5, 601))
        n = int(rng.integers(4000, 9001))
        step = 256 if fmt == "q4_k" else 64
        k = step * int(rng.integers(1, 1024 // step + 1))
        if m * n * k <= 1 << 29:
            return entry, fmt, m, n, k


def route_wide(m, n):
    """The GEMM's launch choice for 4 < M, N >= 4096 (its launch table, restated)."""
    if m > 128:
        if -(-m // 256) * -(-n // 256) >= 192:
            return "tiles_256"
        if -(-m // 128) * -(-n // 128) > 128:
            return "tiles_128"
    best, best_wg = None, 0
    for mt, nt in ((1, 1), (2, 1), (1, 2), (2, 2)):
        wg = -(-n // (32 * nt)) * -(-m // (32 * mt))
        if wg > 256:
            continue
        if best is None or wg > best_wg or (wg == best_wg and (nt > best[1] or
                                                              (nt == best[1] and mt < best[0]))):
            best, best_wg = (mt, nt), wg
    return f"mid_{best[0]}x{best[1]}" if best else "mid_2x2_4waves"


def one_wide_case(o, i):
    entry, fmt, m, n, k = draw_wide(i)
    x = synth.activations(m, k, seed=i)
    w = weights(fmt, n, k, seed=i)
    y = getattr(qmm, entry)(torch.from_numpy(x).cuda(),
                            torch.from_numpy(np.ascontiguousarray(w).reshape(-1)).cuda(), n, k)
    torch.cuda.synchronize()
    yref, s = o.matmul(fmt, x, w, n, k)
    y = y.cpu().numpy().astype(np.float64)
    err = np.abs(y - yref)
    bound = 8e-3 * s
    ok = bool(np.all(np.isfinite(y)) and np.all(err <= bound))
    return ok, f"wide case {i}: {entry} M={m} N={n} K={k} ({route_wide(m, n)}), max err/bound " \
               f"{float(np.max(err / np.maximum(bound, 1e-300))):.3g}"


@pytest.mark.parametrize("group", range(WIDE_GROUPS))
def test_random_gemm_wide(orc, group):
    per = WIDE_CASES // WIDE_GROUPS
    print(f"[random] wide GEMM cases {group * per}..{group * per + per - 1}", flush=True)
    for i in range(group * per, (group + 1) * per):
        ok, what = one_wide_case(orc, i)
        assert ok, what

