"""Every kernel family captured in one HIP graph (torch.cuda.graph) and
replayed: each replay must reproduce the eager outputs bit for bit.

The graph holds one call per case below (each entry point on each of its
launch routes, each call with its own output). The outputs are computed
eagerly first, then overwritten with NaN; the graph is replayed three times,
each replay followed by a synchronization, a bitwise comparison with the
eager outputs, and eager work of the program's own (NaN fills of every
output) before the next replay. The entry points enqueue only kernels (no
memset or copy), so a captured call replays exactly what an eager one runs.
"""

import numpy as np
import pytest
import torch

import block_quantized_matmul_q4_amd as qmm
import synth

pytestmark = pytest.mark.gpu

# (entry, fmt, M, N, K): every launch route of every entry point
CASES = [
    ("gemv", "q4_0", 1, 8192, 2048), ("gemv", "q4_0", 1, 2048, 8192), ("gemv", "q4_0", 3, 1000, 2048),
    ("gemv", "q4_0", 6, 8192, 2048), ("gemv", "q4_0", 12, 8192, 2048), ("gemv", "q4_0", 12, 300, 320),
    ("gemv", "q8_0", 1, 32768, 2048), ("gemv", "q8_0", 2, 4096, 2048), ("gemv", "q8_0", 12, 1000, 1024),
    ("gemv", "q4_k", 1, 8192, 2048), ("gemv", "q4_k", 4, 1000, 1024), ("gemv", "q4_k", 8, 8192, 2048),
    ("gemv", "q4_k", 16, 8192, 2048),
    ("gemm", "q4_0", 2048, 8192, 512), ("gemm", "q4_0", 300, 2048, 512), ("gemm", "q4_0", 128, 8192, 512),
    ("gemm", "q4_0", 256, 8192, 512), ("gemm", "q4_0", 40, 2048, 1024), ("gemm", "q4_0", 3, 500, 512),
    ("gemm", "q8_0", 70, 4090, 512), ("gemm", "q4_k", 100, 8193, 512), ("gemm", "q4_k", 300, 700, 1280),
    ("gated", "q4_0", 1, 8192, 2048), ("gated", "q4_0", 4, 2048, 8192),
    # wide-matrix branches: 64 threads per row past 64 pairs, matrix-core
    # 3-4 rows, 5-8 rows in 4-wave workgroups with prefetch, 9-16 rows on the
    # 16x16 kernel up to N = 4096 and on 16-wave slices below N = 8192, the
    # Q4_K pair kernel, the gated kernel
    # looping over 32-pair chunks, few-tile and 220-tile GEMMs
    ("gemv", "q4_0", 1, 4100, 8192), ("gemv", "q8_0", 4, 4096, 4096),
    ("gemv", "q4_0", 8, 10000, 2048), ("gemv", "q4_0", 12, 4096, 4096), ("gemv", "q4_0", 12, 5000, 2048),
    ("gemv", "q4_k", 4, 8200, 4352), ("gated", "q4_0", 3, 4100, 5120),
    ("gemm", "q4_0", 512, 1000, 1024), ("gemm", "q8_0", 1000, 14000, 128),
    # the gated front half on the matrix cores (packed and apart)
    ("gated", "q4_0", 8, 8192, 2048), ("gated", "q4_0", 12, 1000, 1024), ("gated", "q4_0", 4, 8192, 4096),
    ("gated", "q4_0", 16, 8192, 2048),
]


def weights(fmt, n, k, seed):
    if fmt == "q4_k":
        return synth.q4_k_weights(n, k, seed)
    return synth.q4_0_weights(n, k, seed) if fmt == "q4_0" else synth.q8_0_weights(n, k, seed)


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def test_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    calls, outs = [], []
    for i, (entry, fmt, m, n, k) in enumerate(CASES):
        x = torch.from_numpy(synth.activations(m, k, seed=i)).to(dev)
        w = torch.from_numpy(np.ascontiguousarray(weights(fmt, n, k, i)).reshape(-1)).to(dev)
        y = torch.empty((m, n), device=dev)
        if entry == "gated":
            wu = torch.from_numpy(synth.q4_0_weights(n, k, seed=i + 1000).reshape(-1)).to(dev)
            calls.append(lambda x=x, w=w, wu=wu, y=y, n=n, k=k:
                         qmm.ffn_gate_up_q4_0(x, w, wu, n, k, out=y))
        else:
            fn = getattr(qmm, f"{entry}_{fmt}")
            calls.append(lambda fn=fn, x=x, w=w, y=y, n=n, k=k: fn(x, w, n, k, out=y))
        outs.append(y)
    print(f"[graph] {len(calls)} calls eagerly", flush=True)
    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [y.clone() for y in outs]
    for y in outs:
        y.fill_(float("nan"))
    torch.cuda.synchronize()

    print("[graph] capture", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for r in range(3):
        print(f"[graph] replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for (entry, fmt, m, n, k), y, e in zip(CASES, outs, eager):
            assert torch.equal(y, e), f"replay {r}: {entry}_{fmt} M={m} N={n} K={k} differs from eager"
        for y in outs:                              # the program's own eager work in between
            y.fill_(float("nan"))
        torch.cuda.synchronize()
    del g


def test_graph_replays_on_side_stream():
    """The same capture replayed while eager calls run on another stream."""
    dev = torch.device("cuda:0")
    n, k = 8192, 2048
    x = torch.from_numpy(synth.activations(4, k, seed=7)).to(dev)
    w = torch.from_numpy(synth.q4_0_weights(n, k, seed=7).reshape(-1)).to(dev)
    y_graph = torch.empty((4, n), device=dev)
    y_eager = torch.empty((4, n), device=dev)
    qmm.gemv_q4_0(x, w, n, k, out=y_eager)
    torch.cuda.synchronize()
    ref = y_eager.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qmm.gemv_q4_0(x, w, n, k, out=y_graph)
    side = torch.cuda.Stream()
    for r in range(3):
        print(f"[graph] side-stream replay {r}", flush=True)
        y_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        with torch.cuda.stream(side):
            qmm.gemv_q4_0(x, w, n, k, out=y_eager)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref) and torch.equal(y_eager, ref), r
    del g
