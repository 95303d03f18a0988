#!/usr/bin/env python3
"""One kernel dispatch per entry-point call, checked with the profiler's
kernel trace (run on a GPU; not a pytest module).

    rocprofv3 --kernel-trace --output-format csv -d <dir> -o calls -- \\
        python3 tests/dispatch_calls.py --log <dir>/calls.json
    python3 tests/dispatch_calls.py --check <dir>/calls_kernel_trace.csv --log <dir>/calls.json

The first command allocates every input up front, then calls each case
below exactly once (a device synchronization after each), and writes the
ordered list of calls. The second reads the trace, keeps the library's own
kernels (every other kernel comes from the setup's allocations and copies),
orders them by start time and checks that there is exactly one per call and
that it is one of the kernels the entry point may route to; it prints a
markdown table and exits non-zero on any mismatch.
"""

from __future__ import annotations

import argparse
import csv
import json
import pathlib
import sys

ROOT = pathlib.Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))

# the library's kernels, by the names the trace gives them
LIB_KERNELS = ("gemv_m1_kernel", "gemv_small_m_kernel", "gemv_slice_kernel", "gemv_q4_k_kernel",
               "gemv_q4_k_pair_kernel", "gemm_kernel", "gemm_mid_kernel")
GEMV = ("gemv_m1_kernel", "gemv_small_m_kernel", "gemv_slice_kernel")
ROUTES = {
    "gemv_q4_0": GEMV, "gemv_q8_0": GEMV,
    "gemm_q4_0": ("gemv_m1_kernel", "gemv_small_m_kernel", "gemv_slice_kernel", "gemm_kernel",
                  "gemm_mid_kernel"),
    "gemm_q8_0": ("gemv_m1_kernel", "gemv_small_m_kernel", "gemv_slice_kernel", "gemm_kernel",
                  "gemm_mid_kernel"),
    "gemv_q4_k": ("gemv_q4_k_kernel", "gemv_q4_k_pair_kernel", "gemv_small_m_kernel",
                  "gemv_slice_kernel"),
    "gemm_q4_k": ("gemv_q4_k_kernel", "gemv_q4_k_pair_kernel", "gemv_small_m_kernel", "gemm_kernel",
                  "gemm_mid_kernel"),
    "ffn_gate_up_q4_0": ("gemv_m1_kernel", "gemv_small_m_kernel", "gemv_slice_kernel"),
}
# (entry point, M, N, K): every launch branch of every entry point
CASES = [
    ("gemv_q4_0", 1, 256, 512), ("gemv_q4_0", 1, 8192, 2048), ("gemv_q4_0", 1, 2048, 8192),
    ("gemv_q4_0", 1, 4096, 4096), ("gemv_q4_0", 1, 65536, 2048), ("gemv_q4_0", 2, 1000, 2048),
    ("gemv_q4_0", 3, 300, 8192), ("gemv_q4_0", 4, 8192, 2048), ("gemv_q4_0", 6, 8192, 2048),
    ("gemv_q4_0", 8, 300, 1024), ("gemv_q4_0", 12, 300, 1024), ("gemv_q4_0", 16, 8192, 2048),
    ("gemv_q4_0", 5, 300, 320), ("gemv_q4_0", 1, 4096, 8192), ("gemv_q4_0", 2, 8192, 8192),
    ("gemv_q4_0", 2, 4096, 8192), ("gemv_q4_0", 4, 4096, 8192), ("gemv_q8_0", 1, 2048, 8192),
    ("gemv_q4_0", 8, 16384, 2048), ("gemv_q8_0", 8, 16384, 2048), ("gemv_q4_0", 7, 65536, 2048),
    ("gemv_q4_0", 3, 4096, 4096), ("gemv_q8_0", 4, 14336, 4096), ("gemm_q4_0", 4, 4096, 4096),
    ("gemv_q4_0", 4, 2560, 6912), ("gemv_q8_0", 3, 3072, 3072), ("gemv_q4_0", 4, 1536, 8960),
    ("gemv_q4_0", 4, 32768, 2048), ("gemv_q4_0", 12, 5000, 2048), ("gemv_q4_k", 12, 5000, 8192),
    ("gemv_q4_0", 6, 6144, 4096), ("gemv_q8_0", 6, 6144, 4096), ("gemv_q4_0", 16, 6144, 4096),
    ("gemm_q4_0", 12, 2048, 8192), ("gemm_q8_0", 16, 4096, 320),
    ("gemv_q8_0", 1, 262144, 2048), ("gemv_q8_0", 2, 1000, 2048), ("gemv_q8_0", 4, 300, 8192),
    ("gemv_q8_0", 6, 300, 1024), ("gemv_q8_0", 12, 8192, 1024), ("gemv_q8_0", 12, 300, 1024),
    ("gemm_q4_0", 3, 300, 1024), ("gemm_q4_0", 16, 8192, 2048), ("gemm_q4_0", 100, 2048, 8192),
    ("gemm_q4_0", 300, 300, 512), ("gemm_q4_0", 2048, 8192, 2048),
    ("gemm_q8_0", 2, 300, 1024), ("gemm_q8_0", 64, 4100, 1024), ("gemm_q8_0", 2048, 8192, 512),
    ("gemm_q4_0", 20, 5000, 512), ("gemm_q4_0", 70, 4090, 512), ("gemm_q4_0", 80, 8150, 512),
    ("gemm_q4_0", 100, 8193, 512), ("gemm_q4_0", 200, 8150, 512),
    ("gemm_q4_0", 512, 1024, 4096), ("gemm_q4_0", 2100, 1030, 512), ("gemm_q4_0", 1024, 14336, 512),
    ("gemv_q4_k", 1, 8192, 2048), ("gemv_q4_k", 2, 300, 8192), ("gemv_q4_k", 4, 300, 1024),
    ("gemv_q4_k", 5, 300, 1024), ("gemv_q4_k", 8, 65536, 512), ("gemv_q4_k", 16, 8192, 2048),
    ("gemv_q4_k", 12, 4096, 1024), ("gemv_q4_k", 4, 8192, 2048), ("gemv_q4_k", 4, 8192, 8192),
    ("gemv_q4_k", 1, 4096, 8192), ("gemv_q4_k", 4, 16384, 2048), ("gemv_q4_k", 2, 4096, 4096),
    ("gemv_q4_k", 4, 4096, 8192), ("gemv_q4_k", 3, 3072, 8192), ("gemv_q4_k", 4, 11008, 2048),
    ("gemm_q4_k", 3, 300, 1024), ("gemm_q4_k", 40, 300, 1024), ("gemm_q4_k", 2048, 8192, 2048),
    ("gemm_q4_k", 8, 2048, 8192), ("gemm_q4_k", 12, 5000, 1024),
    ("ffn_gate_up_q4_0", 1, 8192, 2048), ("ffn_gate_up_q4_0", 1, 2048, 8192),
    ("ffn_gate_up_q4_0", 2, 8192, 2048), ("ffn_gate_up_q4_0", 4, 2048, 8192),
    ("ffn_gate_up_q4_0", 1, 4096, 8192), ("ffn_gate_up_q4_0", 8, 8192, 2048),
    ("ffn_gate_up_q4_0", 16, 2048, 8192), ("ffn_gate_up_q4_0", 4, 8192, 4096),
    ("ffn_gate_up_q4_0", 12, 8192, 2048), ("ffn_gate_up_q4_0", 6, 300, 320),
]


def short(name: str) -> str:
    for prefix in ("void ", "qmm::", "(anonymous namespace)::"):
        name = name.replace(prefix, "")
    return name.split("<")[0].split("(")[0].strip()


def run_calls(log_path: pathlib.Path) -> None:
    import numpy as np
    import torch

    import block_quantized_matmul_q4_amd as qmm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rng = np.random.default_rng(0)
    bufs = []
    for entry, m, n, k in CASES:
        fmt = "q4_0" if entry == "ffn_gate_up_q4_0" else entry.split("_", 1)[1]
        row = {"q4_0": k // 32 * 18, "q8_0": k // 32 * 34, "q4_k": k // 256 * 144}[fmt]
        # small random bytes with finite scales (d = 1.0 in fp16) are enough:
        # only the dispatch count matters here
        w = rng.integers(0, 256, size=(n, row), dtype=np.uint8)
        bs = {"q4_0": 18, "q8_0": 34, "q4_k": 144}[fmt]
        blocks = w.reshape(n, -1, bs)
        blocks[:, :, 0], blocks[:, :, 1] = 0x00, 0x3C          # d = 1.0
        if fmt == "q4_k":
            blocks[:, :, 2], blocks[:, :, 3] = 0x00, 0x3C      # dmin = 1.0
        wt = torch.from_numpy(w.reshape(-1)).to(dev)
        wu = torch.from_numpy(w.reshape(-1).copy()).to(dev) if entry == "ffn_gate_up_q4_0" else None
        x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(dev)
        y = torch.empty((m, n), device=dev)
        bufs.append((x, wt, wu, y))
    torch.cuda.synchronize()
    lib = qmm.library()
    log = []
    for (entry, m, n, k), (x, wt, wu, y) in zip(CASES, bufs):
        if entry == "ffn_gate_up_q4_0":
            st = lib.qmm_ffn_gate_up_q4_0(x.data_ptr(), wt.data_ptr(), wu.data_ptr(), y.data_ptr(),
                                          m, n, k, 0)
        else:
            st = getattr(lib, f"qmm_{entry}")(x.data_ptr(), wt.data_ptr(), y.data_ptr(), m, n, k, 0)
        torch.cuda.synchronize()
        if st != 0:
            raise SystemExit(f"{entry} M={m} N={n} K={k}: status {st}: {qmm.qmm_last_error()}")
        log.append({"entry": entry, "M": m, "N": n, "K": k})
        print(f"called {entry} M={m} N={n} K={k}", flush=True)
    log_path.write_text(json.dumps(log, indent=1))


def check(trace: pathlib.Path, log_path: pathlib.Path) -> int:
    calls = json.loads(log_path.read_text())
    rows = [r for r in csv.DictReader(open(trace)) if short(r["Kernel_Name"]) in LIB_KERNELS]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    print("| call | entry point | M | N | K | kernel | grid | ok |")
    print("|---|---|---|---|---|---|---|---|")
    bad = 0
    for i, c in enumerate(calls):
        r = rows[i] if i < len(rows) else None
        name = short(r["Kernel_Name"]) if r else "(none)"
        grid = (f"{r['Grid_Size_X']}x{r['Grid_Size_Y']}" if r else "-")
        ok = r is not None and name in ROUTES[c["entry"]]
        bad += not ok
        print(f"| {i} | `qmm_{c['entry']}` | {c['M']} | {c['N']} | {c['K']} | `{name}` | {grid} | "
              f"{'yes' if ok else 'NO'} |")
    print(f"\n{len(calls)} calls, {len(rows)} library kernel dispatches "
          f"({'one per call' if len(rows) == len(calls) else 'MISMATCH'})")
    return 0 if bad == 0 and len(rows) == len(calls) else 1


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--log", type=pathlib.Path, required=True)
    ap.add_argument("--check", type=pathlib.Path)
    a = ap.parse_args()
    if a.check:
        return check(a.check, a.log)
    run_calls(a.log)
    return 0


if __name__ == "__main__":
    sys.exit(main())
