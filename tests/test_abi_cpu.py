"""C-ABI library on the host (no GPU): it loads, exports every symbol that
include/qmm.h declares, and rejects bad arguments before any HIP call.

Only validation paths are exercised here: each call below fails a host-side
check, so no kernel is launched and the fake addresses are never touched.
"""

import re
import pathlib
import subprocess

import pytest

import block_quantized_matmul_q4_amd as qmm

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "qmm.h"

A = 0x10000          # fake, 256-byte aligned "device" addresses: never read
B = 0x20000000
C = 0x40000000


def declared_functions():
    return re.findall(r"QMM_API\s+[\w\s\*]+?\b(qmm_\w+)\s*\(", HEADER.read_text())


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == set(qmm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = qmm.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(qmm.LIBRARY)],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported
    # nothing else with the public prefix leaks out
    assert {s for s in exported if s.startswith("qmm_")} == set(declared_functions())


def test_status_strings_and_version():
    assert qmm.qmm_status_string(qmm.QMM_OK) == "QMM_OK"
    assert qmm.qmm_status_string(qmm.QMM_EUNSUPPORTED) == "QMM_EUNSUPPORTED"
    assert qmm.qmm_status_string(99) == "QMM_UNKNOWN_STATUS"
    assert qmm.qmm_version() >= 100


ENTRY = {
    "qmm_gemv_q4_0": qmm.qmm_gemv_q4_0,
    "qmm_gemv_q8_0": qmm.qmm_gemv_q8_0,
    "qmm_gemm_q4_0": qmm.qmm_gemm_q4_0,
    "qmm_gemm_q8_0": qmm.qmm_gemm_q8_0,
}


@pytest.mark.parametrize("name", list(ENTRY))
@pytest.mark.parametrize("args,status,fragment", [
    ((0, B, C, 1, 8, 256), qmm.QMM_EINVAL, "null pointer"),
    ((A, 0, C, 1, 8, 256), qmm.QMM_EINVAL, "null pointer"),
    ((A, B, 0, 1, 8, 256), qmm.QMM_EINVAL, "null pointer"),
    ((A, B, C, 0, 8, 256), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, 1, 0, 256), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, 1, 8, 0), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, -3, 8, 256), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, 1, 8, 48), qmm.QMM_EINVAL, "multiple of 32"),
    ((A, B, C, 1, 8, 96), qmm.QMM_EUNSUPPORTED, "unsupported"),
    ((A, B, C, 1, 8, 65536 + 256), qmm.QMM_EUNSUPPORTED, "unsupported"),
    ((A + 4, B, C, 1, 8, 256), qmm.QMM_EALIGN, "misaligned"),
    ((A, B + 2, C, 1, 8, 256), qmm.QMM_EALIGN, "misaligned"),
    ((A, B, C + 2, 1, 8, 256), qmm.QMM_EALIGN, "misaligned"),
    ((A, B, A + 512, 1, 8, 256), qmm.QMM_EINVAL, "overlaps"),   # y inside x
    ((A, B, B + 64, 1, 8, 256), qmm.QMM_EINVAL, "overlaps"),    # y inside w
    ((A, B, C, 1, 2**40, 256), qmm.QMM_EINVAL, "overflow"),
])
def test_rejected_before_launch(name, args, status, fragment):
    got = ENTRY[name](*args, 0)
    assert got == status, (name, args, qmm.qmm_last_error())
    assert fragment in qmm.qmm_last_error()
    assert name in qmm.qmm_last_error()


@pytest.mark.parametrize("name", ["qmm_gemv_q4_0", "qmm_gemv_q8_0"])
def test_gemv_rejects_more_than_16_rows(name):
    assert ENTRY[name](A, B, C, 17, 8, 256, 0) == qmm.QMM_EINVAL
    assert "exceeds 16" in qmm.qmm_last_error()


def header_constant(name):
    m = re.search(rf"#define\s+{name}\s+(\d+)", HEADER.read_text())
    return int(m.group(1))


@pytest.mark.parametrize("name,block", [("qmm_gemm_q4_0", 18), ("qmm_gemm_q8_0", 34)])
def test_gemm_rejects_n_past_its_bound(name, block):
    # a 256-row band of y must stay below 2 GiB for the kernel's offsets
    n_max = header_constant("QMM_GEMM_MAX_N")
    assert 256 * n_max * 4 < 2**31 <= 256 * (n_max + 1) * 4
    w_len = (n_max + 1) * (256 // 32) * block
    y = 0x80000000                          # fake y past the fake w
    assert B + w_len < y
    got = ENTRY[name](A, B, y, 1, n_max + 1, 256, 0)
    assert got == qmm.QMM_EUNSUPPORTED, qmm.qmm_last_error()
    assert "unsupported" in qmm.qmm_last_error() and name in qmm.qmm_last_error()




def test_tensor_front_end_checks_types():
    import torch

    x = torch.zeros(1, 256)
    w = torch.zeros(8 * 8 * 18, dtype=torch.uint8)
    with pytest.raises(ValueError):
        qmm.gemv_q4_0(x, w, 8, 256)          # CPU tensors are refused
    with pytest.raises(TypeError):
        qmm.gemv_q4_0(x.numpy(), w, 8, 256)


@pytest.mark.parametrize("args,status,fragment", [
    ((A, B, 0, C, 1, 8, 256), qmm.QMM_EINVAL, "null pointer (w_up)"),
    ((A, B, B + 8 * 8 * 18 + 2, C, 1, 8, 256), qmm.QMM_EALIGN, "w_up"),
    ((A, B, C, C + 16, 1, 8, 256), qmm.QMM_EINVAL, "overlaps w_up"),
    ((A, B, B + 4096, C, 17, 8, 256), qmm.QMM_EINVAL, "exceeds 16"),
    ((0, B, B + 4096, C, 1, 8, 256), qmm.QMM_EINVAL, "null pointer"),
    ((A, B, B + 4096, C, 1, 8, 96), qmm.QMM_EUNSUPPORTED, "unsupported"),
    ((A, B + 2, B + 4096, C, 1, 8, 256), qmm.QMM_EALIGN, "misaligned"),
])
def test_ffn_gate_up_rejected_before_launch(args, status, fragment):
    got = qmm.qmm_ffn_gate_up_q4_0(*args, 0)
    assert got == status, (args, qmm.qmm_last_error())
    assert fragment in qmm.qmm_last_error()
    assert "qmm_ffn_gate_up_q4_0" in qmm.qmm_last_error()


def test_bench_read_kernels_load_and_reject_bad_arguments():
    """bench.py's reference read kernels: built by build(), loadable on the
    host, and their argument checks fail before any launch."""
    import sys

    sys.path.insert(0, str(ROOT))
    import bench

    lib = bench.bench_read_library()
    assert lib.bench_read_plain(None, 16, A, None) == 1
    assert lib.bench_read_plain(A, 24, A, None) == 1          # not a multiple of 16
    assert lib.bench_read_plain(A + 4, 16, A, None) == 1      # not 16-byte aligned
    assert lib.bench_read_pairs(A, 40, A, None) == 1          # not a multiple of 36
    assert lib.bench_read_pairs(A, 36, None, None) == 1


@pytest.mark.parametrize("args,status,fragment", [
    ((0, B, C, 1, 8, 256), qmm.QMM_EINVAL, "null pointer"),
    ((A, B, C, 0, 8, 256), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, 1, 8, 0), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, 1, 8, 384), qmm.QMM_EINVAL, "multiple of 256"),
    ((A, B, C, 1, 8, 64), qmm.QMM_EINVAL, "multiple of 256"),
    ((A, B, C, 17, 8, 256), qmm.QMM_EINVAL, "exceeds 16"),
    ((A, B, C, 1, 8, 65536 + 256), qmm.QMM_EUNSUPPORTED, "unsupported"),
    ((A + 4, B, C, 1, 8, 256), qmm.QMM_EALIGN, "misaligned"),
    ((A, B + 4, C, 1, 8, 256), qmm.QMM_EALIGN, "misaligned"),
    ((A, B, B + 64, 1, 8, 256), qmm.QMM_EINVAL, "overlaps"),
])
def test_gemv_q4_k_rejected_before_launch(args, status, fragment):
    got = qmm.qmm_gemv_q4_k(*args, 0)
    assert got == status, (args, qmm.qmm_last_error())
    assert fragment in qmm.qmm_last_error()
    assert "qmm_gemv_q4_k" in qmm.qmm_last_error()


@pytest.mark.parametrize("args,status,fragment", [
    ((0, B, C, 4, 8, 256), qmm.QMM_EINVAL, "null pointer"),
    ((A, B, C, 0, 8, 256), qmm.QMM_EINVAL, ">= 1"),
    ((A, B, C, 4, 8, 384), qmm.QMM_EINVAL, "multiple of 256"),
    ((A, B, C, 4, 8, 65536 + 256), qmm.QMM_EUNSUPPORTED, "unsupported"),
    ((A, B + 4, C, 4, 8, 256), qmm.QMM_EALIGN, "misaligned"),
    ((A, B, B + 64, 4, 8, 256), qmm.QMM_EINVAL, "overlaps"),
])
def test_gemm_q4_k_rejected_before_launch(args, status, fragment):
    got = qmm.qmm_gemm_q4_k(*args, 0)
    assert got == status, (args, qmm.qmm_last_error())
    assert fragment in qmm.qmm_last_error()
    assert "qmm_gemm_q4_k" in qmm.qmm_last_error()
