"""The C-ABI layer (csrc/qmm_api.hip) built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer, linked with stand-ins for
the kernel launchers (tests/sanitize/launch_stubs.cpp), and driven through
every entry point by tests/sanitize/abi_driver.cpp: valid and invalid
arguments, extreme sizes, the route of each valid call, the launch-error
path and the per-thread error string. CPU only: no kernel is compiled or
launched."""

import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SAN = ROOT / "tests" / "sanitize"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# every sanitizer option applies to the host pass only
SAN_FLAGS = []
for opt in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"):
    SAN_FLAGS += ["-Xarch_host", opt]


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_abi_layer_under_sanitizers(tmp_path):
    sources = {
        "api.o": ROOT / "block_quantized_matmul_q4_amd" / "csrc" / "qmm_api.hip",
        "stubs.o": SAN / "launch_stubs.cpp",
        "driver.o": SAN / "abi_driver.cpp",
    }
    for obj, src in sources.items():
        cmd = [HIPCC, "-std=c++17", "-O1", "-g", *SAN_FLAGS, "-x", "hip", "--cuda-host-only",
               f"-I{ROOT / 'include'}", "-c", str(src), "-o", str(tmp_path / obj)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, f"compile {src.name}:\n{res.stderr[-3000:]}"
    exe = tmp_path / "abi_driver"
    res = subprocess.run([HIPCC, *SAN_FLAGS, "-o", str(exe), *(str(tmp_path / o) for o in sources)],
                         capture_output=True, text=True)
    assert res.returncode == 0, f"link:\n{res.stderr[-3000:]}"
    # the sanitizers are really in the build
    syms = subprocess.run(["nm", str(tmp_path / "api.o")], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, f"driver failed:\n{run.stdout}\n{run.stderr[-4000:]}"
    assert "abi checks passed" in run.stdout
