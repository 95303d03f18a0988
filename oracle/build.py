"""Compile the CPU oracle (plain C, gcc, OpenMP) into ``libqmm_oracle.so``.

Test infrastructure only. Strict IEEE arithmetic: no -ffast-math, no FMA
contraction, so every product and sum rounds exactly as written.
"""

from __future__ import annotations

import pathlib
import subprocess
import sys

HERE = pathlib.Path(__file__).resolve().parent


def build(source: pathlib.Path | str = HERE / "qmm_oracle.c",
          output: pathlib.Path | str = HERE / "libqmm_oracle.so",
          werror: bool = True) -> pathlib.Path:
    output = pathlib.Path(output)
    tmp = output.with_name(output.name + ".tmp")
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]
    cmd += ["-Werror"] if werror else ["-w"]
    cmd += ["-o", str(tmp), str(source), "-lm"]
    subprocess.run(cmd, check=True)
    tmp.replace(output)
    return output


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
