"""Build liboracle.so with gcc (test infrastructure; see oracle/__init__.py).

-O2 -ffp-contract=off and no fast-math: every binary32 operation of the
dequant definition rounds once, in program order.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")


def library_path(plant: int = 0, outdir: str | None = None) -> str:
    if plant == 0 and outdir is None:
        return os.path.join(HERE, "liboracle.so")
    outdir = outdir or os.path.join(HERE, f"_plant_{plant}")
    return os.path.join(outdir, f"liboracle_plant{plant}.so")


def build(plant: int = 0, outdir: str | None = None, cc: str = "gcc") -> str:
    out = library_path(plant, outdir)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", f"-DQP_PLANT={int(plant)}", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))
