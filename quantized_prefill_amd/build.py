"""Build libqprefill.so (HIP for gfx950) in-tree with hipcc.

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqprefill.so")
ARCH = os.environ.get("QP_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB) -> str:
    objs = []
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    include = os.path.join(os.path.dirname(HERE), "include")
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", include,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + list(extra or [])
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip", f"--offload-arch={ARCH}"] if src.endswith(".hip") else []
        cmd = [hipcc()] + lang + common + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), src))
        objs.append(obj)
    failed = []
    for p, src in procs:
        out_txt = p.communicate()[0].decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; drop that line
        lines = [l for l in out_txt.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = out + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
