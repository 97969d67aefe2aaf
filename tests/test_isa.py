"""Every HIP source compiles for gfx950, and no kernel indexes its registers
at run time or spills to private scratch.

Run-time indexed register access (s_set_gpr_idx / v_movrel) is banned
outright: a private array indexed by a loop counter was once lowered to an
indexed register write hoisted above its bounds guard, which overwrote a store
address and faulted the GPU.  Kernels keep every register array at
compile-time indices instead.  Packed f32 arithmetic is kept out of the
device code too (the build disables the packed-fp32-ops target feature).
Global memory is read and written with global (or buffer) instructions, never
flat ones: a flat load also counts against the LDS wait counter, so every LDS
wait after it waits for HBM as well."""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_prefill_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")

SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))


@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_device_code_has_no_indexed_registers_or_scratch(src, tmp_path):
    asm = tmp_path / "out.s"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", str(asm)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = asm.read_text()
    kernel = None
    bad = []
    packed = []
    flat = []
    for line in text.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kernel = m.group(1)
        if re.search(r"\bs_set_gpr_idx_on\b|\bv_movrel", line):
            bad.append((kernel, line.strip()))
        if re.search(r"\bv_pk_(fma|mul|add)_f32\b", line):
            packed.append((kernel, line.strip()))
        if re.search(r"\bflat_(load|store|atomic)", line):
            flat.append((kernel, line.strip()))
    assert not bad, f"run-time indexed register access: {bad[:4]}"
    assert not packed, f"packed f32 arithmetic in device code: {packed[:4]}"
    assert not flat, f"flat memory instructions in device code: {flat[:4]}"
    scratch = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)
    assert scratch and all(int(s) == 0 for s in scratch), f"private scratch in use: {scratch}"
