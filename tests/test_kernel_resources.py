"""Every HIP kernel of the library keeps its working set in registers: no
vector-register spills and no private (scratch) memory, read from the code
object metadata of a device-only compile with the library's own flags.  A
spill or a stack object in a GEMM kernel costs tens of percent (an
accumulator array placed in scratch memory made the split-fp16 Newton kernel
25% slower), and nothing else in the CPU suite would notice.  Scalar-register
spills go to vector-register lanes, not memory, and are allowed."""

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from matrix_roots_amd import build as mb

HIP_SOURCES = [s for s in mb.SOURCES if s.endswith(".hip")]


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [mb.hipcc(), *mb.COMMON, "-x", "hip", "--cuda-device-only", "-S", os.path.join(mb.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _kernels(asm: str):
    """(name, metadata fields) of every kernel in the AMDGPU metadata block."""
    for m in re.finditer(r"\.name:\s+(\S+)\n(.*?)(?=\n  - \.|\n\.end_amdgpu_metadata|\Z)", asm, re.S):
        fields = {k: int(v) for k, v in re.findall(r"\.(\w+):\s+(\d+)\s*$", m.group(2), re.M)}
        if "vgpr_count" in fields:
            yield m.group(1), fields


@pytest.fixture(scope="module")
def device_asm():
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(min(8, len(HIP_SOURCES))) as ex:
        return dict(zip(HIP_SOURCES, ex.map(lambda s: _device_asm(s, tmp), HIP_SOURCES)))


def test_no_spills_or_scratch(device_asm):
    seen = 0
    bad = []
    for src, asm in device_asm.items():
        for name, f in _kernels(asm):
            seen += 1
            if f.get("vgpr_spill_count", 0) or f.get("private_segment_fixed_size", 0):
                bad.append((src, name, f.get("vgpr_count"), f.get("vgpr_spill_count"),
                            f.get("private_segment_fixed_size")))
    assert seen >= 30, seen  # every kernel source parsed
    assert not bad, bad


def test_direct_to_lds_copies_take_scalar_bases(device_asm):
    """Every direct-to-LDS copy is one instruction on a scalar base with a
    32-bit lane offset (`global_load_lds_dwordx4 vOFF, s[BASE:BASE+1]`), not
    a per-lane 64-bit address (`..., off`): the 64-bit form costs three
    64-bit adds per copy and registers held across the GEMM main loops."""
    copies = 0
    bad = []
    for src, asm in device_asm.items():
        for line in asm.splitlines():
            s = line.strip()
            if s.startswith("global_load_lds"):
                copies += 1
                if not re.match(r"global_load_lds_dword\w*\s+v\d+,\s+s\[\d+:\d+\]", s):
                    bad.append((src, s))
    assert copies >= 100, copies  # the GEMM cores of every source were parsed
    assert not bad, bad[:5]
