"""Checks on the generated gfx950 code that the kernels' correctness relies on (CPU only).

The screening kernel and the yardstick's correlation sweep write M0 in inline assembly to drive its global -> LDS copies; that is
only sound while the compiler itself keeps nothing in M0 in these kernels.  The test compiles
the source to assembly and requires every M0 access to be one of those copies.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_dictionary_coding_amd import build

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("name", ["score_topn.hip", "omp.hip"])
def test_m0_written_only_by_lds_copies(tmp_path, name):
    src = os.path.join(build.CSRC, name)
    out = tmp_path / (name + ".s")
    cmd = [HIPCC, *build.HIPCC_FLAGS, f"-I{build.INCLUDE}", f"-I{build.CSRC}",
           "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = [ln.strip() for ln in out.read_text().splitlines()]
    copies = 0
    for i, ln in enumerate(lines):
        if ln.startswith(";") or not re.search(r"\bm0\b", ln):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"unexpected M0 use: {ln}"
        assert lines[i + 1] == "s_nop 0", lines[i + 1]
        assert lines[i + 2].startswith("global_load_lds_dwordx4 "), lines[i + 2]
        copies += 1
    assert copies > 0


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_softmax_dynamic_lds_is_8_byte_aligned(tmp_path):
    """The attention softmax keeps 64-bit fixed-point weights in dynamic LDS, which starts right
    after the kernel's static LDS: that static size must keep the dynamic base 8-byte aligned
    (misaligned 64-bit LDS accesses fault)."""
    src = os.path.join(build.CSRC, "attend.hip")
    out = tmp_path / "attend.s"
    cmd = [HIPCC, *build.HIPCC_FLAGS, f"-I{build.INCLUDE}", f"-I{build.CSRC}",
           "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    sizes = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n((?:.*\n)*?)\s+\.end_amdhsa_kernel", text):
        if "attend_softmax_kernel" in m.group(1):
            g = re.search(r"amdhsa_group_segment_fixed_size (\d+)", m.group(2))
            sizes[m.group(1)] = int(g.group(1))
    assert sizes, "softmax kernels not found"
    for name, size in sizes.items():
        assert size % 8 == 0, (name, size)
