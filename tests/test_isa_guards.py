"""Checks on the GEMM's gfx950 assembly (compiled here from source, no GPU).

The direct-to-LDS copies write M0 from inline asm without restoring it, which
is only sound while nothing else in those kernels reads or writes M0: the
compiler cannot be told about the write.  This test compiles gemm.hip to
device assembly and fails on any M0 access outside the copies' asm blocks."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a8_int8_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "gemm.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "gemm.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def _kernels(asm):
    names = re.findall(r"^(_Z\S*gemm_kernel\S*):", asm, flags=re.M)
    for n in names:
        i = asm.index(n + ":")
        yield n, asm[i:asm.index(".Lfunc_end", i)]


def test_m0_only_in_copy_asm(gemm_asm):
    kernels = list(_kernels(gemm_asm))
    assert len(kernels) >= 30
    for name, body in kernels:
        in_asm = False
        for line in body.splitlines():
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
            elif t.startswith(";;#ASMEND"):
                in_asm = False
            elif not in_asm and not t.startswith(";") and re.search(r"\bm0\b", t):
                pytest.fail(f"{name}: M0 used outside the copy asm: {t}")


def test_copy_blocks_write_m0_before_the_load(gemm_asm):
    for name, body in _kernels(gemm_asm):
        for blk in re.findall(r";;#ASMSTART(.*?);;#ASMEND", body, flags=re.S):
            if "lds" in blk and ("buffer_load" in blk or "global_load_lds" in blk):
                ops = [l.split()[0] for l in blk.strip().splitlines() if l.strip()]
                assert ops[:2] == ["s_mov_b32", "s_nop"], (name, ops)
