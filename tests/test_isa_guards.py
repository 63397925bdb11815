"""Checks on the GEMM's gfx950 assembly (compiled here from source, no GPU).

The direct-to-LDS copies write M0 from inline asm without restoring it, which
is only sound while nothing else in those kernels reads or writes M0: the
compiler cannot be told about the write.  Copies that share one M0 value rely
on no branch or label between the write and the load.  This test compiles
gemm.hip and gemm_pc.hip to device assembly and fails on any M0 access
outside the copies' asm blocks and on any copy not preceded by an M0 write in
its basic block."""
import os
import sys
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a8_int8_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
sys.path.insert(0, ROOT)
from w4a8_int8_gemm_amd.build import FLAGS  # noqa: E402  (plain list; imports nothing else)


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    # the library's own device flags, so the checked code is the shipped code
    flags = [f for f in FLAGS if f != "-fPIC"]
    text = []
    for src in ("gemm.hip", "gemm_pc.hip"):
        out = str(d / (src + ".s"))
        cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        text.append(open(out).read())
    return "\n".join(text)


def _kernels(asm):
    names = re.findall(r"^(_Z\S*gemm\w*_kernel\S*):", asm, flags=re.M)
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


def test_every_lds_copy_follows_an_m0_write_in_its_block(gemm_asm):
    """A direct-to-LDS load reads M0, which only the copies' own asm sets:
    within each basic block, some asm M0 write must precede every such
    load (at a block boundary M0 counts as unknown)."""
    n_loads = 0
    for name, body in _kernels(gemm_asm):
        m0_known = False
        in_asm = False
        for line in body.splitlines():
            t = line.strip()
            if re.match(r"^\.LBB\w*:", t) or t.startswith("s_cbranch") or t.startswith("s_branch"):
                m0_known = False
            elif t.startswith(";;#ASMSTART"):
                in_asm = True
            elif t.startswith(";;#ASMEND"):
                in_asm = False
            elif in_asm and t.startswith("s_mov_b32 m0"):
                m0_known = True
            elif re.search(r"\b(buffer_load_dword\w*|global_load_lds_dword)\b.*\blds\b", t) or \
                    t.startswith("global_load_lds_dword"):
                assert in_asm, (name, t)
                assert m0_known, f"{name}: LDS copy without a preceding M0 write in its block: {t}"
                n_loads += 1
    assert n_loads > 100
