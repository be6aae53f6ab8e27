"""The expert GEMM's global->LDS copies set M0 in inline asm (M0 carries the
LDS address of a wave's copy).  The compiler treats M0 as reserved and does
not preserve it across asm statements, so this build is correct only while
nothing else in the kernel uses M0.  This test compiles the kernel to gfx950
assembly (CPU only, no GPU needed) and checks that every M0 reference is one
of those writes, each directly followed by its copy instruction.
"""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "combine_expert_amd", "csrc", "expert_gemm.hip")


def test_m0_only_feeds_the_lds_copies(tmp_path):
    from combine_expert_amd import build as hip_build
    out = tmp_path / "expert_gemm.s"
    cmd = [hip_build.HIPCC, *hip_build.FLAGS, "--cuda-device-only", "-S", "-o", str(out),
           "-I", hip_build.INCLUDE, "-I", hip_build.CSRC, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln.split(";")[0].strip() for ln in out.read_text().splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
    m0 = [i for i, ln in enumerate(lines) if re.search(r"\bm0\b", ln)]
    assert m0, "no M0 writes found: the copies are no longer issued as expected"
    for i in m0:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", lines[i]), lines[i]
        assert lines[i + 1].startswith("global_load_lds_dword"), (lines[i], lines[i + 1])
    copies = sum(ln.startswith("global_load_lds_dword") for ln in lines)
    assert copies == len(m0)
