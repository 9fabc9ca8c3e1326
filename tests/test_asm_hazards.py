"""The kernels' hand-written vector-memory instructions against the gfx9 SGPR hazard.

The direct-to-LDS copies of the indexer, the attention kernels and the backward kernels
are inline assembly (`global_load_lds_dword[x4]` with a scalar row base).  On gfx9 a
vector-memory instruction may read an SGPR only 5 wait states after a VALU instruction
wrote it (v_readlane / v_readfirstlane, which is also how the compiler restores spilled
SGPRs).  The compiler pads for its own instructions but not for assembly, so each copy
carries its own `s_nop 4`; without it the copy can read a stale address and fault.

This test compiles every HIP source to gfx950 assembly and checks, for every
vector-memory instruction with an SGPR-pair address, that the instructions since the
last VALU write of that pair give at least 5 wait states (`s_nop N` counts N + 1, any
other instruction 1).  Runs on the CPU (hipcc cross-compiles); skipped without hipcc.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_sparse_attention_hca_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

VMEM_SGPR = re.compile(r"\s*(global_load\w*|global_store\w*|buffer_\w+)\s+.*?\bs\[(\d+):(\d+)\]")
NOP = re.compile(r"s_nop (\d+)")


def hazards(asm: str, need: int = 5):
    """(line, writer, reader) for every VMEM SGPR-address read closer than `need` wait
    states to a VALU write of that SGPR pair."""
    lines = asm.split("\n")
    found = []
    for i, line in enumerate(lines):
        m = VMEM_SGPR.match(line)
        if not m:
            continue
        regs = {f"s{m.group(2)}", f"s{m.group(3)}"}
        ws, j = 0, i - 1
        while j >= 0 and ws < need:
            t = lines[j].strip()
            j -= 1
            if not t or t.startswith((";", ".")) or t.endswith(":"):
                continue
            n = NOP.match(t)
            if n:
                ws += int(n.group(1)) + 1
                continue
            if t.startswith("v_") and len(t.split()) > 1:
                dst = t.split()[1].rstrip(",")
                r = re.match(r"s\[(\d+):(\d+)\]", dst)
                written = {f"s{k}" for k in range(int(r.group(1)), int(r.group(2)) + 1)} if r else {dst}
                if written & regs:
                    found.append((i + 1, t, line.strip()))
                    break
            ws += 1
    return found


def test_checker_flags_a_short_gap():
    asm = "\n".join(["v_readlane_b32 s5, v190, 14", "s_nop 0",
                     "global_load_lds_dwordx4 v128, s[4:5]"])
    assert len(hazards(asm)) == 1
    ok = "\n".join(["v_readlane_b32 s5, v190, 14", "s_nop 4",
                    "global_load_lds_dwordx4 v128, s[4:5]"])
    assert hazards(ok) == []
    other = "\n".join(["v_readlane_b32 s7, v190, 14", "global_load_lds_dwordx4 v128, s[4:5]"])
    assert hazards(other) == []


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as fh:
        return fh.read()


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_vmem_reads_sgpr_too_soon_after_valu_write(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        asms = dict(zip(SOURCES, ex.map(lambda s: _asm(s, str(tmp_path)), SOURCES)))
    bad = {src: hazards(a)[:3] for src, a in asms.items() if hazards(a)}
    assert not bad, bad
