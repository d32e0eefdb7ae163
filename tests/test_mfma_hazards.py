"""The decode kernels' MFMAs are inline asm, so the compiler's hazard checks do
not see them.  This test compiles the kernels for gfx950 to assembly and scans
every MFMA: no VGPR it reads may have been written by a VALU instruction
(including the AGPR-to-VGPR copies the register allocator places right before
an asm statement) fewer than four wait states earlier, counted within the same
straight-line block.  Runs on the CPU (hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_decode_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
NEED = 4  # wait states demanded between a VALU write and an MFMA read of the register


def vgprs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return {f"v{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {tok} if re.fullmatch(r"v\d+", tok) else set()


def scan(asm: str):
    found = []
    block = []  # instructions since the last label
    for line in asm.split("\n"):
        s = line.split(";")[0].strip()
        if not s or s.startswith("."):
            continue
        if s.endswith(":"):
            block = []
            continue
        if s.startswith("v_mfma"):
            ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
            srcs = set().union(*[vgprs(o) for o in ops[1:]])
            ws = 0
            for prev in reversed(block):
                if ws >= NEED:
                    break
                if prev.startswith("s_nop"):
                    ws += int(prev.split()[1], 0) + 1
                    continue
                if prev.startswith("v_") and not prev.startswith("v_mfma"):
                    parts = prev.split(None, 1)
                    dst = vgprs(parts[1].split(",")[0].strip()) if len(parts) > 1 else set()
                    if dst & srcs:
                        found.append((s, prev, ws))
                ws += 1
        block.append(s)
    return found


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_valu_write_reaches_an_mfma_operand_too_early(tmp_path):
    out = tmp_path / "kernels.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "mla_kernels.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    assert asm.count("v_mfma_f32_32x32x16_bf16") > 500, "the decode kernels' MFMAs were not found"
    found = scan(asm)
    assert not found, "\n".join(f"{m}  <-  {p}  ({w} wait states)" for m, p, w in found[:10])


def test_the_scan_flags_a_planted_hazard():
    asm = "\n".join(["k:", "v_accvgpr_read_b32 v21, a151", "s_nop 0",
                     "v_mfma_f32_32x32x16_bf16 v[2:17], v[22:25], v[18:21], v[2:17]",
                     "v_mov_b32 v30, v1", "s_nop 3", "v_mfma_f32_32x32x16_bf16 v[2:17], v[22:25], v[30:33], v[2:17]"])
    found = scan(asm)
    assert len(found) == 1 and "v21" in found[0][1] and found[0][2] == 1
