"""The decode kernels' MFMAs are inline asm, so the compiler's hazard checks do
not see them.  This test compiles the kernels for gfx950 to assembly and scans
every MFMA along the control-flow graph (fall-through and branch edges, so
loop back-edges are followed), in both directions:

  * backward: no VGPR or AGPR the MFMA reads may have been written by a
    non-MFMA vector instruction (including the register allocator's
    v_accvgpr_read/write copies placed right before an asm statement) fewer
    than NEED_IN wait states earlier;
  * forward: no non-MFMA instruction may read or overwrite the MFMA's result
    registers fewer than NEED_OUT wait states later, and no later MFMA may read
    them as its A or B operand that soon (an MFMA accumulating into exactly the
    same registers is the hardware's dependent-accumulation case and is
    allowed).

Wait states are counted as the hardware's hazard rules count them: one per
instruction issued, N + 1 for s_nop N (an intervening MFMA counts one, which
under-counts its real duration, so the check is conservative).  Runs on the
CPU (hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_decode_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
NEED_IN = 4    # a vector write, then an MFMA reading the register (the fences in the source give 4)
NEED_OUT = 20  # a 32x32x16 MFMA's result, then a non-MFMA access (the fences in the source give 20)

_ALL_SOURCES = ("global_store", "buffer_store", "flat_store", "scratch_store", "ds_write", "ds_store",
                "global_atomic", "buffer_atomic", "ds_add", "ds_max", "ds_min", "ds_or", "ds_and")


def regs(tok):
    """Vector registers named by one operand: v5, v[4:7], a3, a[0:15]."""
    tok = tok.strip()
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if re.fullmatch(r"[va]\d+", tok) else set()


def operands(inst):
    parts = inst.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    # operand list up to the first modifier-looking token (offset:, off, glc ...)
    ops = [o.strip() for o in parts[1].split(",")]
    ops = [o.split()[0] if o.split() else o for o in ops]
    return parts[0], ops


def reads_writes(inst):
    """(registers read, registers written) by a vector instruction."""
    name, ops = operands(inst)
    if name.startswith(_ALL_SOURCES) or "_lds" in name:
        return set().union(*[regs(o) for o in ops]) if ops else set(), set()
    if not ops:
        return set(), set()
    return set().union(*[regs(o) for o in ops[1:]]) if len(ops) > 1 else set(), regs(ops[0])


def wait_states(inst):
    if inst.startswith("s_nop"):
        return int(inst.split()[1], 0) + 1
    return 1


def parse(asm):
    """Instructions in order, label -> index of the next instruction, and the
    successors and predecessors of every instruction."""
    insts, labels = [], {}
    for line in asm.split("\n"):
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            labels[s[:-1]] = len(insts)
            continue
        if s.startswith("."):
            continue
        insts.append(s)
    succ = [[] for _ in insts]
    for i, s in enumerate(insts):
        name = s.split()[0]
        tgt = s.split()[1] if len(s.split()) > 1 else None
        if name == "s_branch":
            if tgt in labels:
                succ[i].append(labels[tgt])
            continue
        if name.startswith("s_cbranch") and tgt in labels:
            succ[i].append(labels[tgt])
        if name in ("s_endpgm", "s_setpc_b64"):
            continue
        if i + 1 < len(insts):
            succ[i].append(i + 1)
    pred = [[] for _ in insts]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return insts, succ, pred


def _walk(start, nxt, budget, visit):
    """Visit instructions reachable from `start` along `nxt` edges while fewer
    than `budget` wait states separate them from it: visit(j, ws) -> True stops
    that path."""
    stack = [(j, 0) for j in nxt[start]]
    seen = {}
    while stack:
        j, ws = stack.pop()
        if ws >= budget or seen.get(j, budget + 1) <= ws:
            continue
        seen[j] = ws
        if visit(j, ws):
            continue
        w = wait_states_cache[j]
        for k in nxt[j]:
            stack.append((k, ws + w))


wait_states_cache = []


def scan(asm):
    global wait_states_cache
    insts, succ, pred = parse(asm)
    wait_states_cache = [wait_states(s) for s in insts]
    found = []
    for i, s in enumerate(insts):
        if not s.startswith("v_mfma"):
            continue
        _, ops = operands(s)
        dst = regs(ops[0])
        src_ab = set().union(regs(ops[1]), regs(ops[2]))
        src_c = regs(ops[3]) if len(ops) > 3 else set()
        srcs = src_ab | src_c

        # backward: vector writes of its operands, counting the wait states of
        # the instructions in between (the writer's own issue is not one)
        def back(j, ws):
            p = insts[j]
            if p.startswith("v_mfma") or not (p.startswith("v_") or p.startswith(("ds_", "global_", "buffer_"))):
                return False
            _, wr = reads_writes(p)
            if wr & srcs and p.startswith("v_"):
                found.append(("operand written too early", s, p, ws))
            return False

        stack = [(j, 0) for j in pred[i]]
        seen = {}
        while stack:
            j, ws = stack.pop()
            if ws >= NEED_IN or seen.get(j, NEED_IN + 1) <= ws:
                continue
            seen[j] = ws
            back(j, ws)
            for k in pred[j]:
                stack.append((k, ws + wait_states_cache[j]))

        # forward: readers and overwriters of its result
        def fwd(j, ws):
            p = insts[j]
            if p.startswith("v_mfma"):
                _, pops = operands(p)
                if (regs(pops[1]) | regs(pops[2])) & dst:
                    found.append(("result read as A/B too early", s, p, ws))
                    return True
                pdst = regs(pops[0])
                if pdst & dst:
                    if pdst == dst and len(pops) > 3 and regs(pops[3]) == dst:
                        return True  # the next accumulation into the same registers takes over
                    found.append(("result overlapped by another MFMA", s, p, ws))
                    return True
                return False
            if p.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
                rd, wr = reads_writes(p)
                if (rd | wr) & dst:
                    found.append(("result accessed too early", s, p, ws))
                    return True
            return False

        _walk(i, succ, NEED_OUT, lambda j, ws: fwd(j, ws))
    return found


def _kernels_asm(tmp_path):
    out = tmp_path / "kernels.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "mla_kernels.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_mfma_hazard_in_the_compiled_kernels(tmp_path):
    asm = _kernels_asm(tmp_path)
    assert asm.count("v_mfma_f32_32x32x16_bf16") > 500, "the decode kernels' MFMAs were not found"
    found = scan(asm)
    assert not found, "\n".join(f"{k}: {m}  /  {p}  ({w} wait states)" for k, m, p, w in found[:10])


def test_the_scan_flags_planted_hazards():
    # a VGPR operand written one wait state before the MFMA
    asm = "\n".join(["k:", "v_accvgpr_read_b32 v21, a151", "s_nop 0",
                     "v_mfma_f32_32x32x16_bf16 v[2:17], v[22:25], v[18:21], v[2:17]",
                     "s_nop 15", "s_nop 3",
                     "v_mov_b32 v30, v1", "s_nop 3", "v_mfma_f32_32x32x16_bf16 v[2:17], v[22:25], v[30:33], v[2:17]",
                     "s_nop 15", "s_nop 3", "s_endpgm"])
    found = scan(asm)
    assert len(found) == 1 and "v21" in found[0][2] and found[0][3] == 1, found


def test_the_scan_flags_an_agpr_accumulator_written_too_early():
    asm = "\n".join(["k:", "v_accvgpr_write_b32 a3, 0",
                     "v_mfma_f32_32x32x16_bf16 a[0:15], v[22:25], v[18:21], a[0:15]", "s_nop 15", "s_nop 3",
                     "s_endpgm"])
    found = scan(asm)
    assert len(found) == 1 and found[0][0] == "operand written too early", found


def test_the_scan_flags_a_result_read_too_early():
    asm = "\n".join(["k:", "v_mfma_f32_32x32x16_bf16 a[0:15], v[22:25], v[18:21], a[0:15]",
                     "s_nop 7", "v_accvgpr_read_b32 v40, a5", "s_endpgm"])
    found = scan(asm)
    assert len(found) == 1 and found[0][0] == "result accessed too early" and found[0][3] == 8, found
    # the same with the 20 wait states the fences give passes; so does a
    # dependent accumulation straight after
    ok = "\n".join(["k:", "v_mfma_f32_32x32x16_bf16 a[0:15], v[22:25], v[18:21], a[0:15]",
                    "v_mfma_f32_32x32x16_bf16 a[0:15], v[26:29], v[18:21], a[0:15]",
                    "s_nop 15", "s_nop 3", "v_accvgpr_read_b32 v40, a5", "s_endpgm"])
    assert scan(ok) == []


def test_the_scan_follows_a_loop_back_edge():
    # the MFMA at the loop top reads v30, written at the loop bottom just
    # before the branch back: only the back-edge connects them
    asm = "\n".join(["k:", "s_mov_b32 s0, 4", ".LBB0_1:",
                     "v_mfma_f32_32x32x16_bf16 a[0:15], v[22:25], v[30:33], a[0:15]",
                     "s_nop 15", "s_nop 3", "s_add_u32 s0, s0, -1", "s_cmp_lg_u32 s0, 0",
                     "v_mov_b32 v31, v2", "s_cbranch_scc1 .LBB0_1", "s_endpgm"])
    found = scan(asm)
    assert len(found) == 1 and "v31" in found[0][2], found
