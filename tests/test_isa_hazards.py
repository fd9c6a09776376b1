"""The dense GEMM's accumulators are written by MFMAs issued through inline
asm, so the compiler does not know that a result lands some cycles after the
instruction issues.  This CPU test compiles gemm_bf16.hip for gfx950, keeps
the assembly, and checks on every control-flow path of every kernel instance
that no AGPR an MFMA writes is read (v_accvgpr_read / v_accvgpr_mov) within
32 wait states of that MFMA.  (Reads inside MFMAs, as their tied addend, are
ordered by the hardware and are not checked.)  Such a read gave wrong sums
twice: the output conversion hoisted above the wait states, and a register
copy at the 256 x 224 tile's loop exit."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "quantized_fine_tuning_nf4_amd", "csrc", "gemm_bf16.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
WAIT_STATES = 32


def _regs(spec):
    m = re.match(r"a\[(\d+):(\d+)\]", spec.strip())
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", spec.strip())
    return {int(m.group(1))} if m else set()


def _blocks(lines):
    """Basic blocks (label, [instructions]) and their predecessors."""
    blocks, cur = [], ("entry", [])
    for t in lines:
        if re.match(r"^\.LBB[\w_]+:", t):
            blocks.append(cur)
            cur = (t.split(":")[0], [])
            continue
        if t.startswith("."):
            continue
        cur[1].append(t)
        if t.startswith("s_cbranch") or t.startswith("s_branch"):
            blocks.append(cur)
            cur = (f"ft{len(blocks)}", [])
    blocks.append(cur)
    index = {b[0]: k for k, b in enumerate(blocks)}
    preds = {k: [] for k in range(len(blocks))}
    for k, (_, ins) in enumerate(blocks):
        last = ins[-1] if ins else ""
        if last.startswith("s_branch"):
            if last.split()[1] in index:
                preds[index[last.split()[1]]].append(k)
            continue
        if k + 1 < len(blocks):
            preds[k + 1].append(k)
        if last.startswith("s_cbranch") and last.split()[1] in index:
            preds[index[last.split()[1]]].append(k)
    return blocks, preds


def _cost(t):
    return int(t.split()[1]) + 1 if t.split()[0] == "s_nop" else 1


def _hazards(lines):
    blocks, preds = _blocks(lines)
    found = []

    def back(k, end, src, ws, seen):
        ins = blocks[k][1]
        for j in range(end - 1, -1, -1):
            t = ins[j]
            if t.startswith("v_mfma") and _regs(t.split()[1].rstrip(",")) & src:
                return t, ws
            ws += _cost(t)
            if ws >= WAIT_STATES:
                return None
        for p in preds[k]:
            if (p, ws) not in seen:
                seen.add((p, ws))
                r = back(p, len(blocks[p][1]), src, ws, seen)
                if r:
                    return r
        return None

    for k, (_, ins) in enumerate(blocks):
        for j, t in enumerate(ins):
            if t.startswith("v_accvgpr_read") or t.startswith("v_accvgpr_mov"):
                r = back(k, j, _regs(t.split(",")[-1]), 0, set())
                if r:
                    found.append((t, r))
    return found


def _kernels(asm):
    """Instruction lines of each k_gemm_nt instance in the assembly."""
    out, name, body = {}, None, []
    for raw in asm.splitlines():
        t = raw.strip()
        if not t or t.startswith(";"):
            continue
        m = re.match(r"^(_Z\w*k_gemm_nt\w*):", t)
        if m:
            name, body = m.group(1), []
            continue
        if name:
            if t.startswith("s_endpgm"):
                out[name] = body
                name = None
            else:
                body.append(t)
    return out


def test_checker_finds_a_planted_hazard():
    lines = ["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
             "s_cbranch_scc1 .LBB0_2",
             "v_mov_b32 v8, 0",
             ".LBB0_2:",
             "v_accvgpr_read_b32 v9, a2"]
    assert len(_hazards(lines)) == 1
    safe = lines[:1] + ["s_nop 15", "s_nop 15"] + lines[1:]
    assert _hazards(safe) == []


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not installed")
def test_gemm_reads_no_accumulator_early():
    with tempfile.TemporaryDirectory() as d:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-ffp-contract=off", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-c", SRC, "-o", os.path.join(d, "g.o"), "--save-temps"]
        r = subprocess.run(cmd, cwd=d, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        asm = [f for f in os.listdir(d) if f.endswith("gfx950.s")]
        assert asm, os.listdir(d)
        kernels = _kernels(open(os.path.join(d, asm[0])).read())
    # 3 tile shapes x (r == 16 or not) x (reduction tail or not)
    assert len(kernels) >= 12, sorted(kernels)
    for name, lines in kernels.items():
        assert sum(t.startswith("v_mfma") for t in lines) > 0, name
        h = _hazards(lines)
        assert not h, (name, h[:3])
