"""Guards on the generated gfx950 code of the kernels (host only: hipcc -S).

* Both main loops prefetch tiles with direct-to-LDS loads that stay in flight while the
  current tile is consumed.  The compiler's wait analysis can silently defeat that by
  inserting ``s_waitcnt vmcnt(0)`` (wait for every outstanding load) in front of an LDS read
  it cannot tell apart from the loads in flight, or by spilling to scratch (whose reloads need
  the same wait).  The kernels are compiled the way the library build does, and inside each
  main loop no such wait may follow the tile loads and nothing may spill.
* A matrix-core (MFMA) result may be read or overwritten by another instruction only after
  a number of wait states that the hardware does not enforce; the compiler pads straight-line
  code with ``s_nop``, but it once left a read one instruction behind the MFMA on the taken
  side of a branch, which made the result depend on timing.  Every path after every MFMA in
  every library source is checked.
"""

import os
import re
import shutil
import subprocess

import pytest

from mlra_latent_kv_amd import build

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _asm(src: str, tmp_path) -> str:
    out = tmp_path / (src + ".s")
    cmd = [HIPCC] + build._flags() + build._hip_flags(src) + [
        "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def _kernels(asm: str):
    """(name, body lines, metadata text) of each k_main kernel in the assembly."""
    out = []
    for m in re.finditer(r"^(_ZN3mla\w*k_main_bf16\w*):.*$", asm, re.M):
        name = m.group(1)
        end = asm.index("s_endpgm", m.end())
        meta = asm[asm.index(f".amdhsa_kernel {name}"):]
        meta = meta[:meta.index(".end_amdhsa_kernel")]
        out.append((name, asm[m.end():end].splitlines(), meta))
    return out


def _main_loop(lines):
    """Lines of the innermost loop that issues tile loads: from its header label to the last
    branch back to it.  (The label of a nested loop carries the header note on the next
    line.)"""
    best = None
    for i, ln in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):", ln)
        if not m or "Loop Header" not in ln + (lines[i + 1] if i + 1 < len(lines) else ""):
            continue
        label = m.group(1)
        back = [j for j in range(i + 1, len(lines))
                if re.search(r"s_(c)?branch\w*\s+" + re.escape(label) + r"\b", lines[j])]
        if not back:
            continue
        body = lines[i:back[-1] + 1]
        if any("lds" in x and "buffer_load" in x for x in body):
            if best is None or len(body) < len(best):
                best = body
    return best


@pytest.mark.parametrize("src", ["main_bf16.hip", "main_bf16_wide.hip"])
def test_main_loop_keeps_tile_loads_in_flight(src, tmp_path):
    kernels = _kernels(_asm(src, tmp_path))
    assert kernels, "no main-loop kernel found"
    for name, lines, _meta in kernels:
        body = _main_loop(lines)
        assert body is not None, (name, "main loop not found")
        first_dma = next(i for i, x in enumerate(body) if "buffer_load" in x and "lds" in x)
        waits = [x.strip() for x in body[first_dma:] if re.search(r"s_waitcnt\s.*vmcnt\(0\)", x)]
        assert not waits, (name, "drains the tile loads inside the loop", waits)
        spills = [x.strip() for x in body if "scratch_" in x]
        assert not spills, (name, "spills inside the loop", spills[:4])


# Wait states an instruction that reads or writes an MFMA's destination registers must stay
# behind it: the padding hipcc itself inserts in straight-line code for these shapes on
# gfx950 (bf16 16x16x32: s_nop 7; 32x32x16: s_nop 11).
_MFMA_WAIT = {"16x16": 8, "32x32": 12}


def _regs(spec):
    """Registers an operand names, as (file, index) pairs: VGPRs and accumulation registers
    are separate files."""
    m = re.match(r"([va])\[(\d+):(\d+)\]", spec)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", spec)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _parse(asm: str):
    ins, labels = [], {}
    for raw in asm.splitlines():
        ln = raw.split(";")[0].strip()
        if not ln:
            continue
        m = re.match(r"^(\.LBB\w+):", ln)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if ln.startswith(".") or ln.endswith(":"):
            continue
        parts = ln.split(None, 1)
        ops = [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((parts[0], ops, ln))
    return ins, labels


def mfma_hazards(asm: str):
    """(mfma, consumer, wait states) for every instruction that touches an MFMA's destination
    registers too early on some path (fall-through or branch) after it.  A later MFMA that
    only accumulates into the same registers (source C) is the hardware's own chained case;
    one that rewrites them ends the path."""
    ins, labels = _parse(asm)
    bad = []
    for i, (op, ops, ln) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        need = next(v for k, v in _MFMA_WAIT.items() if k in op)
        dst = _regs(ops[0])
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, ws = stack.pop()
            if j >= len(ins) or ws >= need or (j, ws) in seen:
                continue
            seen.add((j, ws))
            op2, ops2, ln2 = ins[j]
            if op2 == "s_endpgm":
                continue
            if op2.startswith("s_nop"):
                stack.append((j + 1, ws + int(ops2[0], 0) + 1))
                continue
            if op2.startswith("v_mfma"):
                if _regs(ops2[1]) & dst or _regs(ops2[2]) & dst:
                    bad.append((ln, ln2, ws))
                elif not _regs(ops2[0]) & dst:
                    stack.append((j + 1, ws + 1))
                continue  # chained accumulation or redefinition: path ends
            if any(_regs(o) & dst for o in ops2):
                bad.append((ln, ln2, ws))
                continue
            if op2.startswith("s_branch"):
                stack.append((labels[ops2[0]], ws + 1))
                continue
            if op2.startswith("s_cbranch"):
                stack.append((labels[ops2[0]], ws + 1))
            stack.append((j + 1, ws + 1))
    return sorted(set(bad))


def test_hazard_scan_sees_a_read_behind_a_branch():
    """The checker itself: a read of the MFMA result on the taken side of a branch, one wait
    state behind it, is reported; with the compiler's padding it is not."""
    bad = """
        v_mfma_f32_16x16x32_bf16 v[136:139], v[202:205], v[132:135], v[136:139]
        s_cbranch_scc1 .LBB0_21
        s_nop 7
        v_cndmask_b32_e64 v139, v191, v139, s[14:15]
    .LBB0_21:
        v_max_f32_e32 v140, v139, v139
        s_endpgm
    """
    hz = mfma_hazards(bad)
    assert len(hz) == 1 and "v_max_f32" in hz[0][1] and hz[0][2] == 1
    good = bad.replace("s_cbranch_scc1 .LBB0_21", "s_nop 7\n        s_cbranch_scc1 .LBB0_21")
    assert mfma_hazards(good) == []


@pytest.mark.parametrize("src", build.HIP_SOURCES)
def test_no_early_reads_of_mfma_results(src, tmp_path):
    hz = mfma_hazards(_asm(src, tmp_path))
    assert not hz, (src, hz[:4])
