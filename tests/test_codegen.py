"""Guards on the generated gfx950 code of the kernels (host only: hipcc -S).

* Both main loops and the two prefill kernels prefetch tiles with direct-to-LDS loads that
  stay in flight while the current tile is consumed.  The compiler's wait analysis can
  silently defeat that by inserting ``s_waitcnt vmcnt(0)`` (wait for every outstanding load)
  in front of an LDS read it cannot tell apart from the loads in flight, or by spilling to
  scratch (whose reloads need the same wait).  The kernels are compiled the way the library
  build does, and inside each main loop no such wait may follow the tile loads and nothing
  may spill.
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


def _kernels(asm: str, pattern: str = r"k_main_bf16\w*"):
    """(name, body lines, metadata text) of each kernel whose name matches `pattern`."""
    out = []
    for m in re.finditer(r"^(_ZN3mla\w*" + pattern + r"):.*$", asm, re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        meta = asm[asm.index(f".amdhsa_kernel {name}"):]
        meta = meta[:meta.index(".end_amdhsa_kernel")]
        out.append((name, asm[m.end():end].splitlines(), meta))
    return out


def _blocks(lines):
    """Labelled basic blocks (label, note, instruction lines) in text order.  Unlabelled
    fall-through blocks (%bb.N) stay merged into the block before them."""
    blocks = []
    for ln in lines:
        m = re.match(r"^\.(LBB\w+):(.*)$", ln)
        if m:
            blocks.append((m.group(1), m.group(2), []))
        elif blocks and not blocks[-1][2] and ln.strip().startswith(";"):
            # a note continued on its own line (nested loops: "Parent Loop ..." on the label
            # line, "This Inner Loop Header" on the next)
            blocks[-1] = (blocks[-1][0], blocks[-1][1] + ln.strip(), blocks[-1][2])
        elif blocks:
            ins = ln.split(";")[0].strip()
            if ins and not ins.startswith("."):
                blocks[-1][2].append(ins)
    return blocks


def _main_loop(lines):
    """(blocks, header index, loop block indices) of the innermost loop that issues tile
    loads.  Membership comes from the assembler's "in Loop: Header=" notes: the compiler may
    rotate a loop so that its latch precedes the header and falls through into it."""
    blocks = _blocks(lines)
    loops = {}
    for i, (label, note, _) in enumerate(blocks):
        m = re.search(r"in Loop: Header=(BB\w+) Depth", note)
        if "Inner Loop Header" in note:
            loops.setdefault(label[1:], set()).add(i)
        elif m:
            loops.setdefault(m.group(1), set()).add(i)
    best = None
    for hdr, members in loops.items():
        head = next((i for i in members if blocks[i][0] == "L" + hdr), None)
        if head is None or "Inner Loop Header" not in blocks[head][1]:
            continue
        if any("lds" in x and "buffer_load" in x for i in members for x in blocks[i][2]):
            if best is None or len(members) < len(best[2]):
                best = (blocks, head, members)
    return best


def _drains_after_issue(blocks, head, members):
    """vmcnt(0) waits on any path from a tile load of the loop to the next pass through the
    loop header (a wait at the top of an iteration, before the next tile goes out, is the
    kernel's own choice; a wait between issuing a tile and the end of the iteration would
    drain it).  A full wait directly followed by the tile barrier (s_waitcnt lgkmcnt(0);
    s_barrier) is the kernel's explicit wait for a tile it must have complete (the pipelined
    loop keeps exactly one tile in flight), not a drain of loads still ahead."""
    index = {b[0]: i for i, b in enumerate(blocks)}
    starts = [(i, j + 1) for i in members for j, x in enumerate(blocks[i][2])
              if "buffer_load" in x and "lds" in x]
    seen, found, stack = set(), [], list(starts)
    while stack:
        i, j = stack.pop()
        if (i, j) in seen:
            continue
        seen.add((i, j))
        ins = blocks[i][2]
        if j >= len(ins):  # fall through
            if i + 1 in members and i + 1 != head:
                stack.append((i + 1, 0))
            continue
        x = ins[j]
        if re.match(r"s_waitcnt\s.*vmcnt\(0\)", x) and not (
                ins[j + 1:j + 3] == ["s_waitcnt lgkmcnt(0)", "s_barrier"]):
            found.append((blocks[i][0], x))
        m = re.match(r"s_(c)?branch\w*\s+\.(LBB\w+)", x)
        if m:
            t = index.get(m.group(2))
            if t is not None and t in members and t != head:
                stack.append((t, 0))
            if not m.group(1):
                continue  # unconditional: no fall-through
        if x.startswith("s_endpgm"):
            continue
        stack.append((i, j + 1))
    return found


@pytest.mark.parametrize("src,pattern", [("main_bf16.hip", r"k_main_bf16\w*"),
                                         ("main_bf16_wide.hip", r"k_main_bf16\w*"),
                                         ("prefill.hip", r"k_prefill_(?:attn|kv)\w*")])
def test_main_loop_keeps_tile_loads_in_flight(src, pattern, tmp_path):
    """Also the prefill's two kernels: the attention's key-tile ring and the projection's
    double-buffered latent and weight chunks."""
    kernels = _kernels(_asm(src, tmp_path), pattern)
    assert len(kernels) >= (2 if src == "prefill.hip" else 1), "no main-loop kernel found"
    for name, lines, _meta in kernels:
        loop = _main_loop(lines)
        if loop is None and "k_prefill_kvILi128E" in name:
            continue  # 128-wide MLRA branches: two chunks, fully unrolled, no loop
        assert loop is not None, (name, "main loop not found")
        blocks, head, members = loop
        waits = _drains_after_issue(blocks, head, members)
        assert not waits, (name, "drains the tile loads inside the loop", waits)
        spills = [x for i in members for x in blocks[i][2] if "scratch_" in x]
        assert not spills, (name, "spills inside the loop", spills[:4])


def test_drain_scan_sees_a_wait_after_the_issue():
    # rotated loop: the latch (LBB0_3) falls through into the header (LBB0_4)
    loop = """.LBB0_2:                ;   in Loop: Header=BB0_4 Depth=1
\tv_add_u32 v1, v1, v2
{late}.LBB0_3:                ;   in Loop: Header=BB0_4 Depth=1
\ts_add_i32 s4, s4, 1
.LBB0_4:                ; =>This Inner Loop Header: Depth=1
\ts_waitcnt vmcnt(0)
\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds
\ts_cbranch_scc1 .LBB0_2
\ts_branch .LBB0_3
.LBB0_5:
\ts_endpgm
"""
    bad = _main_loop(loop.format(late="\ts_waitcnt vmcnt(0)\n").splitlines())
    assert [w[0] for w in _drains_after_issue(*bad)] == ["LBB0_2"]
    good = _main_loop(loop.format(late="").splitlines())  # the wait at the top only
    assert _drains_after_issue(*good) == []
    # the explicit wait for the one tile in flight, right before the tile barrier
    barrier = "\ts_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n"
    assert _drains_after_issue(*_main_loop(loop.format(late=barrier).splitlines())) == []


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
