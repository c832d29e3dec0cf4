"""Guards on the generated gfx950 code of the main-loop kernels (host only: hipcc -S).

Both main loops prefetch tiles with direct-to-LDS loads that stay in flight while the current
tile is consumed.  The compiler's wait analysis can silently defeat that by inserting
``s_waitcnt vmcnt(0)`` (wait for every outstanding load) in front of an LDS read it cannot
tell apart from the loads in flight, or by spilling to scratch (whose reloads need the same
wait).  These tests compile the kernels the way the library build does and check that
inside each main loop no such wait follows the tile loads, and that nothing spills.
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
