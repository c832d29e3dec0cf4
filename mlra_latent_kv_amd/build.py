"""Build ``libmla_decode.so`` (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m mlra_latent_kv_amd.build`` (or ``build()``).  Each source compiles to
an object under ``_build/`` in parallel, then links into
``mlra_latent_kv_amd/libmla_decode.so``.  It always recompiles.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_decode.so")
PROBE_LIB = os.path.join(PKG, "libmla_probe.so")  # read-stream probe (benchmark support)
ARCH = "gfx950"

HIP_SOURCES = ["api.hip", "kernels_generic.hip", "kernels_bf16_aux.hip", "main_bf16.hip",
               "main_bf16_wide.hip", "append.hip", "prefill.hip"]
CXX_SOURCES = ["plan.cpp"]
PROBE_SOURCES = ["probe.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Sources whose MFMAs keep the compiler's default accumulation-register (AGPR) form: the
# 128-head main loop holds its 256-register output there for the whole loop.
AGPR_FORM_SOURCES = {"main_bf16_wide.hip"}


def _hip_flags(src: str = ""):
    # packed-fp32 instruction selection is disabled for all device code
    flags = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops"]
    if os.path.basename(src) not in AGPR_FORM_SOURCES:
        # keep MFMA accumulators in VGPRs: the softmax may rescale them every tile, and
        # VALU cannot operate on AGPRs (each rescale would copy them out and back)
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return flags


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags()
    if src.endswith(".hip"):
        cmd += _hip_flags(src)
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    und = subprocess.run(["nm", "-u", "-C", tmp], capture_output=True, text=True).stdout
    missing = [ln.strip() for ln in und.splitlines() if "mla::" in ln]
    if missing:
        raise RuntimeError(f"unresolved library symbols: {missing}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CXX_SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in HIP_SOURCES + CXX_SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
