"""Build the HIP library ``libfa.so`` in-tree for gfx950 with hipcc.

    python exact_attention_125_amd/build.py   (runs without importing the package, whose
                                              import needs the built library)

Every source under ``csrc/`` is compiled to an object in ``_build/`` (in parallel) and
linked into ``exact_attention_125_amd/libfa.so``.  All device code is compiled with packed
fp32 instructions disabled.  The device code of the kernels that issue MFMAs and LDS reads as
inline assembly is also compiled to assembly and checked (``isa_check.py``); a finding fails
the build.
"""
from __future__ import annotations

import concurrent.futures as cf
import importlib.util
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = os.environ.get("FA_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


# sources whose MFMAs are inline assembly (full check) and whose LDS reads are (LDS check)
ASM_MFMA = ("bwd_dkdv.hip", "bwd_dq.hip")
ASM_LDS = ("fwd_main.hip",)


def _isa_check_module():
    spec = importlib.util.spec_from_file_location("fa_isa_check", os.path.join(PKG, "isa_check.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _check(item):
    name, mfma = item
    _isa_check_module().check_sources([os.path.join(CSRC, name)], COMMON, _hipcc(), BUILD, mfma=mfma)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    checks = [(n, True) for n in ASM_MFMA] + [(n, False) for n in ASM_LDS]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(checks))) as ex:
        pending = [ex.submit(_check, c) for c in checks]
        objs = list(ex.map(_compile, srcs))
        for f in pending:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
