"""Build libgdpa.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python -m generalized_attention_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libgdpa.so")

# (the kernel families sit in separate units so that they compile in parallel; largest first)
SOURCES = ["gdpa_bwd_pw.hip", "gdpa_fwd_any.hip", "gdpa_bwd_mix_all.hip", "gdpa_bwd_mix_d128.hip",
           "gdpa_bwd_mix_d64.hip", "gdpa_bwd_mix_d32.hip", "gdpa_bwd_agpr.hip", "gdpa_bwd_sm.hip", "gdpa_fwd.hip",
           "gdpa_bwd.hip", "gdpa_api.cpp", "gdpa_sched.hip", "gdpa_fp32.hip"]
# Per-source options. Most backward kernels keep MFMA results in the VGPR form (no register-class
# copies between the score accumulators and the element-wise code); the kernel families that this
# compiler cannot build that way live in sources of their own.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"gdpa_bwd.hip": _VGPR_FORM, "gdpa_bwd_pw.hip": _VGPR_FORM, "gdpa_bwd_sm.hip": _VGPR_FORM}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are switched off: every kernel is written with scalar fp32.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
          "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 16)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
