"""Build libfa.so (the HIP library behind include/fa.h) in-tree for gfx950.

    python -m exact_attention_17_amd.build          # or build_library()

One hipcc invocation compiles the C-ABI layer and the kernels into a shared
library next to this file.  Packed-fp32 instruction selection is disabled
(-packed-fp32-ops), so the compiler emits scalar fp32 VALU ops only.
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# The same sources with -DFA_DEBUG: every direct-to-LDS tile load first fills
# its destination with bf16 NaN, so a missing wait or barrier shows as NaN in
# the outputs (tests/test_debug_build.py compares it with the release library).
DEBUG_LIB_PATH = os.path.join(PKG_DIR, "libfa_debug.so")
# A streaming-read bandwidth probe for the benchmark (its own library; the
# attention library does not contain it).
MEMBW_LIB_PATH = os.path.join(PKG_DIR, "libfa_membw.so")
MEMBW_SOURCE = "membw.hip"
SOURCES = ["fa_api.cpp", "plan.cpp", "prefill_fwd.hip", "prefill_wide.hip", "decode_paged.hip",
           "attn_bwd.hip", "debug_checks.hip"]
ARCH = "gfx950"


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libfa.so")


def compile_command(out=LIB_PATH, extra=(), sources=SOURCES):
    cmd = [hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", INCLUDE, "-I", CSRC, "-o", out]
    cmd += list(extra)
    cmd += [os.path.join(CSRC, s) for s in sources]
    return cmd


def build_library(verbose=False, extra=(), debug=False, membw=False):
    """Compile every HIP source into LIB_PATH, or with debug=True into
    DEBUG_LIB_PATH with -DFA_DEBUG, or with membw=True the bandwidth probe
    into MEMBW_LIB_PATH (always recompiles)."""
    target = MEMBW_LIB_PATH if membw else DEBUG_LIB_PATH if debug else LIB_PATH
    tmp = target + ".tmp"
    cmd = compile_command(tmp, list(extra) + (["-DFA_DEBUG"] if debug else []),
                          [MEMBW_SOURCE] if membw else SOURCES)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_library(verbose=True, debug=True))
    print(build_library(verbose=True, membw=True))
