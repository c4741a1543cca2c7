"""Build libtriattn.so in-tree with hipcc for gfx950.

    python -m protein_pair_representation_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libtriattn.so")
SOURCES = [os.path.join(PKG_DIR, "csrc", "triattn_kernels.hip"),
           os.path.join(PKG_DIR, "csrc", "triattn_abi.cpp"),
           os.path.join(PKG_DIR, "csrc", "aaq_kernels.hip"),
           os.path.join(PKG_DIR, "csrc", "aaq_abi.cpp"),
           os.path.join(PKG_DIR, "csrc", "knn_kernels.hip"),
           os.path.join(PKG_DIR, "csrc", "knn_abi.cpp")]
# measurement-only library: issue costs of the attention loop's instruction mix (bench.py --issue-probe)
PROBE_PATH = os.path.join(PKG_DIR, "libissueprobe.so")
PROBE_SOURCES = [os.path.join(PKG_DIR, "csrc", "issue_probe.hip")]
ARCH = "gfx950"
# Packed fp32 instructions are switched off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build libtriattn.so")


def build(verbose: bool = False, out: str = LIB_PATH, extra_flags=(), sources=None) -> str:
    """Compile the kernels and the C ABI into `out` (always recompiles); extra_flags
    are added to the hipcc line (e.g. host-only instrumentation for a test build)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-shared", "-I", os.path.join(ROOT, "include"),
           *(sources or SOURCES), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("unknown target feature", "packed-fp32-ops", "warning generated", "warnings generated")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    """Compile the issue-cost probe library (measurement only, not the attention path)."""
    return build(verbose=verbose, out=PROBE_PATH, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
