"""Build ``libddtree.so`` in-tree with hipcc for gfx950 only.

    python tree_verify_mla_absorb_amd/build.py

(Run it as a script: importing the package loads the library, which may not exist yet.)

The library is a plain C-ABI shared object (``include/ddtree.h``); it links against the HIP
runtime only.  Every HIP source is compiled with packed-fp32 instruction selection turned off.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["verify_attn.hip", "compact_kv.hip", "accept.hip", "compact_layers.hip", "append_kv.hip", "build_tree.hip", "ddtree_api.hip"]
LIB = os.path.join(PKG, "libddtree.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libddtree.so")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libddtree.so`` next to this file; returns its path."""
    objs = []
    procs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for cmd, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed ({p.returncode}): {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout.decode(errors='replace')}")
    os.replace(tmp, LIB)
    write_build_info()
    return LIB


BUILD_INFO = os.path.join(PKG, "libddtree.build.json")


def write_build_info() -> None:
    """Record what the library was built from next to it (git HEAD when the tree is a checkout,
    the compiler's version line), so that a copy of the tree without its history still says."""
    import json

    def run(cmd):
        try:
            r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, timeout=30)
            return r.stdout.strip() if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None

    info = {
        "git_head": run(["git", "-C", ROOT, "rev-parse", "HEAD"]),
        "git_dirty": bool(run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"])),
        "hipcc": (run([hipcc(), "--version"]) or "").splitlines()[0:1],
        "arch": ARCH,
    }
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
