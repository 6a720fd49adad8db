"""Build the HIP library (gfx950) in-tree: ``python grouped_expert_ffn_amd/build.py``.

This file uses the standard library only, so it runs (and imports) without
the package, whose import needs the library already built.

Every ``csrc/*.hip`` file is compiled to an object in parallel under
``_build/``, then linked into ``libmoe_dispatch.so`` next to this file.
"""
from __future__ import annotations

import glob
import json
import os
import shutil
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_dispatch.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept off: hipcc would otherwise fuse pairs of
# float operations into v_pk_* instructions.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _write_build_info():
    """Record the git commit the library was built from (and whether the
    tree had changes), so a copy of the tree without its .git directory can
    still name the sources of its library."""
    info = {"built_at": int(time.time()), "git_sha": None, "git_dirty": None}
    root = os.path.dirname(PKG)
    try:
        sha = subprocess.run(["git", "-C", root, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=30)
        if sha.returncode == 0:
            info["git_sha"] = sha.stdout.strip()
            st = subprocess.run(["git", "-C", root, "status", "--porcelain", "--", "include",
                                 "grouped_expert_ffn_amd/csrc"], capture_output=True, text=True,
                                timeout=30)
            info["git_dirty"] = bool(st.stdout.strip()) if st.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(BUILD, "build_info.json"), "w") as f:
        json.dump(info, f)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link the shared library.
    Always recompiles. Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        return _run([hipcc, *COMMON_FLAGS, "-c", src, "-o", obj])

    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        outs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    _write_build_info()
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
