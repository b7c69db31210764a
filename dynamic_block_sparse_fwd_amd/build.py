"""Build libnsa.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnsa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # never let the compiler form packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs (no AGPR round trips for the softmax arithmetic)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


BUILD_INFO = os.path.join(PKG, "libnsa.buildinfo.json")


def source_digest() -> str:
    """sha256 (first 16 hex digits) over every file of csrc/, names and contents, in name order."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _write_build_info() -> None:
    """Record the commit the library was built from (when the tree is a git checkout), so that a
    copy of the tree without its history can still name it; the source digest ties the record
    to the sources it describes."""
    import json

    sha, dirty = None, None
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
        if sha:
            st = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--",
                                 os.path.join(PKG, "csrc")], capture_output=True, text=True,
                                timeout=10).stdout
            dirty = bool(st.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    with open(BUILD_INFO, "w") as fh:
        json.dump({"git_sha": sha, "csrc_modified_since_commit": dirty,
                   "library_source_sha256": source_digest()}, fh)


def build(verbose: bool = False) -> str:
    """Compile every kernel source and the C-ABI layer into one shared library."""
    objs = []
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    procs = []
    for src in sources():
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        cmd = ["hipcc", *HIPCC_FLAGS, "-c", "-I", os.path.join(ROOT, "include"), src, "-o", obj]
        cmd.remove("-shared")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    failed = False
    for p, src in procs:
        _, err = p.communicate()
        lines = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed = True
            print("hipcc failed on %s" % src, file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed")
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
