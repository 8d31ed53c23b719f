"""Build the seqcomp HIP library (gfx950) in-tree with hipcc.

Usage: python -m kv_sequence_compression_amd.build [-v]
Produces kv_sequence_compression_amd/libseqcomp.so from csrc/*.hip and
csrc/abi.cpp (objects go to kv_sequence_compression_amd/_build/), and the
measurement-only libseqcomp_probe.so from probe/ceilings.hip.
"""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libseqcomp.so")
# measurement-only module for bench.py: the pooling call's traffic with no
# arithmetic, and the bf16 matrix cores with no data movement
PROBE_SRC = os.path.join(PKG, "probe", "ceilings.hip")
PROBE_LIB = os.path.join(PKG, "libseqcomp_probe.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # gfx950 packed-fp32 instructions stay off (the host pass warns that it
    # does not know the feature; that is harmless).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the seqcomp library)")


def sources():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    return srcs + [os.path.join(CSRC, "abi.cpp")]


# The source files each measured kernel is built from (a stored counter
# summary is valid for a kernel while these files are unchanged).
KERNEL_SOURCES = {
    "gemm": ["csrc/gemm.hip", "csrc/common.hpp", "csrc/amdgcn.hpp", "csrc/launch.hpp"],
    "pool": ["csrc/pool.hip", "csrc/common.hpp", "csrc/launch.hpp"],
    "indexer": ["csrc/indexer.hip", "csrc/common.hpp", "csrc/amdgcn.hpp", "csrc/launch.hpp"],
    "mqa": ["csrc/mqa.hip", "csrc/common.hpp", "csrc/amdgcn.hpp", "csrc/launch.hpp"],
}


def source_digest(files=None) -> str:
    """SHA-256 over library sources (paths relative to the package; default:
    every source and the public header).  Identifies the kernels a stored
    profile or counter summary was taken on."""
    h = hashlib.sha256()
    if files is None:
        paths = sources() + sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")) + [
            os.path.join(ROOT, "include", "seqcomp.h")]
    else:
        paths = [os.path.join(PKG, f) for f in files]
    for path in paths:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append(([hipcc, *COMMON, *lang, "-c", src, "-o", obj], obj))

    def run(cmd):
        p = subprocess.run(cmd, capture_output=True, text=True)
        if verbose or p.returncode:
            sys.stderr.write(" ".join(cmd) + "\n" + p.stdout + p.stderr)
        if p.returncode:
            raise RuntimeError(f"hipcc failed on {cmd[-3]}")

    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(run, [j[0] for j in jobs]))
    tmp = LIB + ".tmp"
    run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[1] for j in jobs]])
    os.replace(tmp, LIB)
    ptmp = PROBE_LIB + ".tmp"
    run([hipcc, *COMMON, "-shared", "-o", ptmp, PROBE_SRC])
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
