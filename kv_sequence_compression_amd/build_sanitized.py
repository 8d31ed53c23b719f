"""Host-sanitized build of the seqcomp library, for the CPU tests of the C ABI.

Usage: python -m kv_sequence_compression_amd.build_sanitized [out.so]

The host code (argument validation, workspace layout, launch sizing) is built
with AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built
as usual (every sanitizer flag is scoped to the host pass).  Loading the result
from an uninstrumented Python needs the ASan runtime preloaded; see
tests/test_abi_sanitized.py.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from .build import ARCH, COMMON, PKG, _hipcc, sources

BUILD = os.path.join(PKG, "_build_asan")
LIB = os.path.join(PKG, "libseqcomp_asan.so")
HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-g"]


def runtime_path() -> str:
    """The shared ASan runtime that the sanitized library links against."""
    out = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build(out: str = LIB) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append(([hipcc, *COMMON, *HOST_FLAGS, *lang, "-c", src, "-o", obj], obj))

    def run(cmd):
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode:
            sys.stderr.write(" ".join(cmd) + "\n" + p.stdout + p.stderr)
            raise RuntimeError(f"hipcc failed on {cmd[-3]}")

    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(run, [j[0] for j in jobs]))
    tmp = out + ".tmp"
    run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_FLAGS, "-shared-libsan", "-o", tmp,
         *[j[1] for j in jobs]])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else LIB))
