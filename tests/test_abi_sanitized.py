"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host pass
(kv_sequence_compression_amd/build_sanitized.py; device code unchanged) and
tests/test_abi_cpu.py runs against it in a child process with the ASan
runtime preloaded.  Those tests drive every validation path of every entry
point with fake device addresses and reach no kernel launch, so they run
without a GPU.  A planted over-read of a host array shows that the sanitizer
is live in that setup.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc_available():
    return any(p and os.path.exists(p) for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                                                shutil.which("hipcc")))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not _hipcc_available():
        pytest.skip("hipcc is needed to build the sanitized library")
    sys.path.insert(0, ROOT)
    from kv_sequence_compression_amd import build_sanitized as bs
    out = str(tmp_path_factory.mktemp("asan") / "libseqcomp_asan.so")
    bs.build(out)
    rt = bs.runtime_path()
    if not os.path.exists(rt):
        pytest.skip("no shared ASan runtime next to hipcc")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", SEQCOMP_LIBRARY=out)
    return env


def test_abi_validation_is_clean_under_sanitizers(sanitized):
    """Every case of tests/test_abi_cpu.py, host code sanitized: no report."""
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=sanitized, capture_output=True, text=True,
                       timeout=600)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr


def test_sanitizer_catches_a_planted_overread(sanitized):
    """seqcomp_num_entries told that a 2-element offsets array has 50
    sequences reads past it: ASan must stop the process."""
    code = (
        "import ctypes\n"
        "from kv_sequence_compression_amd import _lib\n"
        "lib = _lib.load()\n"
        "libc = ctypes.CDLL(None)\n"
        "libc.malloc.restype = ctypes.c_void_p\n"
        "p = libc.malloc(16)\n"
        "a = ctypes.cast(p, ctypes.POINTER(ctypes.c_int64))\n"
        "a[0] = 0; a[1] = 8\n"
        "print(lib.seqcomp_num_entries(a, 50, 4))\n"
    )
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode != 0
    assert "heap-buffer-overflow" in p.stderr
