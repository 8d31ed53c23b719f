"""ctypes loader of the in-tree HIP library ``libseqcomp.so``.

Argument marshalling only.  Raises ImportError with a clear message when the
library has not been built: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

# SEQCOMP_LIBRARY names another build of the same library (the host-sanitized
# one of the C ABI tests); by default the in-tree libseqcomp.so.
LIB_PATH = os.environ.get("SEQCOMP_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libseqcomp.so")

# Mirror of the enums in include/seqcomp.h.
OK = 0
E_SCRATCH = 10
F32, BF16, FP8_E4M3 = 0, 1, 2
MODE_CSA, MODE_HCA = 0, 1
OP_POOL_CSA, OP_POOL_HCA, OP_FUSED = 0, 1, 2

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_vp = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)
_size = ctypes.c_size_t

# name -> (restype, argtypes); must match include/seqcomp.h
SIGNATURES = {
    "seqcomp_version": (_c_int, []),
    "seqcomp_status_string": (ctypes.c_char_p, [_c_int]),
    "seqcomp_num_entries": (_c_i64, [_i64p, _c_i64, _c_i64]),
    "seqcomp_workspace_bytes": (_size, [_c_int, _c_int, _c_i64, _c_i64, _i64p, _c_i64, _c_int]),
    "seqcomp_project": (_c_int, [_vp, _c_i64, _c_i64, _c_int, _vp, _c_i64, _vp, _c_i64, _c_int, _vp]),
    "seqcomp_pool_csa": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_int, _vp, _vp, _c_i64, _c_i64,
                                  _i64p, _vp, _c_i64, _vp, _c_int, _vp, _vp, _size, _vp]),
    "seqcomp_pool_hca": (_c_int, [_vp, _vp, _c_i64, _c_int, _vp, _c_i64, _c_i64,
                                  _i64p, _vp, _c_i64, _vp, _c_int, _vp, _vp, _size, _vp]),
    "seqcomp_compress_fused": (_c_int, [_c_int, _c_i64, _vp, _c_i64, _c_int, _vp, _c_i64, _vp, _vp,
                                        _i64p, _vp, _c_i64, _vp, _c_int, _vp, _vp, _size, _vp]),
    "seqcomp_compress_fused_noalloc": (_c_int, [_c_int, _c_i64, _vp, _c_i64, _c_int, _vp, _c_i64, _vp, _vp,
                                                _i64p, _vp, _c_i64, _vp, _c_int, _vp, _vp]),
    "seqcomp_csa_append": (_c_int, [_vp, _c_i64, _c_i64, _c_int, _vp, _c_i64, _vp, _vp, _vp, _vp,
                                    _vp, _c_int, _vp, _vp, _size, _vp]),
    "seqcomp_append_workspace_bytes": (_size, [_c_i64, _c_i64, _c_int]),
    "seqcomp_rope_store": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _i64p, _vp, _c_i64, _vp, _c_i64, ctypes.c_double,
                                    _vp, _c_i64, _vp, _vp, _vp, _vp, _size, _vp]),
    "seqcomp_rope_store_workspace_bytes": (_size, [_c_i64, _i64p, _c_i64]),
    "seqcomp_indexer_topk": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _c_int, _i64p, _vp, _i64p, _vp, _c_i64,
                                      _vp, _c_i64, _vp, _vp, _vp, _size, _vp]),
    "seqcomp_indexer_workspace_bytes": (_size, [_i64p, _c_i64]),
    "seqcomp_shared_kv_mqa": (_c_int, [_vp, _vp, _c_i64, _c_i64, _c_int, _i64p, _vp, _i64p, _vp, _c_i64, _vp, _vp,
                                       _vp, ctypes.c_float, _vp, _c_int, _vp, _vp, _size, _vp]),
    "seqcomp_mqa_workspace_bytes": (_size, [_i64p, _c_i64]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libseqcomp.so once and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m kv_sequence_compression_amd.build` "
            "(or __graft_entry__.build()); the compressor has no non-HIP implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
