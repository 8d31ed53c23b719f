"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects malformed arguments before any HIP call (so these run
without a GPU; no call here reaches a kernel launch)."""

import ctypes
import os
import re

import numpy as np
import pytest

from kv_sequence_compression_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seqcomp.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared():
    txt = open(HEADER, encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(seqcomp_\w+)\s*\(", txt)))


def _status_codes():
    txt = open(HEADER, encoding="utf-8").read()
    return {k: int(v) for k, v in re.findall(r"(SEQCOMP_E_\w+|SEQCOMP_OK)\s*=\s*(\d+)", txt)}


S = _status_codes()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.SIGNATURES), names
    for nm in names:
        assert hasattr(lib, nm)


def test_version_and_status_strings(lib):
    assert lib.seqcomp_version() == 10000
    for code in range(0, 12):
        assert lib.seqcomp_status_string(code)
    assert lib.seqcomp_status_string(S["SEQCOMP_E_ALIAS"]).decode().startswith("an output overlaps")


def _cu(*vals):
    return np.ascontiguousarray(np.array(vals, dtype=np.int64))


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def test_num_entries_and_workspace(lib):
    cu = _cu(0, 64, 100, 100, 107)
    assert lib.seqcomp_num_entries(_p(cu), 4, 4) == 16 + 9 + 0 + 1
    assert lib.seqcomp_num_entries(_p(cu), 4, 128) == 0
    assert lib.seqcomp_num_entries(_p(_cu(1, 5)), 1, 4) == -1
    assert lib.seqcomp_num_entries(_p(_cu(0, 5, 3)), 2, 4) == -1
    assert lib.seqcomp_num_entries(_p(cu), 4, 0) == -1
    # bf16 output: tile table only; fp8 adds fp32 staging; fused CSA adds halo triples
    one = _cu(0, 8192)
    tiles = 8192 // 256
    # CSA pooling: tiles of 4 entries (one per wave) at c = 512 -> 512 tiles of 16 rows
    assert lib.seqcomp_workspace_bytes(_lib.OP_POOL_CSA, 0, 4, 512, _p(one), 1, _lib.BF16) == 512 * 16
    # HCA pooling, m' = 128: one entry per tile (8 waves of 16 rows) -> 64 tiles
    assert lib.seqcomp_workspace_bytes(_lib.OP_POOL_HCA, 0, 128, 512, _p(one), 1, _lib.BF16) == 64 * 16
    # m' = 8: 8 entries per tile -> 128 tiles
    assert lib.seqcomp_workspace_bytes(_lib.OP_POOL_HCA, 0, 8, 512, _p(one), 1, _lib.BF16) == 128 * 16
    assert lib.seqcomp_workspace_bytes(_lib.OP_POOL_CSA, 0, 4, 512, _p(one), 1, _lib.FP8_E4M3) == 512 * 16 + 2048 * 512 * 4
    # narrower channels: 512 / c entries per wave (c = 128: 16 entries, 64 rows per tile)
    assert lib.seqcomp_workspace_bytes(_lib.OP_POOL_CSA, 0, 4, 128, _p(one), 1, _lib.BF16) == (8192 // 64) * 16
    assert lib.seqcomp_workspace_bytes(_lib.OP_FUSED, 0, 4, 512, _p(one), 1, _lib.BF16) == 512 + tiles * 6 * 512 * 4
    assert lib.seqcomp_workspace_bytes(_lib.OP_FUSED, 1, 128, 512, _p(_cu(0, 100)), 1, _lib.BF16) == 0
    assert lib.seqcomp_workspace_bytes(7, 0, 4, 512, _p(one), 1, _lib.BF16) == ctypes.c_size_t(-1).value


# Fake, 16-byte-aligned "device" addresses: validation never dereferences them.
A, B_, C_, D_ = 0x10000000, 0x20000000, 0x30000000, 0x40000000
BIAS, BIAS2, CU_DEV, OUT, SCALE, WS = 0x50000000, 0x50100000, 0x50200000, 0x60000000, 0x70000000, 0x80000000


def pool_csa(lib, **kw):
    a = dict(Ca=A, Cb=B_, Za=C_, Zb=D_, ld=512, in_dt=_lib.BF16, Ba=BIAS, Bb=BIAS2, m=4, c=512,
             cu=_cu(0, 8192), cu_dev=CU_DEV, out=OUT, out_dt=_lib.BF16, scale=0, ws=WS, ws_bytes=1 << 20)
    a.update(kw)
    cu = a["cu"]
    return lib.seqcomp_pool_csa(a["Ca"], a["Cb"], a["Za"], a["Zb"], a["ld"], a["in_dt"], a["Ba"], a["Bb"], a["m"],
                                a["c"], _p(cu), a["cu_dev"], cu.size - 1, a["out"], a["out_dt"], a["scale"], a["ws"],
                                a["ws_bytes"], None)


def fused(lib, **kw):
    a = dict(mode=_lib.MODE_CSA, m=4, H=A, d=7168, in_dt=_lib.BF16, Wt=B_, c=512, Ba=BIAS, Bb=BIAS2,
             cu=_cu(0, 8192), cu_dev=CU_DEV, out=OUT, out_dt=_lib.BF16, scale=0, ws=WS, ws_bytes=1 << 24)
    a.update(kw)
    cu = a["cu"]
    return lib.seqcomp_compress_fused(a["mode"], a["m"], a["H"], a["d"], a["in_dt"], a["Wt"], a["c"], a["Ba"],
                                      a["Bb"], _p(cu), a["cu_dev"], cu.size - 1, a["out"], a["out_dt"], a["scale"],
                                      a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(in_dt=7), "SEQCOMP_E_DTYPE"),
    (dict(in_dt=_lib.FP8_E4M3), "SEQCOMP_E_DTYPE"),
    (dict(out_dt=9), "SEQCOMP_E_DTYPE"),
    (dict(Ca=0), "SEQCOMP_E_NULL"),
    (dict(Bb=0), "SEQCOMP_E_NULL"),
    (dict(cu_dev=0), "SEQCOMP_E_NULL"),
    (dict(out=0), "SEQCOMP_E_NULL"),
    (dict(out_dt=_lib.FP8_E4M3, scale=0), "SEQCOMP_E_NULL"),
    (dict(Za=C_ + 2), "SEQCOMP_E_ALIGN"),
    (dict(ld=516), "SEQCOMP_E_ALIGN"),
    (dict(ld=256), "SEQCOMP_E_SHAPE"),
    (dict(ld=(1 << 32) + 8), "SEQCOMP_E_SHAPE"),             # row offsets of T rows would overflow
    (dict(cu=_cu(1, 8192)), "SEQCOMP_E_SEQLENS"),
    (dict(cu=_cu(0, 100, 50)), "SEQCOMP_E_SEQLENS"),
    (dict(m=0), "SEQCOMP_E_UNSUPPORTED"),
    (dict(m=17), "SEQCOMP_E_UNSUPPORTED"),
    (dict(c=24, ld=24), "SEQCOMP_E_UNSUPPORTED"),
    (dict(ws=0), "SEQCOMP_E_WORKSPACE"),
    (dict(ws_bytes=16), "SEQCOMP_E_WORKSPACE"),
    (dict(out=A + 4096), "SEQCOMP_E_ALIAS"),
    (dict(ws=BIAS), "SEQCOMP_E_ALIAS"),
    (dict(out=WS), "SEQCOMP_E_ALIAS"),
])
def test_pool_rejects_bad_arguments(lib, kw, code):
    assert pool_csa(lib, **kw) == S[code]


def test_zero_entries_return_ok_without_buffers(lib):
    """A batch with no complete block has zero entries: OK, nothing launched,
    so NULL buffers are accepted."""
    assert pool_csa(lib, cu=_cu(0, 3), Ca=0, Cb=0, Za=0, Zb=0, out=0, ws=0, ws_bytes=0, cu_dev=0) == S["SEQCOMP_OK"]
    assert fused(lib, cu=_cu(0, 100), mode=_lib.MODE_HCA, m=128, Bb=0, H=0, out=0, ws=0, ws_bytes=0) == S["SEQCOMP_OK"]


@pytest.mark.parametrize("kw,code", [
    (dict(mode=3), "SEQCOMP_E_UNSUPPORTED"),
    (dict(m=8), "SEQCOMP_E_UNSUPPORTED"),
    (dict(mode=_lib.MODE_HCA, m=4), "SEQCOMP_E_UNSUPPORTED"),
    (dict(mode=_lib.MODE_HCA, m=128), "SEQCOMP_E_SHAPE"),          # HCA takes no B^b
    (dict(d=7200), "SEQCOMP_E_UNSUPPORTED"),
    (dict(c=500), "SEQCOMP_E_UNSUPPORTED"),
    (dict(H=0), "SEQCOMP_E_NULL"),
    (dict(Wt=B_ + 8), "SEQCOMP_E_ALIGN"),
    (dict(ws_bytes=100), "SEQCOMP_E_WORKSPACE"),
    (dict(out=A), "SEQCOMP_E_ALIAS"),
    (dict(ws=B_ + 1024), "SEQCOMP_E_ALIAS"),
    (dict(cu=_cu(0, -4)), "SEQCOMP_E_SEQLENS"),
    (dict(cu=_cu(0, 1 << 31)), "SEQCOMP_E_SHAPE"),
])
def test_fused_rejects_bad_arguments(lib, kw, code):
    assert fused(lib, **kw) == S[code]


def test_project_rejects_bad_arguments(lib):
    f = lib.seqcomp_project
    assert f(A, 64, 64, _lib.BF16, B_, 128, OUT, 128, _lib.FP8_E4M3, None) == S["SEQCOMP_E_DTYPE"]
    assert f(A, 64, 60, _lib.BF16, B_, 128, OUT, 128, _lib.BF16, None) == S["SEQCOMP_E_UNSUPPORTED"]
    assert f(A, 64, 64, _lib.BF16, B_, 120, OUT, 120, _lib.BF16, None) == S["SEQCOMP_E_UNSUPPORTED"]
    assert f(A, 64, 64, _lib.BF16, B_, 128, OUT, 100, _lib.BF16, None) == S["SEQCOMP_E_SHAPE"]
    assert f(0, 64, 64, _lib.BF16, B_, 128, OUT, 128, _lib.BF16, None) == S["SEQCOMP_E_NULL"]
    assert f(A, 64, 64, _lib.BF16, B_, 128, A + 64, 128, _lib.BF16, None) == S["SEQCOMP_E_ALIAS"]
    assert f(A, 0, 64, _lib.BF16, B_, 128, 0, 128, _lib.BF16, None) == S["SEQCOMP_OK"]
    # a 256-row tile of H must stay addressable with 32-bit byte offsets
    assert f(A, 64, 1 << 22, _lib.F32, B_, 16, OUT, 16, _lib.F32, None) == S["SEQCOMP_E_UNSUPPORTED"]
    assert fused(lib, d=1 << 22, c=16, in_dt=_lib.F32) == S["SEQCOMP_E_UNSUPPORTED"]
    # ... and a 256-row tile of Y too
    assert f(A, 64, 64, _lib.BF16, B_, 16, OUT, 1 << 22, _lib.BF16, None) == S["SEQCOMP_E_UNSUPPORTED"]


STATE, STATE2 = 0x90000000, 0x98000000


def append(lib, **kw):
    a = dict(H=A, nb=100, d=7168, in_dt=_lib.BF16, Wt=B_, c=512, Ba=BIAS, Bb=BIAS2, st_in=STATE, st_out=STATE2,
             out=OUT, out_dt=_lib.BF16, scale=0, ws=WS, ws_bytes=1 << 27)
    a.update(kw)
    return lib.seqcomp_csa_append(a["H"], a["nb"], a["d"], a["in_dt"], a["Wt"], a["c"], a["Ba"], a["Bb"],
                                  a["st_in"], a["st_out"], a["out"], a["out_dt"], a["scale"], a["ws"], a["ws_bytes"],
                                  None)


def test_append_workspace(lib):
    f = lib.seqcomp_append_workspace_bytes
    part = 64 * 1024                                     # split-K partials of one 128 x 128 tile and split
    # 64 blocks, c = 512: 2 x 16 tiles of 128 x 128, K split 8 ways
    assert f(64, 512, _lib.BF16) == 32 * 8 * part
    # 100 blocks: 4 x 16 tiles, 4 ways; fp8 adds the fp32 staging of the entries
    assert f(100, 512, _lib.BF16) == 64 * 4 * part
    assert f(100, 512, _lib.FP8_E4M3) == 64 * 4 * part + 100 * 512 * 4
    # 1 or 2 blocks: one weight row per wave, no tiles and no partials (fp8
    # keeps its staging); 3 blocks: 16 tiles, 16 ways
    assert f(1, 512, _lib.BF16) == 0
    assert f(2, 512, _lib.BF16) == 0
    assert f(2, 512, _lib.FP8_E4M3) == 2 * 512 * 4
    assert f(3, 512, _lib.BF16) == 16 * 16 * part
    # c = 160 (5 channel tiles): 5 tiles, capped at 32 ways
    assert f(20, 160, _lib.BF16) == 5 * 32 * part
    # 400 blocks: 7 x 8 tiles of 256 x 256 are too few, 13 x 16 = 208 of 128 x 128 run unsplit
    assert f(400, 512, _lib.BF16) == 0
    # 1024 blocks: 16 x 8 = 128 tiles of 256 x 256, K split 2 ways (256 KiB per tile and split);
    # 4096 blocks: 512 tiles of 256 x 256, no split
    assert f(1024, 512, _lib.BF16) == 128 * 2 * 256 * 1024
    assert f(4096, 512, _lib.BF16) == 0
    assert f(4096, 512, _lib.FP8_E4M3) == 4096 * 512 * 4
    assert f(0, 512, _lib.FP8_E4M3) == 0
    assert f(-1, 512, _lib.BF16) == ctypes.c_size_t(-1).value
    assert f(1, 512, 9) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,code", [
    (dict(in_dt=_lib.FP8_E4M3), "SEQCOMP_E_DTYPE"),
    (dict(out_dt=5), "SEQCOMP_E_DTYPE"),
    (dict(nb=-1), "SEQCOMP_E_SHAPE"),
    (dict(nb=1 << 30), "SEQCOMP_E_SHAPE"),
    (dict(d=7200), "SEQCOMP_E_UNSUPPORTED"),
    (dict(c=100), "SEQCOMP_E_UNSUPPORTED"),
    (dict(d=1 << 22, c=16, in_dt=_lib.F32), "SEQCOMP_E_UNSUPPORTED"),
    (dict(H=0), "SEQCOMP_E_NULL"),
    (dict(st_in=0), "SEQCOMP_E_NULL"),
    (dict(st_out=0), "SEQCOMP_E_NULL"),
    (dict(out=0), "SEQCOMP_E_NULL"),
    (dict(out_dt=_lib.FP8_E4M3, scale=0, ws=WS, ws_bytes=1 << 20), "SEQCOMP_E_NULL"),
    (dict(out_dt=_lib.FP8_E4M3, scale=SCALE, ws_bytes=64 * 4 * 64 * 1024), "SEQCOMP_E_WORKSPACE"),   # no staging
    (dict(ws=0, ws_bytes=0), "SEQCOMP_E_WORKSPACE"),     # the split-K partials of a small batch
    (dict(st_in=STATE + 4), "SEQCOMP_E_ALIGN"),
    (dict(st_out=STATE + 16), "SEQCOMP_E_ALIAS"),          # partial overlap with the input state
    (dict(st_out=A + 4096), "SEQCOMP_E_ALIAS"),            # the new state over H
    (dict(out=STATE2 + 64), "SEQCOMP_E_ALIAS"),            # entries over the new state
    (dict(nb=0, H=0, out=0, st_in=0, st_out=0), "SEQCOMP_OK"),
])
def test_append_rejects_bad_arguments(lib, kw, code):
    assert append(lib, **kw) == S[code]


NOPE, SCL, ROPE, SLOTS, POS0 = 0xA0000000, 0xA8000000, 0xB0000000, 0xB8000000, 0xBC000000


def rope_store(lib, **kw):
    a = dict(ent=A, in_dt=_lib.F32, c=512, m=4, cu=_cu(0, 8192), cu_dev=CU_DEV, pos0=0, r=64, base=10000.0,
             slots=0, n_slots=2048, nope=NOPE, scale=SCL, rope=ROPE, ws=WS, ws_bytes=1 << 20)
    a.update(kw)
    cu = a["cu"]
    return lib.seqcomp_rope_store(a["ent"], a["in_dt"], a["c"], a["m"], _p(cu), a["cu_dev"], cu.size - 1, a["pos0"],
                                  a["r"], a["base"], a["slots"], a["n_slots"], a["nope"], a["scale"], a["rope"],
                                  a["ws"], a["ws_bytes"], None)


def test_rope_store_workspace(lib):
    f = lib.seqcomp_rope_store_workspace_bytes
    assert f(4, _p(_cu(0, 8192)), 1) == 512          # 32 tiles of 64 entries, 16 B each
    assert f(4, _p(_cu(0, 3)), 1) == 0
    assert f(0, _p(_cu(0, 8)), 1) == ctypes.c_size_t(-1).value
    assert f(4, _p(_cu(0, -1)), 1) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,code", [
    (dict(in_dt=_lib.FP8_E4M3), "SEQCOMP_E_DTYPE"),
    (dict(c=100), "SEQCOMP_E_UNSUPPORTED"),
    (dict(m=0), "SEQCOMP_E_UNSUPPORTED"),
    (dict(r=60), "SEQCOMP_E_UNSUPPORTED"),
    (dict(r=520), "SEQCOMP_E_UNSUPPORTED"),
    (dict(base=0.0), "SEQCOMP_E_SHAPE"),
    (dict(base=float("nan")), "SEQCOMP_E_SHAPE"),
    (dict(n_slots=100), "SEQCOMP_E_SHAPE"),                 # no slot map: one row per entry needed
    (dict(n_slots=(1 << 40) + 1), "SEQCOMP_E_SHAPE"),      # cache byte ranges would overflow
    (dict(cu=_cu(0, -4)), "SEQCOMP_E_SEQLENS"),
    (dict(ent=0), "SEQCOMP_E_NULL"),
    (dict(scale=0), "SEQCOMP_E_NULL"),
    (dict(rope=0), "SEQCOMP_E_NULL"),
    (dict(nope=NOPE + 8), "SEQCOMP_E_ALIGN"),
    (dict(ws_bytes=8), "SEQCOMP_E_WORKSPACE"),
    (dict(nope=A + 64), "SEQCOMP_E_ALIAS"),                 # cache over the entries
    (dict(slots=SLOTS, rope=SLOTS - 64), "SEQCOMP_E_ALIAS"),
    (dict(cu=_cu(0, 3), ent=0, nope=0, scale=0, rope=0), "SEQCOMP_OK"),
])
def test_rope_store_rejects_bad_arguments(lib, kw, code):
    assert rope_store(lib, **kw) == S[code]


CU_K_DEV = 0x50300000


def indexer(lib, **kw):
    a = dict(q=A, w=B_, keys=C_, H=64, D=128, in_dt=_lib.BF16, cu_q=_cu(0, 4096), cu_q_dev=CU_DEV,
             cu_k=_cu(0, 262144), cu_k_dev=CU_K_DEV, nv=D_, k=1024, idx=OUT, sc=SCALE, ws=WS, ws_bytes=1 << 20)
    a.update(kw)
    cq, ck = a["cu_q"], a["cu_k"]
    return lib.seqcomp_indexer_topk(a["q"], a["w"], a["keys"], a["H"], a["D"], a["in_dt"], _p(cq), a["cu_q_dev"],
                                    _p(ck), a["cu_k_dev"], cq.size - 1, a["nv"], a["k"], a["idx"], a["sc"], a["ws"],
                                    a["ws_bytes"], None)


def test_indexer_workspace(lib):
    f = lib.seqcomp_indexer_workspace_bytes
    assert f(_p(_cu(0, 4096)), 1) == 512 * 16          # 512 tiles of 8 queries
    assert f(_p(_cu(0, 9, 9, 10)), 3) == 256           # 3 tiles, rounded up to 256 bytes
    assert f(_p(_cu(0, 0)), 1) == 0
    assert f(_p(_cu(0, -1)), 1) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,code", [
    (dict(in_dt=_lib.F32), "SEQCOMP_E_DTYPE"),
    (dict(H=32), "SEQCOMP_E_UNSUPPORTED"),
    (dict(D=64), "SEQCOMP_E_UNSUPPORTED"),
    (dict(k=0), "SEQCOMP_E_UNSUPPORTED"),
    (dict(k=1025), "SEQCOMP_E_UNSUPPORTED"),
    (dict(cu_k=_cu(0, 1 << 23)), "SEQCOMP_E_UNSUPPORTED"),     # key offsets must stay below 2^31 bytes
    (dict(cu_q=_cu(0, 5, 4), cu_k=_cu(0, 5, 9)), "SEQCOMP_E_SEQLENS"),
    (dict(cu_k=_cu(1, 9)), "SEQCOMP_E_SEQLENS"),
    (dict(q=0), "SEQCOMP_E_NULL"),
    (dict(keys=0), "SEQCOMP_E_NULL"),
    (dict(idx=0), "SEQCOMP_E_NULL"),
    (dict(cu_k_dev=0), "SEQCOMP_E_NULL"),
    (dict(w=B_ + 4), "SEQCOMP_E_ALIGN"),
    (dict(nv=D_ + 2), "SEQCOMP_E_ALIGN"),
    (dict(ws_bytes=16), "SEQCOMP_E_WORKSPACE"),
    (dict(idx=A + 4096), "SEQCOMP_E_ALIAS"),                     # selection over the queries
    (dict(sc=OUT + 4096), "SEQCOMP_E_ALIAS"),                    # scores over the selection
    (dict(ws=C_ + 256), "SEQCOMP_E_ALIAS"),                      # workspace over the keys
    (dict(nv=0, sc=0, idx=0), "SEQCOMP_E_NULL"),                 # n_valid and scores are optional, idx is not
])
def test_indexer_rejects_bad_arguments(lib, kw, code):
    assert indexer(lib, **kw) == S[code]


def test_indexer_empty_calls_launch_nothing(lib):
    # no queries: OK before any pointer is looked at; keys may be absent when there are none
    assert indexer(lib, cu_q=_cu(0, 0), q=0, w=0, idx=0, sc=0, ws=0, ws_bytes=0) == S["SEQCOMP_OK"]
    assert indexer(lib, cu_k=_cu(0, 0), keys=0, cu_q=_cu(0, 0), q=0, w=0, idx=0, ws=0) == S["SEQCOMP_OK"]


KSINK, VSINK, LSE = 0x50400000, 0x50500000, 0x90000000


def mqa(lib, **kw):
    a = dict(q=A, kv=C_, H=128, D=512, in_dt=_lib.BF16, cu_q=_cu(0, 4096), cu_q_dev=CU_DEV, cu_k=_cu(0, 8192),
             cu_k_dev=CU_K_DEV, nv=D_, ks=KSINK, vs=VSINK, scale=0.044, out=OUT, out_dt=_lib.BF16, lse=LSE, ws=WS,
             ws_bytes=1 << 20)
    a.update(kw)
    cq, ck = a["cu_q"], a["cu_k"]
    return lib.seqcomp_shared_kv_mqa(a["q"], a["kv"], a["H"], a["D"], a["in_dt"], _p(cq), a["cu_q_dev"], _p(ck),
                                     a["cu_k_dev"], cq.size - 1, a["nv"], a["ks"], a["vs"], a["scale"], a["out"],
                                     a["out_dt"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_mqa_workspace(lib):
    f = lib.seqcomp_mqa_workspace_bytes
    assert f(_p(_cu(0, 4096)), 1) == 4096 * 16         # one tile record per query
    assert f(_p(_cu(0, 3, 3, 5)), 3) == 256
    assert f(_p(_cu(0, 0)), 1) == 0
    assert f(_p(_cu(2, 5)), 1) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,code", [
    (dict(in_dt=_lib.F32), "SEQCOMP_E_DTYPE"),
    (dict(out_dt=_lib.FP8_E4M3), "SEQCOMP_E_DTYPE"),
    (dict(H=64), "SEQCOMP_E_UNSUPPORTED"),
    (dict(D=128), "SEQCOMP_E_UNSUPPORTED"),
    (dict(scale=float("nan")), "SEQCOMP_E_SHAPE"),
    (dict(scale=float("inf")), "SEQCOMP_E_SHAPE"),
    (dict(cu_k=_cu(0, 1 << 21)), "SEQCOMP_E_UNSUPPORTED"),     # entry offsets must stay below 2^31 bytes
    (dict(cu_q=_cu(0, 5, 4), cu_k=_cu(0, 5, 9)), "SEQCOMP_E_SEQLENS"),
    (dict(q=0), "SEQCOMP_E_NULL"),
    (dict(kv=0), "SEQCOMP_E_NULL"),
    (dict(out=0), "SEQCOMP_E_NULL"),
    (dict(ks=0), "SEQCOMP_E_NULL"),                             # a sink value needs a sink key
    (dict(vs=VSINK + 4), "SEQCOMP_E_ALIGN"),
    (dict(nv=D_ + 2), "SEQCOMP_E_ALIGN"),
    (dict(ws_bytes=64), "SEQCOMP_E_WORKSPACE"),
    (dict(out=A + 4096), "SEQCOMP_E_ALIAS"),                     # output over the queries
    (dict(lse=OUT + 4096), "SEQCOMP_E_ALIAS"),                   # log-sum-exp over the output
    (dict(ws=C_ + 1024), "SEQCOMP_E_ALIAS"),                     # workspace over the entries
])
def test_mqa_rejects_bad_arguments(lib, kw, code):
    assert mqa(lib, **kw) == S[code]


def test_mqa_empty_calls_launch_nothing(lib):
    assert mqa(lib, cu_q=_cu(0, 0), q=0, out=0, lse=0, ws=0, ws_bytes=0) == S["SEQCOMP_OK"]


def test_hip_failure_maps_to_e_hip(lib):
    """A well-formed call passes validation and reaches its first HIP call;
    on a host with no GPU that call fails and the entry point returns
    SEQCOMP_E_HIP (the fused call at a kernel launch, the allocation-free one
    when it looks up the device's scratch)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("needs a host without a GPU: with one these calls would launch on fake addresses")
    assert fused(lib) == S["SEQCOMP_E_HIP"]
    cu = _cu(0, 8192)
    assert lib.seqcomp_compress_fused_noalloc(_lib.MODE_CSA, 4, A, 7168, _lib.BF16, B_, 512, BIAS, BIAS2, _p(cu), CU_DEV,
                                              1, OUT, _lib.BF16, 0, None) == S["SEQCOMP_E_HIP"]


def test_noalloc_rejects_beyond_its_scratch(lib):
    """The allocation-free call rejects, before any HIP call, a batch whose
    workspace would exceed its 64 MiB (fp8 staging of 200704 tokens at
    c = 512), and validates its other arguments like the workspace form."""
    cu = _cu(0, 200704)
    f = lib.seqcomp_compress_fused_noalloc
    assert f(_lib.MODE_CSA, 4, A, 64, _lib.BF16, B_, 512, BIAS, BIAS2, _p(cu), CU_DEV, 1, OUT, _lib.FP8_E4M3, SCALE,
             None) == S["SEQCOMP_E_SCRATCH"]
    one = _cu(0, 8192)
    assert f(_lib.MODE_CSA, 3, A, 7168, _lib.BF16, B_, 512, BIAS, BIAS2, _p(one), CU_DEV, 1, OUT, _lib.BF16, 0,
             None) == S["SEQCOMP_E_UNSUPPORTED"]
    assert f(_lib.MODE_CSA, 4, 0, 7168, _lib.BF16, B_, 512, BIAS, BIAS2, _p(one), CU_DEV, 1, OUT, _lib.BF16, 0,
             None) == S["SEQCOMP_E_NULL"]
    assert f(_lib.MODE_CSA, 4, A, 7168, _lib.BF16, B_, 512, BIAS, BIAS2, _p(one), CU_DEV, 1, A + 4096, _lib.BF16, 0,
             None) == S["SEQCOMP_E_ALIAS"]
