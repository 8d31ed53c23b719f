"""Argument checks of the Python binding, on the host: every check that
runs before the first device operation (dtype, shape, layout, device) turns
a wrong tensor into an exception.  The kernels take raw pointers, so without
these a host tensor, a short bias or a strided view would be read out of
place.  No GPU is needed: every call here raises before touching one."""

import numpy as np
import pytest
import torch

import kv_sequence_compression_amd as sc

T, D, C = 64, 64, 32


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _fused_ok():
    return dict(H=_t(T, D), Wt=_t(4 * C, D), Ba=_t(4, C, dtype=torch.float32), Bb=_t(4, C, dtype=torch.float32))


@pytest.mark.parametrize("change,err,match", [
    (dict(H=_t(T, D, dtype=torch.float16)), TypeError, "H: dtype"),
    (dict(H=_t(D, T).t()), ValueError, "H must be contiguous"),
    (dict(Wt=_t(4 * C, D + 64)), ValueError, "shape"),
    (dict(Wt=_t(4 * C + 1, D)), ValueError, "shape"),
    (dict(Wt=_t(4 * C, D, dtype=torch.float32)), TypeError, "Wt"),
    (dict(Ba=_t(8, C, dtype=torch.float32)), ValueError, "Ba must have shape"),
    (dict(Bb=_t(4, C)), TypeError, "Bb: dtype"),
    (dict(), ValueError, "must be on a GPU"),
])
def test_fused_csa_argument_checks(change, err, match):
    a = _fused_ok()
    a.update(change)
    with pytest.raises(err, match=match):
        sc.compress_fused("csa", a["H"], a["Wt"], a["Ba"], a["Bb"], 4, None, "bf16")
    with pytest.raises(err, match=match):
        sc.compress_fused_noalloc("csa", a["H"], a["Wt"], a["Ba"], a["Bb"], 4, None, "bf16")


def test_fused_hca_and_mode_checks():
    H, Wt, B = _t(256, D), _t(2 * C, D), _t(128, C, dtype=torch.float32)
    with pytest.raises(ValueError, match="Bb must be None"):
        sc.compress_fused("hca", H, Wt, B, B, 128)
    with pytest.raises(ValueError, match="B must have shape"):
        sc.compress_fused("hca", H, Wt, _t(4, C, dtype=torch.float32), None, 128)
    with pytest.raises(ValueError, match="mode"):
        sc.compress_fused("mla", H, Wt, B, None, 128)
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.compress_fused("hca", H, Wt, B, None, 128)


def test_project_argument_checks():
    H, Wt = _t(T, D), _t(96, D)
    with pytest.raises(ValueError, match="shape"):
        sc.project(H, _t(96, D + 64))
    with pytest.raises(ValueError, match="out must have shape"):
        sc.project(H, Wt, "f32", out=_t(T, 95, dtype=torch.float32))
    with pytest.raises(TypeError, match="out: dtype"):
        sc.project(H, Wt, "f32", out=_t(T, 96))
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.project(H, Wt, "f32", out=_t(T, 128, dtype=torch.float32)[:, :96])   # a strided view is allowed


def test_pool_argument_checks():
    Y = _t(T, 4 * C)
    Ca, Cb, Za, Zb = Y[:, :C], Y[:, C:2 * C], Y[:, 2 * C:3 * C], Y[:, 3 * C:]
    B = _t(4, C, dtype=torch.float32)
    with pytest.raises(ValueError, match="Cb must have shape"):
        sc.pool_csa(Ca, _t(T, C + 16), Za, Zb, B, B, 4)
    with pytest.raises(ValueError, match="row stride"):
        sc.pool_csa(Ca, _t(T, C), Za, Zb, B, B, 4)
    with pytest.raises(ValueError, match="unit channel stride"):
        sc.pool_csa(_t(C, T).t(), _t(C, T).t(), _t(C, T).t(), _t(C, T).t(), B, B, 4)
    with pytest.raises(ValueError, match="Ba must have shape"):
        sc.pool_csa(Ca, Cb, Za, Zb, _t(8, C, dtype=torch.float32), B, 8 // 2)
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.pool_csa(Ca, Cb, Za, Zb, B, B, 4)
    with pytest.raises(ValueError, match="B must have shape"):
        sc.pool_hca(Ca, Za, B, 128)
    with pytest.raises(TypeError, match="Z: dtype"):
        sc.pool_hca(Ca, _t(T, C, dtype=torch.float32), _t(128, C, dtype=torch.float32), 128)


def test_append_argument_checks():
    H, Wt, B = _t(4 * 8, D), _t(4 * C, D), _t(4, C, dtype=torch.float32)
    with pytest.raises(ValueError, match="whole blocks"):
        sc.csa_append(_t(30, D), Wt, B, B)
    with pytest.raises(ValueError, match="state must have shape"):
        sc.csa_append(H, Wt, B, B, _t(8, 3, C + 16, dtype=torch.float32))
    with pytest.raises(TypeError, match="state_out: dtype"):
        sc.csa_append(H, Wt, B, B, None, state_out=_t(8, 3, C))
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.csa_append(H, Wt, B, B)


def test_rope_store_argument_checks():
    ent = _t(16, 128, dtype=torch.float32)
    good = (_t(16, 64, dtype=torch.uint8), _t(16, dtype=torch.float32), _t(16, 64))
    with pytest.raises(ValueError, match="cache nope must have shape"):
        sc.rope_store(ent, 4, [0, 64], (_t(16, 63, dtype=torch.uint8), good[1], good[2]), 64)
    with pytest.raises(TypeError, match="cache rope: dtype"):
        sc.rope_store(ent, 4, [0, 64], (good[0], good[1], _t(16, 64, dtype=torch.float32)), 64)
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.rope_store(ent, 4, [0, 64], good, 64)


def test_indexer_and_mqa_argument_checks():
    q, w, keys = _t(8, 64, 128), _t(8, 64, dtype=torch.float32), _t(100, 128)
    with pytest.raises(TypeError, match="q: dtype"):
        sc.indexer_topk(q.float(), w, keys, 16)
    with pytest.raises(ValueError, match="w must have shape"):
        sc.indexer_topk(q, _t(8, 32, dtype=torch.float32), keys, 16)
    with pytest.raises(ValueError, match="keys must be"):
        sc.indexer_topk(q, w, _t(100, 64), 16)
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.indexer_topk(q, w, keys, 16)
    qa, kv = _t(4, 128, 512), _t(50, 512)
    with pytest.raises(ValueError, match="kv must be"):
        sc.shared_kv_mqa(qa, _t(50, 256))
    with pytest.raises(ValueError, match="k_sink must have shape"):
        sc.shared_kv_mqa(qa, kv, k_sink=_t(256))
    with pytest.raises(ValueError, match="must be on a GPU"):
        sc.shared_kv_mqa(qa, kv)


def test_offsets_may_not_pass_the_rows_given():
    sc._need_rows(np.array([0, 10, 20]), 20, "cu")
    sc._need_rows(np.array([0]), 0, "cu")
    with pytest.raises(ValueError, match="past the 19 rows"):
        sc._need_rows(np.array([0, 10, 20]), 19, "cu")
