"""seqcomp: the token-level KV sequence compressor (CSA / HCA) on MI355X.

Python face of the C ABI in ``include/seqcomp.h``.  These wrappers only
marshal torch tensors into pointers, sizes and the current HIP stream, and
allocate the outputs and the workspace with torch; every step of the
computation runs in the HIP kernels of ``libseqcomp.so``.

Functions (each returns torch tensors on the inputs' device):

* ``project(H, Wt, out_dtype, out=None)``               -> Y = H Wt^T
* ``pool_csa(Ca, Cb, Za, Zb, Ba, Bb, m, cu_seqlens, out_dtype)`` -> (entries, scale|None)
* ``pool_hca(C, Z, B, m, cu_seqlens, out_dtype)``       -> (entries, scale|None)
* ``compress_fused(mode, H, Wt, Ba, Bb, m, cu_seqlens, out_dtype)`` -> (entries, scale|None)
* ``csa_append(H, Wt, Ba, Bb, state, out_dtype, state_out)`` -> (entries, scale|None, state)
* ``csa_empty_state(nb, c, device)``                   -> the state of sequences with no block yet
* ``rope_store(entries, m, cu_seqlens, cache, ...)``     partial RoPE + bf16/fp8 store into a cache
* ``indexer_topk(q, w, keys, k, ...)``                   -> (indices, scores|None) of the k best keys
* ``shared_kv_mqa(q, kv, ...)``                          -> (out, lse|None), dense attention with a sink

``out_dtype`` is one of "f32", "bf16", "fp8" (OCP E4M3FN codes stored as
uint8 with one fp32 scale per entry).

Every tensor argument is checked before the call: its dtype, its shape (the
sizes the kernels will read), a dense layout, and the device of the first
input.  The kernels take raw pointers, so a host tensor, a short buffer or a
strided view would otherwise be read out of place.  Sequence offsets may not
reach past the rows given.
"""

from __future__ import annotations

import collections
import ctypes

import numpy as np
import torch

from . import _lib

__all__ = ["SeqcompError", "project", "pool_csa", "pool_hca", "compress_fused", "compress_fused_noalloc",
           "csa_append", "csa_empty_state", "rope_store", "rope_cache", "indexer_topk", "shared_kv_mqa",
           "num_entries", "workspace_bytes", "version", "lib"]

_DT_CODE = {"f32": _lib.F32, "bf16": _lib.BF16, "fp8": _lib.FP8_E4M3}
_TORCH_IN = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}
_TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


class SeqcompError(RuntimeError):
    """A seqcomp call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().seqcomp_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def lib():
    return _lib.load()


def version() -> int:
    return lib().seqcomp_version()


def _check(status: int, where: str):
    if status != _lib.OK:
        raise SeqcompError(status, where)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name: str, dtypes, shape=None, dense: bool = True):
    """Check one tensor argument's dtype, shape and layout (its device is
    checked with the others' by _one_gpu)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not supported ({', '.join(str(d) for d in dtypes)})")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, not {tuple(t.shape)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _one_gpu(**tensors) -> torch.device:
    """All given tensors (None entries skipped) on one GPU; returns it."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU, not {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other inputs on {dev}")
    return dev


def _need_rows(host: np.ndarray, rows: int, name: str):
    """Offsets must reach no further than the rows the caller passed."""
    if host.size >= 1 and host[-1] > rows:
        raise ValueError(f"{name} reaches row {int(host[-1])}, past the {rows} rows given")


_IN = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)


def _in_code(t: torch.Tensor) -> int:
    if t.dtype not in _TORCH_IN:
        raise TypeError(f"input dtype {t.dtype} not supported (float32 or bfloat16)")
    return _TORCH_IN[t.dtype]


_DEV_COPIES = collections.OrderedDict()   # (device, stream, dtype, bytes) -> read-only device tensor
_DEV_COPIES_MAX = 64
_DEV_COPIES_HELD = {}   # copies that a captured graph reads: kept, whatever the cache evicts
_DEV_COPY_MAX_BYTES = 1 << 16


def _to_device(a, dtype, device):
    """`a` on `device` as a contiguous tensor of `dtype`, never written by the
    library.  Small host arrays (sequence offsets, visible counts) are kept
    by content, so a call that repeats a batch layout copies nothing; others
    go through a freshly pinned buffer and an asynchronous copy on the
    current stream.  A copy from pageable memory would make the host wait for
    the stream to drain, leaving the GPU idle between back-to-back calls."""
    if isinstance(a, torch.Tensor) and a.device.type != "cpu":
        return a.to(device=device, dtype=dtype).contiguous()
    t = torch.as_tensor(np.ascontiguousarray(np.asarray(a)), dtype=dtype).contiguous()
    key = None
    if t.numel() * t.element_size() <= _DEV_COPY_MAX_BYTES:
        # the stream is part of the key: the copy was ordered on it
        key = (str(torch.device(device)), torch.cuda.current_stream(device).cuda_stream, dtype, t.numpy().tobytes())
        hit = _DEV_COPIES.get(key)
        if hit is not None:
            _DEV_COPIES.move_to_end(key)
            if torch.cuda.is_current_stream_capturing():
                # the graph keeps this address for every replay: freeing the
                # copy on eviction would let the allocator hand it out again
                _DEV_COPIES_HELD[key] = hit
            return hit
    if torch.cuda.is_current_stream_capturing():
        # a copy captured into a graph would re-read a temporary pinned
        # buffer on every replay
        raise RuntimeError("host metadata (sequence offsets, visible counts) cannot be copied to the device during "
                           "graph capture: make the same call once on the capturing stream before capturing, so "
                           "that its device copy is kept")
    d = t.pin_memory().to(device, non_blocking=True)
    if key is not None:
        _DEV_COPIES[key] = d
        if len(_DEV_COPIES) > _DEV_COPIES_MAX:
            _DEV_COPIES.popitem(last=False)
    return d


def _cu_arrays(cu_seqlens, device):
    """Host int64 array (kept alive by the caller) and its device copy."""
    if isinstance(cu_seqlens, torch.Tensor):
        host = cu_seqlens.detach().to("cpu", torch.int64).numpy()
    else:
        host = np.asarray(cu_seqlens, dtype=np.int64)
    host = np.ascontiguousarray(host, dtype=np.int64)
    return host, _to_device(host, torch.int64, device)


def _i64p(host: np.ndarray):
    return host.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def num_entries(cu_seqlens, m: int) -> int:
    host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = lib().seqcomp_num_entries(_i64p(host), host.size - 1, int(m))
    if n < 0:
        raise ValueError("malformed cu_seqlens or m")
    return int(n)


def workspace_bytes(op: int, mode: int, m: int, c: int, cu_seqlens, out_dtype: str) -> int:
    host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = lib().seqcomp_workspace_bytes(op, mode, int(m), int(c), _i64p(host), host.size - 1, _DT_CODE[out_dtype])
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("malformed workspace query")
    return int(n)


def _alloc_out(E: int, c: int, out_dtype: str, device):
    out = torch.empty((E, c), dtype=_TORCH_OUT[out_dtype], device=device)
    scale = torch.empty((E,), dtype=torch.float32, device=device) if out_dtype == "fp8" else None
    return out, scale


def _alloc_ws(nbytes: int, device):
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def project(H: torch.Tensor, Wt: torch.Tensor, out_dtype: str = "bf16", out: torch.Tensor = None) -> torch.Tensor:
    """Y[T x n_out] = H[T x d] Wt[n_out x d]^T (eq. attn-seqcomp-csa-proj, all streams at once).

    `out`, if given, is a [T x n_out] view with unit column stride and any row
    stride >= n_out (e.g. the left columns of a wider buffer); it is written
    in place and returned."""
    _need(H, "H", _IN)
    if H.dim() != 2:
        raise ValueError("H must be [T x d]")
    T, d = H.shape
    n_out = Wt.shape[0] if isinstance(Wt, torch.Tensor) and Wt.dim() == 2 else -1
    _need(Wt, "Wt", (H.dtype,), (n_out, d))
    if out is not None:
        _need(out, "out", (_TORCH_OUT[out_dtype],), (T, n_out), dense=False)
    _one_gpu(H=H, Wt=Wt, out=out)
    if out is None:
        Y = torch.empty((T, n_out), dtype=_TORCH_OUT[out_dtype], device=H.device)
    else:
        if out.shape != (T, n_out) or out.stride(1) != 1 or out.dtype != _TORCH_OUT[out_dtype]:
            raise ValueError(f"out must be a [{T} x {n_out}] {_TORCH_OUT[out_dtype]} view with unit column stride")
        Y = out
    _check(lib().seqcomp_project(_ptr(H), T, d, _in_code(H), _ptr(Wt), n_out, _ptr(Y), Y.stride(0),
                                 _DT_CODE[out_dtype], _stream(H.device)), "seqcomp_project")
    return Y


def _pool_args(x, name: str, like=None):
    _need(x, name, _IN if like is None else (like.dtype,), None if like is None else like.shape, dense=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name}: pooling streams must be 2-D with unit channel stride")
    return x.stride(0)


def pool_csa(Ca, Cb, Za, Zb, Ba, Bb, m: int, cu_seqlens=None, out_dtype: str = "bf16"):
    """CSA pooling of materialised streams; returns (entries [E x c], scale [E] or None)."""
    ld = _pool_args(Ca, "Ca")
    if any(_pool_args(x, n, Ca) != ld for x, n in ((Cb, "Cb"), (Za, "Za"), (Zb, "Zb"))):
        raise ValueError("the four streams must share one row stride")
    c = Ca.shape[1]
    _need(Ba, "Ba", _F32, (m, c))
    _need(Bb, "Bb", _F32, (m, c))
    dev = _one_gpu(Ca=Ca, Cb=Cb, Za=Za, Zb=Zb, Ba=Ba, Bb=Bb)
    host, cu_dev = _cu_arrays([0, Ca.shape[0]] if cu_seqlens is None else cu_seqlens, dev)
    _need_rows(host, Ca.shape[0], "cu_seqlens")
    E = num_entries(host, m)
    out, scale = _alloc_out(E, c, out_dtype, dev)
    ws_n = workspace_bytes(_lib.OP_POOL_CSA, 0, m, c, host, out_dtype)
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_pool_csa(_ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), ld, _in_code(Ca), _ptr(Ba), _ptr(Bb),
                                  int(m), c, _i64p(host), _ptr(cu_dev), host.size - 1, _ptr(out),
                                  _DT_CODE[out_dtype], _ptr(scale), _ptr(ws), ws_n, _stream(dev)),
           "seqcomp_pool_csa")
    return out, scale


def pool_hca(C, Z, B, m: int, cu_seqlens=None, out_dtype: str = "bf16"):
    """HCA pooling of materialised streams; returns (entries [E x c], scale [E] or None)."""
    ld = _pool_args(C, "C")
    if _pool_args(Z, "Z", C) != ld:
        raise ValueError("C and Z must share one row stride")
    c = C.shape[1]
    _need(B, "B", _F32, (m, c))
    dev = _one_gpu(C=C, Z=Z, B=B)
    host, cu_dev = _cu_arrays([0, C.shape[0]] if cu_seqlens is None else cu_seqlens, dev)
    _need_rows(host, C.shape[0], "cu_seqlens")
    E = num_entries(host, m)
    out, scale = _alloc_out(E, c, out_dtype, dev)
    ws_n = workspace_bytes(_lib.OP_POOL_HCA, 0, m, c, host, out_dtype)
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_pool_hca(_ptr(C), _ptr(Z), ld, _in_code(C), _ptr(B), int(m), c, _i64p(host),
                                  _ptr(cu_dev), host.size - 1, _ptr(out), _DT_CODE[out_dtype], _ptr(scale),
                                  _ptr(ws), ws_n, _stream(dev)), "seqcomp_pool_hca")
    return out, scale


def _fused_args(mode: str, H, Wt, Ba, Bb, m: int):
    """Checks shared by both fused entry points; returns (mode code, T, d, c)."""
    if mode not in ("csa", "hca"):
        raise ValueError('mode must be "csa" or "hca"')
    _need(H, "H", _IN)
    if H.dim() != 2:
        raise ValueError("H must be [T x d]")
    T, d = H.shape
    S = 4 if mode == "csa" else 2
    c = Wt.shape[0] // S if isinstance(Wt, torch.Tensor) and Wt.dim() == 2 else 0
    _need(Wt, f"Wt ([{S}*c x d])", (H.dtype,), (S * c, d))
    if mode == "csa":
        _need(Ba, "Ba", _F32, (m, c))
        _need(Bb, "Bb", _F32, (m, c))
    else:
        _need(Ba, "B", _F32, (m, c))
        if Bb is not None:
            raise ValueError("HCA takes one bias: Bb must be None")
    _one_gpu(H=H, Wt=Wt, Ba=Ba, Bb=Bb)
    return {"csa": _lib.MODE_CSA, "hca": _lib.MODE_HCA}[mode], T, d, c


def compress_fused(mode: str, H, Wt, Ba, Bb, m: int, cu_seqlens=None, out_dtype: str = "bf16"):
    """Fused projection + pooling (mode "csa" with m=4, or "hca" with m=128)."""
    mcode, T, d, c = _fused_args(mode, H, Wt, Ba, Bb, m)
    dev = H.device
    host, cu_dev = _cu_arrays([0, T] if cu_seqlens is None else cu_seqlens, dev)
    _need_rows(host, T, "cu_seqlens")
    E = num_entries(host, m)
    out, scale = _alloc_out(E, c, out_dtype, dev)
    ws_n = workspace_bytes(_lib.OP_FUSED, mcode, m, c, host, out_dtype)
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_compress_fused(mcode, int(m), _ptr(H), d, _in_code(H), _ptr(Wt), c, _ptr(Ba),
                                        _ptr(Bb), _i64p(host), _ptr(cu_dev), host.size - 1, _ptr(out),
                                        _DT_CODE[out_dtype], _ptr(scale), _ptr(ws), ws_n, _stream(dev)),
           "seqcomp_compress_fused")
    return out, scale


def compress_fused_noalloc(mode: str, H, Wt, Ba, Bb, m: int, cu_seqlens=None, out_dtype: str = "bf16", out=None,
                           out_scale=None):
    """compress_fused through the allocation-free entry point: the library
    uses its own per-device scratch (64 MiB) instead of a workspace.  `out`
    (and `out_scale` for fp8) may be passed pre-allocated; otherwise they are
    allocated here, outside the library call."""
    mcode, T, d, c = _fused_args(mode, H, Wt, Ba, Bb, m)
    dev = H.device
    host, cu_dev = _cu_arrays([0, T] if cu_seqlens is None else cu_seqlens, dev)
    _need_rows(host, T, "cu_seqlens")
    E = num_entries(host, m)
    if out is None:
        out, out_scale = _alloc_out(E, c, out_dtype, dev)
    else:
        _need(out, "out", (_TORCH_OUT[out_dtype],), (E, c))
        if out_dtype == "fp8":
            _need(out_scale, "out_scale", _F32, (E,))
        _one_gpu(H=H, out=out, out_scale=out_scale if out_dtype == "fp8" else None)
    _check(lib().seqcomp_compress_fused_noalloc(mcode, int(m), _ptr(H), d, _in_code(H), _ptr(Wt), c, _ptr(Ba),
                                                _ptr(Bb), _i64p(host), _ptr(cu_dev), host.size - 1, _ptr(out),
                                                _DT_CODE[out_dtype], _ptr(out_scale), _stream(dev)),
           "seqcomp_compress_fused_noalloc")
    return out, out_scale


def csa_empty_state(nb: int, c: int, device) -> torch.Tensor:
    """State [nb, 3, c] fp32 of sequences that have no block yet (M = -inf, S = A = 0)."""
    st = torch.zeros((nb, 3, c), dtype=torch.float32, device=device)
    st[:, 0, :] = float("-inf")
    return st


def csa_append(H, Wt, Ba, Bb, state=None, out_dtype: str = "bf16", state_out=None):
    """CSA decode append: H [4 nb x d] holds one newly completed block of 4
    tokens per sequence; returns (entries [nb x c], scale [nb] or None,
    state_out [nb, 3, c]).  `state` is what the previous call returned for
    these sequences (None: every sequence starts here).  Passing
    state_out=state updates the state in place."""
    _need(H, "H", _IN)
    if H.dim() != 2:
        raise ValueError("H must be [4 nb x d]")
    T, d = H.shape
    if T % 4 != 0:
        raise ValueError("H must hold whole blocks of 4 rows")
    nb = T // 4
    c = Wt.shape[0] // 4 if isinstance(Wt, torch.Tensor) and Wt.dim() == 2 else 0
    _need(Wt, "Wt ([4*c x d])", (H.dtype,), (4 * c, d))
    _need(Ba, "Ba", _F32, (4, c))
    _need(Bb, "Bb", _F32, (4, c))
    if state is not None:
        _need(state, "state", _F32, (nb, 3, c))
    if state_out is not None:
        _need(state_out, "state_out", _F32, (nb, 3, c))
    dev = _one_gpu(H=H, Wt=Wt, Ba=Ba, Bb=Bb, state=state, state_out=state_out)
    if state is None:
        state = csa_empty_state(nb, c, dev)
    if state_out is None:
        state_out = torch.empty_like(state)
    out, scale = _alloc_out(nb, c, out_dtype, dev)
    ws_n = lib().seqcomp_append_workspace_bytes(nb, c, _DT_CODE[out_dtype])
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_csa_append(_ptr(H), nb, d, _in_code(H), _ptr(Wt), c, _ptr(Ba), _ptr(Bb), _ptr(state),
                                    _ptr(state_out), _ptr(out), _DT_CODE[out_dtype], _ptr(scale), _ptr(ws), ws_n,
                                    _stream(dev)), "seqcomp_csa_append")
    return out, scale, state_out


def rope_cache(n_slots: int, c: int, rope_dims: int, device):
    """An empty mixed-precision entry cache: (nope [n_slots, c - r] uint8 E4M3
    codes, scale [n_slots] float32, rope [n_slots, r] bfloat16)."""
    return (torch.zeros((n_slots, c - rope_dims), dtype=torch.uint8, device=device),
            torch.zeros((n_slots,), dtype=torch.float32, device=device),
            torch.zeros((n_slots, rope_dims), dtype=torch.bfloat16, device=device))


def rope_store(entries, m: int, cu_seqlens, cache, rope_dims: int = 64, rope_base: float = 10000.0,
               pos0=None, slots=None):
    """Partial RoPE on the last `rope_dims` dimensions of every packed entry
    (position: its block centre plus pos0 of its sequence) and the store into
    `cache` = (nope, scale, rope) at rows `slots` (default: row e for entry e)."""
    _need(entries, "entries", _IN)
    if entries.dim() != 2:
        raise ValueError("entries must be [E x c]")
    E, c = entries.shape
    nope, scale, rope = cache
    _need(scale, "cache scale", _F32)
    n_slots = scale.shape[0] if scale.dim() == 1 else -1
    _need(nope, "cache nope", (torch.uint8,), (n_slots, c - rope_dims))
    _need(rope, "cache rope", _BF16, (n_slots, rope_dims))
    dev = _one_gpu(entries=entries, nope=nope, scale=scale, rope=rope)
    host, cu_dev = _cu_arrays(cu_seqlens, dev)
    if num_entries(host, m) != E:
        raise ValueError(f"cu_seqlens and m give {num_entries(host, m)} entries, entries holds {E}")
    p0 = None if pos0 is None else _to_device(pos0, torch.int64, dev)
    sl = None if slots is None else _to_device(slots, torch.int64, dev)
    if p0 is not None and p0.numel() != host.size - 1:
        raise ValueError("pos0 must hold one position per sequence")
    if sl is not None and sl.numel() != E:
        raise ValueError("slots must hold one cache row per entry")
    ws_n = lib().seqcomp_rope_store_workspace_bytes(int(m), _i64p(host), host.size - 1)
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_rope_store(_ptr(entries), _in_code(entries), c, int(m), _i64p(host), _ptr(cu_dev),
                                    host.size - 1, _ptr(p0), int(rope_dims), float(rope_base), _ptr(sl), n_slots,
                                    _ptr(nope), _ptr(scale), _ptr(rope), _ptr(ws), ws_n, _stream(dev)),
           "seqcomp_rope_store")
    return cache


def indexer_topk(q, w, keys, k: int, cu_q=None, cu_k=None, n_valid=None, with_scores: bool = True):
    """Lightning-indexer selection: for every query t the k keys s of its
    sequence with the largest I[t, s] = sum_h w[t, h] ReLU(q[t, h] . keys[s]),
    ties to the smaller index, listed by increasing key index (-1 past the
    visible keys).  q [T x 64 x 128] bf16, w [T x 64] fp32, keys [N x 128]
    bf16; cu_q / cu_k pack queries and keys by sequence (default: one
    sequence); n_valid [T] int32: keys visible to each query (default: all).
    Returns (idx int32 [T x k], scores fp32 [T x k] or None)."""
    _need(q, "q", _BF16)
    if q.dim() != 3:
        raise ValueError("q must be [T x H x D]")
    T, Hh, D = q.shape
    _need(w, "w", _F32, (T, Hh))
    _need(keys, "keys", _BF16)
    if keys.dim() != 2 or keys.shape[1] != D:
        raise ValueError("keys must be [N x D]")
    N = keys.shape[0]
    dev = _one_gpu(q=q, w=w, keys=keys)
    hq, cq = _cu_arrays([0, T] if cu_q is None else cu_q, dev)
    hk, ck = _cu_arrays([0, N] if cu_k is None else cu_k, dev)
    if hq.size != hk.size:
        raise ValueError("cu_q and cu_k must describe the same number of sequences")
    _need_rows(hq, T, "cu_q")
    _need_rows(hk, N, "cu_k")
    nv = None if n_valid is None else _to_device(n_valid, torch.int32, dev)
    if nv is not None and nv.numel() < (int(hq[-1]) if hq.size else 0):
        raise ValueError("n_valid must hold one count per query")
    idx = torch.empty((T, int(k)), dtype=torch.int32, device=dev)
    sc = torch.empty((T, int(k)), dtype=torch.float32, device=dev) if with_scores else None
    ws_n = lib().seqcomp_indexer_workspace_bytes(_i64p(hq), hq.size - 1)
    if ws_n == ctypes.c_size_t(-1).value:
        raise ValueError("malformed cu_q")
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_indexer_topk(_ptr(q), _ptr(w), _ptr(keys), q.shape[1], q.shape[2], _in_code(q),
                                      _i64p(hq), _ptr(cq), _i64p(hk), _ptr(ck), hq.size - 1, _ptr(nv), int(k),
                                      _ptr(idx), _ptr(sc), _ptr(ws), ws_n, _stream(dev)),
           "seqcomp_indexer_topk")
    return idx, sc


def shared_kv_mqa(q, kv, cu_q=None, cu_k=None, n_valid=None, k_sink=None, v_sink=None, scale=None,
                  out_dtype: str = "bf16", with_lse: bool = False):
    """Dense shared-KV multi-query attention with an attention sink:
    out[t, h] = softmax(scale * q[t, h] . [k_sink, e_1..e_n]) . [v_sink, e_1..e_n]
    over the entries e of t's sequence that t sees.  q [T x 128 x 512] bf16,
    kv [N x 512] bf16 (entries are keys and values); cu_q / cu_k pack them by
    sequence (default: one sequence); n_valid [T] int32 (default: all);
    k_sink / v_sink [512] bf16 or None; scale defaults to 1/sqrt(512).
    Returns (out [T x 128 x 512] of out_dtype, lse [T x 128] fp32 or None)."""
    _need(q, "q", _BF16)
    if q.dim() != 3:
        raise ValueError("q must be [T x H x D]")
    T, _, D = q.shape
    _need(kv, "kv", _BF16)
    if kv.dim() != 2 or kv.shape[1] != D:
        raise ValueError("kv must be [N x D]")
    N = kv.shape[0]
    if k_sink is not None:
        _need(k_sink, "k_sink", _BF16, (D,))
    if v_sink is not None:
        _need(v_sink, "v_sink", _BF16, (D,))
    dev = _one_gpu(q=q, kv=kv, k_sink=k_sink, v_sink=v_sink)
    hq, cq = _cu_arrays([0, T] if cu_q is None else cu_q, dev)
    hk, ck = _cu_arrays([0, N] if cu_k is None else cu_k, dev)
    if hq.size != hk.size:
        raise ValueError("cu_q and cu_k must describe the same number of sequences")
    _need_rows(hq, T, "cu_q")
    _need_rows(hk, N, "cu_k")
    nv = None if n_valid is None else _to_device(n_valid, torch.int32, dev)
    if nv is not None and nv.numel() < (int(hq[-1]) if hq.size else 0):
        raise ValueError("n_valid must hold one count per query")
    sc_ = float(scale) if scale is not None else 1.0 / float(np.sqrt(q.shape[2]))
    out = torch.empty(tuple(q.shape), dtype=_TORCH_OUT[out_dtype], device=dev)
    lse = torch.empty((T, q.shape[1]), dtype=torch.float32, device=dev) if with_lse else None
    ws_n = lib().seqcomp_mqa_workspace_bytes(_i64p(hq), hq.size - 1)
    if ws_n == ctypes.c_size_t(-1).value:
        raise ValueError("malformed cu_q")
    ws = _alloc_ws(ws_n, dev)
    _check(lib().seqcomp_shared_kv_mqa(_ptr(q), _ptr(kv), q.shape[1], q.shape[2], _in_code(q), _i64p(hq), _ptr(cq),
                                       _i64p(hk), _ptr(ck), hq.size - 1, _ptr(nv), _ptr(k_sink), _ptr(v_sink), sc_,
                                       _ptr(out), _DT_CODE[out_dtype], _ptr(lse), _ptr(ws), ws_n, _stream(dev)),
           "seqcomp_shared_kv_mqa")
    return out, lse
