"""Partial RoPE and the mixed-precision store of compressed entries.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:

* "Ch 05 · HCA — 长上下文的全景镜", the section on partial RoPE: rotary
  position encoding turns every pair of adjacent dimensions by a
  position-dependent angle, and only the last r = 64 of the c = 512 entry
  dimensions carry it; the other c - r stay position-free.  A compressed
  entry has no single position; the page says the segment's position is
  carried approximately by the RoPE of the segment centre.
* "混合压缩注意力双方案解析：CSA与HCA技术对比与选型指南", section 3
  (mixed-precision storage): the RoPE dimensions are stored in bf16, the
  other KV values in fp8.

Readings where the pages are silent (this library's, stated once here):

* pair k of the r RoPE dimensions is (c - r + 2k, c - r + 2k + 1) and turns
  by pos * theta_k with theta_k = base^(-2k / r), base 10000 by default
  (the usual rotary frequencies; the pages give no base);
* the position of entry i of a sequence is the centre of the block it
  compresses, m i + (m - 1) / 2 tokens from the sequence start, plus the
  caller's offset of that sequence (pos0, 0 by default);
* the fp8 part uses the per-entry scale rule of ``fp8_entry_quantize`` over
  the c - r position-free dimensions only.
"""

from __future__ import annotations

import numpy as np

from .encode import fp8_entry_quantize, round_bf16


def entry_positions(cu_seqlens, m: int, pos0=None) -> np.ndarray:
    """Position (float64) of every packed entry: block centre m i + (m-1)/2
    within its sequence, plus pos0[b] for sequence b."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = []
    for b in range(cu.size - 1):
        E = (int(cu[b + 1]) - int(cu[b])) // m
        off = 0.0 if pos0 is None else float(pos0[b])
        out.append(off + m * np.arange(E, dtype=np.float64) + (m - 1) / 2.0)
    return np.concatenate(out) if out else np.zeros(0)


def rope_partial(X, pos, r: int, base: float = 10000.0) -> np.ndarray:
    """Rotate the last r dimensions of every row of X (E x c) by its position.

    For pair k (k = 0 .. r/2 - 1) at columns (j, j + 1), j = c - r + 2k:
        x'_j     = x_j cos(a) - x_{j+1} sin(a)
        x'_{j+1} = x_j sin(a) + x_{j+1} cos(a),   a = pos * base^(-2k / r).
    The first c - r columns are returned unchanged.
    """
    X = np.array(X, dtype=np.float64, copy=True)
    pos = np.asarray(pos, dtype=np.float64)
    E, c = X.shape
    assert r % 2 == 0 and 0 <= r <= c
    for k in range(r // 2):
        j = c - r + 2 * k
        a = pos * base ** (-2.0 * k / r)
        cs, sn = np.cos(a), np.sin(a)
        x, y = X[:, j].copy(), X[:, j + 1].copy()
        X[:, j] = x * cs - y * sn
        X[:, j + 1] = x * sn + y * cs
    return X


def rope_mixed_store(X, pos, r: int, base: float = 10000.0):
    """Entries as stored in the cache: (fp8 codes of the c - r position-free
    dimensions (E x (c - r)) uint8, their per-entry scales (E,), and the r
    rotated dimensions rounded to bf16 (E x r) float64)."""
    Y = rope_partial(X, pos, r, base)
    c = Y.shape[1]
    codes, scales = fp8_entry_quantize(Y[:, : c - r])
    return codes, scales, round_bf16(Y[:, c - r:])
