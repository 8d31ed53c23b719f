"""Float64 definition of the token-level compressor (CSA and HCA).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation follows the pages: hidden states H (n x d), KV streams C^a, C^b
(n x c), logit streams Z^a, Z^b (n x c), learned position biases B^a, B^b
(m x c), block size m (CSA, 4) or m' (HCA, 128), compressed entries C^Comp
(floor(n/m) x c).

Readings taken where the pages are silent or disagree (each is listed, with
its reason, in the design notes of the repository):

* Z is per channel (n x c), because B is m x c in "序列压缩注意力"; the CSA
  chapter's "n-dim Z" is the special case of identical columns.
* CSA normalises jointly over the 2m rows of the window, as the equation
  eq. attn-seqcomp-csa-softmax says, not per m-row segment.
* Row r of B^a (B^b, B) is added to the r-th row of its block.
* A trailing partial block (n mod m rows) forms no entry: E = floor(n/m),
  as in "Ch 04 · CSA" section 3 ("floor(n/m) segments") and "Ch 05 · HCA"
  section 5 (4000 tokens give 31 HCA entries).
* Sequences of a packed batch are independent; entry 0 of every sequence
  takes the boundary rule of eq. attn-seqcomp-overlap-bound.
* The softmax subtracts the per-channel maximum before exponentiating; this
  leaves the exact value unchanged.
"""

from __future__ import annotations

import numpy as np


def n_entries(n: int, m: int) -> int:
    """Number of compressed entries of one sequence of n tokens: floor(n/m).

    "Ch 04 · CSA" section 3 cuts the sequence into floor(n/m) segments; a
    partial tail block is dropped.
    """
    if m <= 0:
        raise ValueError("block size m must be positive")
    return int(n) // int(m)


def project(H: np.ndarray, W: np.ndarray) -> np.ndarray:
    """One stream of eq. attn-seqcomp-csa-proj: X = H W, in float64.

    H is (rows x d), W is (d x c) exactly as written on the page
    ("序列压缩注意力", eq. attn-seqcomp-csa-proj); the result is (rows x c).
    """
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if H.ndim != 2 or W.ndim != 2 or H.shape[1] != W.shape[0]:
        raise ValueError(f"shape mismatch: H {H.shape}, W {W.shape}")
    return H @ W


def _softmax_pool(logits: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Row-wise softmax over axis 1 of `logits`, then the Hadamard-weighted sum.

    logits, values: (E, rows, c).  For every entry and channel:
    S_j = exp(l_j) / sum_k exp(l_k) over the rows of the window, and the entry
    is sum_j S_j * v_j  ("序列压缩注意力", eq. attn-seqcomp-csa-softmax and
    eq. attn-seqcomp-csa-pool; eq. attn-seqcomp-hca for HCA).
    A logit of -inf has weight exactly 0 (exp(-inf) = 0).
    """
    top = logits.max(axis=1, keepdims=True)          # finite: >= 1 finite row
    w = np.exp(logits - top)
    S = w / w.sum(axis=1, keepdims=True)
    return (S * values).sum(axis=1)


def csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m: int, e0: int = 0, e1: int | None = None) -> np.ndarray:
    """CSA entries [e0, e1) of ONE sequence from its projected streams.

    Ca, Cb, Za, Zb: (n x c); Ba, Bb: (m x c).  Entry i reads
    * a-stream rows [m i, m(i+1) - 1]        (table tbl-attn-seqcomp-overlap),
    * b-stream rows [m(i-1), m i - 1],
    and takes ONE softmax per channel over those 2m rows of Z + B
    (eq. attn-seqcomp-csa-softmax), then sum S^a C^a + sum S^b C^b
    (eq. attn-seqcomp-csa-pool).  For i = 0 the b rows [-m, -1] do not exist:
    their logits are -inf and their vectors 0 (eq. attn-seqcomp-overlap-bound),
    so entry 0 is the a-stream alone.
    """
    Ca, Cb, Za, Zb = (np.asarray(x, dtype=np.float64) for x in (Ca, Cb, Za, Zb))
    Ba = np.asarray(Ba, dtype=np.float64)
    Bb = np.asarray(Bb, dtype=np.float64)
    n, c = Ca.shape
    if not (Cb.shape == Za.shape == Zb.shape == (n, c)):
        raise ValueError("all four streams must have the same shape")
    if Ba.shape != (m, c) or Bb.shape != (m, c):
        raise ValueError(f"B^a and B^b must be ({m}, {c})")
    E = n_entries(n, m)
    if e1 is None:
        e1 = E
    if not (0 <= e0 <= e1 <= E):
        raise ValueError(f"entry range [{e0}, {e1}) outside [0, {E})")
    k = e1 - e0
    if k == 0:
        return np.zeros((0, c))

    # a-stream: the current block of every entry.
    La = Za[m * e0:m * e1].reshape(k, m, c) + Ba[None]
    Va = Ca[m * e0:m * e1].reshape(k, m, c)

    # b-stream: the previous block; entry 0 gets logit -inf and vector 0.
    Lb = np.full((k, m, c), -np.inf)
    Vb = np.zeros((k, m, c))
    first = max(e0, 1)                              # first entry with a real block i-1
    if first < e1:
        rows = slice(m * (first - 1), m * (e1 - 1))
        Lb[first - e0:] = Zb[rows].reshape(e1 - first, m, c) + Bb[None]
        Vb[first - e0:] = Cb[rows].reshape(e1 - first, m, c)

    logits = np.concatenate([La, Lb], axis=1)       # (k, 2m, c): joint window
    values = np.concatenate([Va, Vb], axis=1)
    return _softmax_pool(logits, values)


def hca_pool_sequence(C, Z, B, m: int, e0: int = 0, e1: int | None = None) -> np.ndarray:
    """HCA entries [e0, e1) of ONE sequence (eq. attn-seqcomp-hca).

    C, Z: (n x c); B: (m x c).  Entry i is the softmax over the m rows
    [m i, m(i+1) - 1] of Z + B, per channel, applied to the same rows of C.
    One stream, no overlap ("Ch 05 · HCA" section 2).
    """
    C = np.asarray(C, dtype=np.float64)
    Z = np.asarray(Z, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    n, c = C.shape
    if Z.shape != (n, c):
        raise ValueError("C and Z must have the same shape")
    if B.shape != (m, c):
        raise ValueError(f"B must be ({m}, {c})")
    E = n_entries(n, m)
    if e1 is None:
        e1 = E
    if not (0 <= e0 <= e1 <= E):
        raise ValueError(f"entry range [{e0}, {e1}) outside [0, {E})")
    k = e1 - e0
    if k == 0:
        return np.zeros((0, c))
    L = Z[m * e0:m * e1].reshape(k, m, c) + B[None]
    V = C[m * e0:m * e1].reshape(k, m, c)
    return _softmax_pool(L, V)


def _check_cu(cu_seqlens, total_rows: int) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > total_rows:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and stay within the rows")
    return cu


def csa_pool(Ca, Cb, Za, Zb, Ba, Bb, m: int, cu_seqlens=None) -> np.ndarray:
    """Packed-batch CSA pooling: sequences [cu[b], cu[b+1]) are independent.

    Returns the entries of all sequences, sequence by sequence
    (sum_b floor(L_b/m) rows).
    """
    n = np.asarray(Ca).shape[0]
    cu = _check_cu([0, n] if cu_seqlens is None else cu_seqlens, n)
    outs = [csa_pool_sequence(Ca[s:t], Cb[s:t], Za[s:t], Zb[s:t], Ba, Bb, m)
            for s, t in zip(cu[:-1], cu[1:])]
    c = np.asarray(Ca).shape[1]
    return np.concatenate(outs, axis=0) if outs else np.zeros((0, c))


def hca_pool(C, Z, B, m: int, cu_seqlens=None) -> np.ndarray:
    """Packed-batch HCA pooling, sequences independent."""
    n = np.asarray(C).shape[0]
    cu = _check_cu([0, n] if cu_seqlens is None else cu_seqlens, n)
    outs = [hca_pool_sequence(C[s:t], Z[s:t], B, m) for s, t in zip(cu[:-1], cu[1:])]
    c = np.asarray(C).shape[1]
    return np.concatenate(outs, axis=0) if outs else np.zeros((0, c))


def csa_compress_sequence(H, W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m: int,
                          e0: int = 0, e1: int | None = None) -> np.ndarray:
    """Projection + CSA pooling for entries [e0, e1) of one sequence.

    Only the rows those entries read are projected: a rows [m e0, m e1) and
    b rows [m(e0-1), m(e1-1)) -- the projection of eq. attn-seqcomp-csa-proj
    is row-wise, so this is the same value as projecting all of H.
    """
    H = np.asarray(H, dtype=np.float64)
    n = H.shape[0]
    E = n_entries(n, m)
    if e1 is None:
        e1 = E
    if not (0 <= e0 <= e1 <= E):
        raise ValueError(f"entry range [{e0}, {e1}) outside [0, {E})")
    lo = max(e0 - 1, 0) * m          # first row any of these entries reads
    hi = e1 * m
    Hs = H[lo:hi]
    Ca, Cb = project(Hs, W_KVa), project(Hs, W_KVb)
    Za, Zb = project(Hs, W_Za), project(Hs, W_Zb)
    base = lo // m                    # entry index of the first block in Hs
    # Entry i of the sequence is entry (i - base) of the window Hs, except that
    # the window's own entry 0 would wrongly take the -inf boundary when
    # base > 0; ask for the entries starting one block in.
    return csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m, e0 - base, e1 - base)


def hca_compress_sequence(H, W_KV, W_Z, B, m: int, e0: int = 0, e1: int | None = None) -> np.ndarray:
    """Projection + HCA pooling for entries [e0, e1) of one sequence."""
    H = np.asarray(H, dtype=np.float64)
    E = n_entries(H.shape[0], m)
    if e1 is None:
        e1 = E
    if not (0 <= e0 <= e1 <= E):
        raise ValueError(f"entry range [{e0}, {e1}) outside [0, {E})")
    Hs = H[e0 * m:e1 * m]
    return hca_pool_sequence(project(Hs, W_KV), project(Hs, W_Z), B, m)


def csa_compress(H, W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m: int, cu_seqlens=None) -> np.ndarray:
    """Packed-batch CSA compressor (projection then pooling), float64."""
    n = np.asarray(H).shape[0]
    cu = _check_cu([0, n] if cu_seqlens is None else cu_seqlens, n)
    c = np.asarray(W_KVa).shape[1]
    outs = [csa_compress_sequence(H[s:t], W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m)
            for s, t in zip(cu[:-1], cu[1:])]
    return np.concatenate(outs, axis=0) if outs else np.zeros((0, c))


def hca_compress(H, W_KV, W_Z, B, m: int, cu_seqlens=None) -> np.ndarray:
    """Packed-batch HCA compressor (projection then pooling), float64."""
    n = np.asarray(H).shape[0]
    cu = _check_cu([0, n] if cu_seqlens is None else cu_seqlens, n)
    c = np.asarray(W_KV).shape[1]
    outs = [hca_compress_sequence(H[s:t], W_KV, W_Z, B, m) for s, t in zip(cu[:-1], cu[1:])]
    return np.concatenate(outs, axis=0) if outs else np.zeros((0, c))
