"""Lightning indexer: ReLU index scores over compressed keys and top-k.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Ch 04 · CSA — 长上下文的快通道", section 4 (lightning indexer).  For
query t and compressed indexer key s the score sums, over the n_h^I = 64
indexer heads (c^I = 128 dims each), the head weight times the rectified dot
product of that head's query with the key:

    I[t, s] = sum_h  w[t, h] * ReLU(q[t, h] . K[s])

and query t keeps the compressed entries whose scores are among its k largest
(k = 1024 or 512).

Readings (this library's, where the section leaves the step open):
* the selection is a set; it is returned as key indices in increasing order
  (the order in which the entries sit in memory), with their scores;
* ties are broken towards the smaller key index, so the set is unique;
* query t sees only its first n_valid[t] keys (those whose blocks are
  complete at its position); when fewer than k are visible, all of them are
  selected and the remaining slots hold index -1 and score -inf.
"""

from __future__ import annotations

import numpy as np


def index_scores(Q, w, K, n_valid=None) -> np.ndarray:
    """I[t, s] for Q (T x H x c), w (T x H), K (N x c), in float64; keys at
    s >= n_valid[t] score -inf (invisible)."""
    Q = np.asarray(Q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    T, H, c = Q.shape
    N = K.shape[0]
    dots = (Q.reshape(T * H, c) @ K.T).reshape(T, H, N)      # q[t, h] . K[s]
    I = np.einsum("th,ths->ts", w, np.maximum(dots, 0.0))     # sum_h w ReLU(.)
    if n_valid is not None:
        visible = np.arange(N)[None, :] < np.asarray(n_valid).reshape(T, 1)
        I = np.where(visible, I, -np.inf)
    return I


def top_k(I, k: int):
    """(indices int64 T x k, scores T x k): per row, the k visible keys of
    largest score (ties towards the smaller index), listed by increasing key
    index; -1 / -inf fill the slots past the visible keys."""
    I = np.asarray(I, dtype=np.float64)
    T, N = I.shape
    idx = np.full((T, k), -1, dtype=np.int64)
    val = np.full((T, k), -np.inf)
    for t in range(T):
        visible = [s for s in range(N) if I[t, s] > -np.inf]
        ranked = sorted(visible, key=lambda s: (-I[t, s], s))
        chosen = sorted(ranked[:k])
        idx[t, : len(chosen)] = chosen
        val[t, : len(chosen)] = I[t, chosen]
    return idx, val
