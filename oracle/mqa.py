"""Dense shared-KV multi-query attention with an attention sink.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* "Ch 05 · HCA — 长上下文的全景镜", section 2: after compression, HCA runs
  dense attention over all n/m' compressed entries (no top-k), through the
  shared-KV multi-query attention of the CSA chapter;
* "Ch 04 · CSA — 长上下文的快通道", section 6: all n_h = 128 query heads
  share one KV;
* "Ch 05 · HCA", section 4, item 3 (attention sink): a learned virtual key
  k_sink joins the keys inside the softmax, with value v_sink or zero:
  (alpha_sink, alpha_1, ..., alpha_n) = Softmax(q . [k_sink, k_1, ..., k_n]).

Readings (this library's): an entry serves as both key and value (one KV
vector per entry, shared by every head); logits are scaled by `scale`
(1/sqrt(c) in the standard form); query t sees its sequence's first
n_valid[t] entries (the blocks of m' tokens complete at its position); the
sink key and value are shared by all heads, like the entries; with no sink
and no visible entry the output is zero and the log-sum-exp -inf.
"""

from __future__ import annotations

import numpy as np


def shared_kv_mqa(Q, KV, n_valid, scale: float, k_sink=None, v_sink=None):
    """O (T x H x c) and log-sum-exp of the logits (T x H), float64.

    Q: T x H x c queries; KV: N x c entries (keys = values); n_valid[t]: the
    entries query t sees, KV[:n_valid[t]]; k_sink, v_sink: c-vectors or None
    (no sink / zero sink value)."""
    Q = np.asarray(Q, dtype=np.float64)
    KV = np.asarray(KV, dtype=np.float64)
    T, H, c = Q.shape
    O = np.zeros((T, H, c))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        keys = KV[: int(n_valid[t])]
        vals = keys
        if k_sink is not None:
            keys = np.vstack([np.asarray(k_sink, dtype=np.float64)[None, :], keys])
            vs = np.zeros(c) if v_sink is None else np.asarray(v_sink, dtype=np.float64)
            vals = np.vstack([vs[None, :], vals])
        if keys.shape[0] == 0:
            continue
        logits = scale * (Q[t] @ keys.T)                     # H x n: q_h . k_s for every head
        mx = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - mx)
        tot = e.sum(axis=1, keepdims=True)
        O[t] = (e / tot) @ vals                              # softmax over the keys, then weighted values
        lse[t] = (mx + np.log(tot))[:, 0]
    return O, lse
