"""GPU parity of the lightning indexer (seqcomp_indexer_topk) with the oracle.

Exact cases: integer inputs in [-3, 3] (and integer ramps of at most 250):
every product and partial sum is then an integer below 2^24, so the fp32
kernel and the float64 oracle compute the same scores; both break ties
towards the smaller key index, so the selections must be identical --
indices and scores compared for equality.

Random bf16 cases: when two scores lie within rounding of each other either
may be selected.  Per query the bound is beta = 200 u max_s sum_h |w_h|
sum_i |q_hi K_si| (u = 2^-24; derivation in helpers.indexer_score_bound);
the selection must be valid under it (helpers.check_topk_valid): returned
scores within beta of the oracle's, indices distinct, increasing and visible,
every key above the oracle's k-th score + 2 beta selected, none below the
k-th - 2 beta.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, indexer_score_bound, check_topk_valid

pytestmark = pytest.mark.gpu


def _oracle(case, nv, k, rows=None):
    """Oracle scores and selection of the queries `rows` (default: all)."""
    T = case.q.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    Q = to64(case.q[torch.from_numpy(rows).to(case.q.device)])
    w = to64(case.w[torch.from_numpy(rows).to(case.w.device)])
    seq = np.searchsorted(case.cu_q, rows, side="right") - 1
    keys = to64(case.keys)
    I_rows, idx_rows, val_rows, beta = [], [], [], []
    for j, t in enumerate(rows):
        K = keys[case.cu_k[seq[j]]:case.cu_k[seq[j] + 1]]
        I = oracle.index_scores(Q[j:j + 1], w[j:j + 1], K, n_valid=[nv[t]])
        idx, val = oracle.top_k(I, k)
        I_rows.append(I[0])
        idx_rows.append(idx[0])
        val_rows.append(val[0])
        beta.append(indexer_score_bound(Q[j:j + 1], w[j:j + 1], K[:nv[t]])[0])
    return I_rows, np.array(idx_rows), np.array(val_rows), np.array(beta)


def _visible(case, rng, full_frac=0.5):
    """Per query: all of its sequence's keys, none, a few or a random count."""
    nv = np.zeros(case.q.shape[0], dtype=np.int32)
    for b in range(len(case.cu_q) - 1):
        nk = int(case.cu_k[b + 1] - case.cu_k[b])
        for t in range(case.cu_q[b], case.cu_q[b + 1]):
            r = rng.random()
            nv[t] = nk if r < full_frac else (0 if r < full_frac + 0.05 else int(rng.integers(0, nk + 1)))
    return nv


@pytest.mark.parametrize("k", [1, 64, 1024])
def test_indexer_exact_integer_ragged_batch(gpu_device, k):
    """Integer inputs, 5 sequences (ragged query tiles, a sequence without
    queries, one without keys), visible counts from 0 to all: exact."""
    case = synth.indexer_case([13, 1, 40, 0, 9], [300, 5, 2000, 50, 0], seed=1, device=gpu_device, integer=True)
    nv = _visible(case, np.random.default_rng(7))
    idx, scores = sc.indexer_topk(case.q, case.w, case.keys, k, case.cu_q, case.cu_k, nv)
    _, ref_idx, ref_val, _ = _oracle(case, nv, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(scores.cpu().double().numpy(), ref_val)


@pytest.mark.parametrize("order", ["rising", "falling"])
@pytest.mark.parametrize("k", [100, 1024])
def test_indexer_exact_monotone_scores(gpu_device, order, k):
    """Scores that rise with the key index accept every key (a compaction
    every ~500 keys); falling scores accept almost none after the first k.
    Keys are v * (1 + s // 64) (ties in runs of 64), all heads query v with
    weight 1: exact."""
    N, T = 16000, 3
    v = torch.from_numpy(np.random.default_rng(3).choice([-1.0, 1.0], size=128).astype(np.float32))
    g = torch.arange(N, dtype=torch.float32) // 64 + 1
    if order == "falling":
        g = g.flip(0)
    keys = (g[:, None] * v[None, :]).to(torch.bfloat16).to(gpu_device)
    q = v.expand(T, 64, 128).to(torch.bfloat16).contiguous().to(gpu_device)
    w = torch.ones((T, 64), dtype=torch.float32, device=gpu_device)
    nv = np.array([N, N - 1000, 777], dtype=np.int32)
    idx, scores = sc.indexer_topk(q, w, keys, k, n_valid=nv)
    I = oracle.index_scores(to64(q), to64(w), to64(keys), n_valid=nv)
    ref_idx, ref_val = oracle.top_k(I, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(scores.cpu().double().numpy(), ref_val)


@pytest.mark.parametrize("k", [512, 1024])
def test_indexer_random_causal_chunk(gpu_device, k):
    """bf16 N(0,1) inputs: one sequence of 24000 tokens (6000 keys, m = 4);
    its last 61 tokens query with causal visibility floor((p + 1) / 4)."""
    n_tok, T = 24000, 61
    case = synth.indexer_case([T], [n_tok // 4], seed=2, device=gpu_device)
    nv = synth.causal_visible(np.arange(n_tok - T, n_tok), 4)
    idx, scores = sc.indexer_topk(case.q, case.w, case.keys, k, case.cu_q, case.cu_k, nv)
    I, _, _, beta = _oracle(case, nv, k)
    check_topk_valid(idx.cpu().numpy(), scores.cpu().double().numpy(), np.array(I), nv, k, beta)
    # the kernel is deterministic, and the score pointer is optional
    idx2, none = sc.indexer_topk(case.q, case.w, case.keys, k, case.cu_q, case.cu_k, nv, with_scores=False)
    assert none is None and torch.equal(idx, idx2)


def test_indexer_nothing_visible(gpu_device):
    """No visible key (n_valid 0, or a sequence without keys): all -1 / -inf."""
    case = synth.indexer_case([5, 4], [100, 0], seed=4, device=gpu_device)
    nv = np.array([0, 0, 0, 0, 0, 3, 3, 3, 3], dtype=np.int32)
    idx, scores = sc.indexer_topk(case.q, case.w, case.keys, 16, case.cu_q, case.cu_k, nv)
    assert bool((idx == -1).all()) and bool(torch.isneginf(scores).all())


def test_indexer_full_config_sampled(gpu_device):
    """1M-token context: 262144 keys (m = 4), the last 4096 tokens query
    (causal), k = 1024, bf16.  Sampled queries (tile edges, first, last,
    random) against the oracle under the rounding bound."""
    cfg = synth.CONFIGS["indexer_1m"]
    n_tok, T, m, k = cfg["n_tokens"], cfg["n_queries"], cfg["m"], cfg["k"]
    case = synth.indexer_case([T], [n_tok // m], seed=0, device=gpu_device)
    nv = synth.causal_visible(np.arange(n_tok - T, n_tok), m)
    idx, scores = sc.indexer_topk(case.q, case.w, case.keys, k, case.cu_q, case.cu_k, nv)
    rows = np.array(sorted({0, 1, 7, 8, 2047, T - 1} | set(np.random.default_rng(12).choice(T, 3, replace=False).tolist())))
    I, _, _, beta = _oracle(case, nv, k, rows)
    sel = torch.from_numpy(rows).to(gpu_device)
    check_topk_valid(idx[sel].cpu().numpy(), scores[sel].cpu().double().numpy(), np.array(I), nv[rows], k, beta)
