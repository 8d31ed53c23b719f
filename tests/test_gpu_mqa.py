"""GPU parity of the dense shared-KV MQA with attention sink
(seqcomp_shared_kv_mqa) against the float64 oracle.

Tolerance (helpers.check_mqa): per output element
|gpu - ref| <= 2^-7 sum_s alpha_s |v_s| (+ 2^-8 |ref| for bf16 output).  The
kernel's products are exact (bf16 x bf16 in fp32) and its sums fp32; the one
coarse step is the rounding of each probability to bf16 (relative 2^-9)
before the value product, and the bound gives it a 4x margin.  The
log-sum-exp is checked to 1e-4.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, mqa_abs_weighted, check_mqa

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(512.0)


def _ref(case, nv, rows, sink):
    """Oracle outputs of queries `rows` (each against its own sequence)."""
    seq = np.searchsorted(case.cu_q, rows, side="right") - 1
    Q = to64(case.q[torch.from_numpy(np.asarray(rows)).to(case.q.device)])
    KV = to64(case.kv)
    ks = to64(case.k_sink) if sink != "none" else None
    vs = to64(case.v_sink) if sink == "key+value" else None
    O, L, A = [], [], []
    for j, t in enumerate(rows):
        K = KV[case.cu_k[seq[j]]:case.cu_k[seq[j] + 1]]
        o, l = oracle.shared_kv_mqa(Q[j:j + 1], K, [nv[t]], SCALE, ks, vs)
        O.append(o[0]); L.append(l[0])
        A.append(mqa_abs_weighted(Q[j:j + 1], K, [nv[t]], SCALE, ks, vs)[0])
    return np.array(O), np.array(L), np.array(A)


def _run(case, nv, sink, out_dtype):
    ks = case.k_sink if sink != "none" else None
    vs = case.v_sink if sink == "key+value" else None
    return sc.shared_kv_mqa(case.q, case.kv, case.cu_q, case.cu_k, nv, ks, vs, SCALE, out_dtype, with_lse=True)


@pytest.mark.parametrize("sink", ["none", "key", "key+value"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_mqa_ragged_batch(gpu_device, sink, out_dtype):
    """Three sequences (one without entries), visible counts 0, partial tiles
    and all; f32 and bf16 output, with and without a sink."""
    case = synth.mqa_case([3, 1, 5], [300, 0, 130], seed=1, device=gpu_device)
    nv = np.array([300, 0, 77, 0, 130, 64, 1, 129, 65], dtype=np.int32)
    out, lse = _run(case, nv, sink, out_dtype)
    O, L, A = _ref(case, nv, np.arange(9), sink)
    check_mqa(to64(out), O, A, out_dtype, to64(lse), L)


def test_mqa_peaked_logits(gpu_device):
    """Queries with std 4 make the attention peaked (logit std 4): a few
    entries carry most of the weight and the probabilities span a wide range
    below the first tile's maximum; 2000 entries, sink with value."""
    case = synth.mqa_case([6], [2000], seed=2, device=gpu_device, q_std=4.0)
    nv = np.array([2000, 1999, 1000, 64, 63, 1500], dtype=np.int32)
    out, lse = _run(case, nv, "key+value", "f32")
    O, L, A = _ref(case, nv, np.arange(6), "key+value")
    check_mqa(to64(out), O, A, "f32", to64(lse), L)


def test_mqa_growing_logits_restart(gpu_device):
    """Logits that grow along the sequence far past the first tile's maximum:
    entry s has s in dimension 0 and half the heads have 8 there, so their
    logit rises by about 0.5 (log2 units) per entry -- over 64 above the
    first tile's maximum by the third tile, and again later, which restarts
    the sweep with a raised reference (several times for the longest
    queries).  The other heads stay ordinary; sink with value."""
    case = synth.mqa_case([4], [400], seed=3, device=gpu_device)
    case.kv[:, 0] = torch.arange(400, device=gpu_device, dtype=torch.float32).to(torch.bfloat16)
    case.q[:, :64, 0] = 8.0
    nv = np.array([400, 333, 190, 129], dtype=np.int32)
    for out_dtype in ("f32", "bf16"):
        out, lse = _run(case, nv, "key+value", out_dtype)
        O, L, A = _ref(case, nv, np.arange(4), "key+value")
        check_mqa(to64(out), O, A, out_dtype, to64(lse), L)


def test_mqa_restart_at_the_last_step(gpu_device):
    """Logits that rise by about 1.5 (log2 units) per entry in half the heads:
    from entry ~105 on, the second tile exceeds the first tile's maximum by
    more than 64, so the two-tile sweeps (110 and 128 visible) restart at their
    last step, just before the value product of the last tile, and the
    five-tile sweep restarts again at later tiles.  One-tile sweeps (64, and 65
    with a one-entry second tile) do not restart; sink with value."""
    case = synth.mqa_case([5], [300], seed=4, device=gpu_device)
    case.kv[:, 0] = (2.0 * torch.arange(300, device=gpu_device, dtype=torch.float32)).to(torch.bfloat16)
    case.q[:, :64, 0] = 12.0
    nv = np.array([110, 128, 64, 300, 65], dtype=np.int32)
    out, lse = _run(case, nv, "key+value", "f32")
    O, L, A = _ref(case, nv, np.arange(5), "key+value")
    check_mqa(to64(out), O, A, "f32", to64(lse), L)


def test_mqa_defaults_match_explicit_arguments(gpu_device):
    """Omitted visible counts mean every entry of the query's sequence, the
    default scale is 1/sqrt(512), and leaving out the log-sum-exp changes
    nothing else: the outputs equal the explicit call's bit for bit, and the
    oracle's within the usual bound."""
    case = synth.mqa_case([3, 2], [150, 64], seed=6, device=gpu_device)
    full = np.array([150] * 3 + [64] * 2, dtype=np.int32)
    a, la = sc.shared_kv_mqa(case.q, case.kv, case.cu_q, case.cu_k, full, case.k_sink, case.v_sink, SCALE, "f32",
                             with_lse=True)
    b, lb = sc.shared_kv_mqa(case.q, case.kv, case.cu_q, case.cu_k, None, case.k_sink, case.v_sink, None, "f32")
    assert lb is None
    assert torch.equal(a, b)
    O, L, A = _ref(case, full, np.arange(5), "key+value")
    check_mqa(to64(b), O, A, "f32", to64(la), L)


def test_mqa_full_config_sampled(gpu_device):
    """HCA at 1M context: 8192 entries (2^20 tokens, m' = 128); the last 4096
    tokens attend with causal visibility; sink with value; bf16 out.  Sampled
    queries (first, last, random) against the oracle."""
    cfg = synth.CONFIGS["hca_mqa_1m"]
    n_tok, T, m = cfg["n_tokens"], cfg["n_queries"], cfg["m"]
    case = synth.mqa_case([T], [n_tok // m], seed=0, device=gpu_device, q_std=cfg["q_std"])
    nv = synth.causal_visible(np.arange(n_tok - T, n_tok), m)
    out, lse = _run(case, nv, "key+value", "bf16")
    rows = np.array(sorted({0, 1, 127, T - 1} | set(np.random.default_rng(14).choice(T, 2, replace=False).tolist())))
    O, L, A = _ref(case, nv, rows, "key+value")
    sel = torch.from_numpy(rows).to(gpu_device)
    check_mqa(to64(out[sel]), O, A, "bf16", to64(lse[sel]), L)
