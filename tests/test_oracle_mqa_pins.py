"""Pins of the shared-KV MQA oracle with attention sink (oracle/mqa.py).

Sources: "Ch 05 · HCA — 长上下文的全景镜" (dense attention over every
compressed entry; the attention sink as a learned virtual key inside the
softmax, with value v_sink or zero) and "Ch 04 · CSA — 长上下文的快通道",
section 6 (all query heads share one KV).

Facts used, none produced by the oracle itself: torch's scaled-dot-product
attention (a library routine) in float64 on the CPU, with the sink as one more
key/value row in front; torch.logsumexp; closed forms (one visible entry gives
that entry; equal logits give the mean; two keys and a sink give the
three-way weights written out); shift invariance along a direction every key
shares; and planted mistakes (no sink, a sink value where zero is meant, a
missing scale, a softmax over heads) that these checks reject.
"""

import numpy as np
import pytest
import torch

import oracle


def _data(T=3, H=4, c=8, N=9, seed=0):
    rng = np.random.default_rng([seed, 77])
    return rng.normal(size=(T, H, c)), rng.normal(size=(N, c)), rng.normal(size=c), rng.normal(size=c)


def _sdpa(Q, KV, nv, scale, k_sink=None, v_sink=None):
    """torch float64 SDPA per query, the sink prepended as an ordinary key."""
    T, H, c = Q.shape
    out = np.zeros((T, H, c))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        K = KV[: nv[t]]
        V = K
        if k_sink is not None:
            K = np.vstack([k_sink[None], K])
            V = np.vstack([(np.zeros(c) if v_sink is None else v_sink)[None], V])
        if K.shape[0] == 0:
            continue
        q = torch.from_numpy(Q[t])[None]                     # 1 x H x c
        k = torch.from_numpy(K)[None, None].expand(1, H, -1, -1)
        v = torch.from_numpy(V)[None, None].expand(1, H, -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], k, v, scale=scale)
        out[t] = o[0, :, 0].numpy()
        lse[t] = torch.logsumexp(scale * (q[0] @ torch.from_numpy(K).T), dim=1).numpy()
    return out, lse


@pytest.mark.parametrize("sink", ["none", "key", "key+value"])
def test_matches_library_attention(sink):
    Q, KV, ks, vs = _data()
    nv = np.array([9, 4, 1])
    k_sink = None if sink == "none" else ks
    v_sink = vs if sink == "key+value" else None
    O, lse = oracle.shared_kv_mqa(Q, KV, nv, 0.35, k_sink, v_sink)
    O2, lse2 = _sdpa(Q, KV, nv, 0.35, k_sink, v_sink)
    np.testing.assert_allclose(O, O2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    Q, KV, ks, vs = _data()
    # one visible entry, no sink: the output is that entry for every head
    O, _ = oracle.shared_kv_mqa(Q, KV, [1, 1, 1], 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(KV[0], O.shape), rtol=1e-15)
    # zero queries: equal logits, the output is the mean of the visible entries
    # (with a sink whose value is v: (v + sum) / (n + 1))
    O, lse = oracle.shared_kv_mqa(np.zeros_like(Q), KV, [9, 5, 2], 0.5)
    for t, n in enumerate([9, 5, 2]):
        np.testing.assert_allclose(O[t], np.broadcast_to(KV[:n].mean(0), O[t].shape), rtol=1e-13)
        np.testing.assert_allclose(lse[t], np.log(n), rtol=1e-15)
    O, _ = oracle.shared_kv_mqa(np.zeros_like(Q), KV, [3, 3, 3], 0.5, ks, vs)
    np.testing.assert_allclose(O[0, 0], (vs + KV[:3].sum(0)) / 4, rtol=1e-13)
    # two keys and a sink of zero value, weights written out
    q = np.array([[[1.0, 0.0]]])
    K = np.array([[2.0, 0.0], [0.0, 1.0]])
    O, lse = oracle.shared_kv_mqa(q, K, [2], 1.0, k_sink=np.array([1.0, 0.0]))
    z = np.exp(2.0) + np.exp(0.0) + np.exp(1.0)              # logits 2 (key 0), 0 (key 1), 1 (sink)
    np.testing.assert_allclose(O[0, 0], (np.exp(2.0) * K[0] + np.exp(0.0) * K[1]) / z, rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(z), rtol=1e-15)


def test_empty_visibility():
    Q, KV, ks, vs = _data()
    O, lse = oracle.shared_kv_mqa(Q, KV, [0, 0, 0], 0.3)
    assert np.all(O == 0) and np.all(np.isneginf(lse))
    O, lse = oracle.shared_kv_mqa(Q, KV, [0, 0, 0], 0.3, ks, vs)   # only the sink: its value, weight 1
    np.testing.assert_allclose(O, np.broadcast_to(vs, O.shape), rtol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * Q @ ks, rtol=1e-14)


def test_shift_invariance():
    # every key and the sink have 1 in the last coordinate, so adding 5 to that
    # coordinate of every query moves all logits of a head (sink included) by
    # 0.4 * 5 = 2: the weights stay, the log-sum-exp grows by 2
    Q, KV, ks, vs = _data(c=8)
    KV = KV.copy(); KV[:, 7] = 1.0
    ks = ks.copy(); ks[7] = 1.0
    O1, lse1 = oracle.shared_kv_mqa(Q, KV, [9, 6, 3], 0.4, ks, vs)
    Q2 = Q.copy(); Q2[..., 7] += 5.0                             # every logit of a head + 0.4 * 5
    O2, lse2 = oracle.shared_kv_mqa(Q2, KV, [9, 6, 3], 0.4, ks, vs)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse1 + 2.0, rtol=1e-12)


def test_planted_mistakes_are_caught():
    Q, KV, ks, vs = _data()
    nv = np.array([9, 4, 1])
    ref, _ = _sdpa(Q, KV, nv, 0.35, ks, None)
    no_sink, _ = oracle.shared_kv_mqa(Q, KV, nv, 0.35)
    sink_value, _ = oracle.shared_kv_mqa(Q, KV, nv, 0.35, ks, ks)        # k_sink used as its value
    no_scale, _ = oracle.shared_kv_mqa(Q, KV, nv, 1.0, ks, None)
    assert not np.allclose(no_sink, ref)
    assert not np.allclose(sink_value, ref)
    assert not np.allclose(no_scale, ref)

    def heads_softmax(Q, KV, nv, scale):                                # normalised over heads, not keys
        out = np.zeros_like(Q)
        for t in range(Q.shape[0]):
            lg = scale * Q[t] @ KV[: nv[t]].T
            e = np.exp(lg - lg.max(0, keepdims=True))
            out[t] = (e / e.sum(0, keepdims=True)) @ KV[: nv[t]]
        return out
    ref0, _ = _sdpa(Q, KV, nv, 0.35)
    assert not np.allclose(heads_softmax(Q, KV, nv, 0.35), ref0)
