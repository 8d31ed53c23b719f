"""Reentrancy: the library keeps no mutable state between calls (the
allocation-free entry point's scratch aside), so calls on different streams
may overlap.  Two streams run the fused compressor, the pooling call and the
decode append on different batches at the same time; every result must equal
the same call made alone, bit for bit."""

import pytest
import torch

import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth

pytestmark = pytest.mark.gpu


def _work(case, pool_in, app):
    b = case.biases
    out = [sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, case.cu_seqlens, "fp8")]
    Ca, Cb, Za, Zb = pool_in
    out.append(sc.pool_csa(Ca, Cb, Za, Zb, b["Ba"], b["Bb"], 4, case.cu_seqlens, "bf16"))
    H, state = app
    st = state.clone()
    out.append(sc.csa_append(H, case.Wt_cat, b["Ba"], b["Bb"], st, "bf16", state_out=st))
    return out


def _flat(res):
    ts = []
    for r in res:
        ts.extend(x for x in r if x is not None)
    return ts


def test_two_streams_overlap(gpu_device):
    cases, pools, apps = [], [], []
    for k, lengths in enumerate(([3000, 17, 900], [2048, 1300, 5, 640])):
        case = synth.compressor_case("csa", lengths, 256, 128, 4, seed=60 + k, in_dtype="bf16", bias_std=0.3,
                                     device=gpu_device)
        T = int(sum(lengths))
        pools.append([synth.normal((T, 128), 1.0, (61 + k, i), gpu_device, "bf16") for i in range(4)])
        nb = 96 + 40 * k
        apps.append((case.H[:4 * nb], sc.csa_empty_state(nb, 128, gpu_device)))
        cases.append(case)
    alone = [_flat(_work(cases[k], pools[k], apps[k])) for k in range(2)]     # also warms the offsets' copies
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(gpu_device) for _ in range(2)]
    for s, k in zip(streams, range(2)):                                       # the offsets' copies, per stream
        with torch.cuda.stream(s):
            _work(cases[k], pools[k], apps[k])
    torch.cuda.synchronize()
    for rep in range(3):
        got = [None, None]
        for s, k in zip(streams, range(2)):
            with torch.cuda.stream(s):
                got[k] = _flat(_work(cases[k], pools[k], apps[k]))
        torch.cuda.synchronize()
        for k in range(2):
            assert len(got[k]) == len(alone[k])
            for a, g in zip(alone[k], got[k]):
                assert torch.equal(a, g), f"stream {k}, repetition {rep}"
