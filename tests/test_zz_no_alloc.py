"""The allocation-free fused entry point (seqcomp_compress_fused_noalloc),
called through the C ABI, against the workspace form seqcomp_compress_fused.

Both run the same kernels on the same inputs, so the entries (and fp8 codes
and scales) must be bit-identical: stricter than the oracle bar, which the
first case also checks.  Each case makes two calls in a row on the shared
per-device scratch, the second with a smaller batch, so state left behind by
the first call cannot leak into the second.  A call that would need more
than the 64 MiB of scratch is rejected before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import _lib, synth
from helpers import to64, row_rel_err

pytestmark = pytest.mark.gpu


def _pair(case, out_dtype):
    b = case.biases
    if case.mode == "csa":
        args = ("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], case.m, case.cu_seqlens, out_dtype)
    else:
        args = ("hca", case.H, case.Wt_cat, b["B"], None, case.m, case.cu_seqlens, out_dtype)
    got = sc.compress_fused_noalloc(*args)
    ref = sc.compress_fused(*args)
    torch.cuda.synchronize()
    return got, ref


def _same(got, ref):
    assert got[0].shape == ref[0].shape
    assert torch.equal(got[0], ref[0])
    if ref[1] is not None:
        assert torch.equal(got[1], ref[1])


@pytest.mark.parametrize("mode,out_dtype", [("csa", "bf16"), ("csa", "fp8"), ("hca", "bf16"), ("hca", "f32")])
def test_noalloc_matches_workspace_form_twice(gpu_device, mode, out_dtype):
    """Two calls in a row (a ragged batch of several tiles per sequence, then
    a smaller one): bit-identical to seqcomp_compress_fused."""
    m = 4 if mode == "csa" else 128
    big = [3000, 5, 1200, 777] if mode == "csa" else [5000, 100, 1300]
    small = [600, 9] if mode == "csa" else [700]
    for k, lengths in enumerate((big, small)):
        case = synth.compressor_case(mode, lengths, 256, 128, m, seed=40 + k, in_dtype="bf16", bias_std=0.3,
                                     device=gpu_device)
        got, ref = _pair(case, out_dtype)
        _same(got, ref)
        if k == 0 and out_dtype == "bf16":
            W = {nm: to64(v) for nm, v in case.W.items()}
            bb = {nm: to64(v) for nm, v in case.biases.items()}
            if mode == "csa":
                o = oracle.csa_compress(to64(case.H), W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], bb["Ba"],
                                        bb["Bb"], m, case.cu_seqlens)
            else:
                o = oracle.hca_compress(to64(case.H), W["W_KV"], W["W_Z"], bb["B"], m, case.cu_seqlens)
            assert row_rel_err(to64(got[0]), o).max() <= 2e-2


def test_noalloc_full_size_csa_then_smaller(gpu_device):
    """The CSA full workload (8192 tokens, d = 7168, c = 512, bf16), then a
    smaller packed batch at the same shape: bit-identical to the workspace
    form both times."""
    cfg = synth.CONFIGS["csa_full"]
    for k, lengths in enumerate(([8192], [3000, 1028])):
        case = synth.compressor_case("csa", lengths, cfg["d"], cfg["c"], 4, seed=k, in_dtype="bf16",
                                     bias_std=cfg["bias_std"], device=gpu_device)
        got, ref = _pair(case, "bf16")
        _same(got, ref)


def test_noalloc_rejects_calls_beyond_the_scratch(gpu_device):
    """A CSA call with fp8 output over 200K tokens needs ~100 MB of fp32
    staging: rejected with SEQCOMP_E_SCRATCH before any launch, and the
    output is left untouched."""
    lengths = [200704]
    c, d = 512, 64
    cu = synth.cu_from_lengths(lengths)
    H = torch.zeros((int(cu[-1]), d), dtype=torch.bfloat16, device=gpu_device)
    Wt = torch.zeros((4 * c, d), dtype=torch.bfloat16, device=gpu_device)
    B = torch.zeros((4, c), dtype=torch.float32, device=gpu_device)
    out = torch.full((int(cu[-1]) // 4, c), 7, dtype=torch.uint8, device=gpu_device)
    scale = torch.full((int(cu[-1]) // 4,), 3.0, dtype=torch.float32, device=gpu_device)
    with pytest.raises(sc.SeqcompError) as ei:
        sc.compress_fused_noalloc("csa", H, Wt, B, B, 4, cu, "fp8", out=out, out_scale=scale)
    assert ei.value.status == _lib.E_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7).all()) and bool((scale == 3.0).all())
