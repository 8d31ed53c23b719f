"""A seeded sweep of irregular shapes through the fused compressor, the
pooling calls and the decode append, each case against the float64 oracle.

The hand-picked parity cases elsewhere cover the edges one at a time; this
sweep combines them at random (seed fixed, so every run checks the same
cases): 1-6 packed sequences of 0-2600 tokens, d in {64, ..., 448}, c any
multiple of 16 up to 624 (1040 for pooling), fp32 and bf16 operands, every
output type, pooling m from 1 to 16 (CSA) and 1 to 256 (HCA).

Tolerances:
* fused and append, fp32 entries: max abs <= 5e-5.  The fp32 sums over
  d <= 448 err by ~2^-24 sqrt(d) |h w| (a few 1e-6 here); the bound keeps a
  tenfold margin while a dropped bias (std 0.5) moves entries by ~0.1;
* bf16 entries: per-row relative <= 2^-8 (one bf16 rounding plus the sums);
* fp8 entries: the codes equal the oracle encoder's on the call's own fp32
  entries (except within 1e-6 relative of a rounding midpoint), and stay
  within one E4M3 step of the oracle's entries;
* pooling from fp32 streams: max abs <= 1e-5.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, max_abs_err, row_rel_err, check_fp8, fp8_codes_match_encoder
from test_gpu_append import _append_all

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(20261204)


def _fused_cases(n):
    out = []
    for i in range(n):
        mode = ("csa", "hca")[i % 2]
        nseq = int(_RNG.integers(1, 7))
        lengths = _RNG.integers(0, 1400 if mode == "csa" else 2600, size=nseq).tolist()
        d = int(_RNG.choice([64, 128, 192, 256, 384, 448]))
        c = int(16 * _RNG.integers(1, 40))
        in_dtype = ("f32", "bf16")[(i // 2) % 2]
        out.append((i, mode, lengths, d, c, in_dtype))
    return out


def _pool_cases(n):
    out = []
    for i in range(n):
        nseq = int(_RNG.integers(1, 7))
        lengths = _RNG.integers(0, 3000, size=nseq).tolist()
        c = int(16 * _RNG.integers(1, 66))
        m_csa = int(_RNG.integers(1, 17))
        m_hca = int(_RNG.integers(1, 257))
        out.append((i, lengths, c, m_csa, m_hca))
    return out


def _append_cases():
    # the small-batch forms (one or two sequences, split-K small tiles) and a split big-tile batch
    out = []
    for i, nb in enumerate((1, 2, 3, 37, 300, 600)):
        d = int(_RNG.choice([64, 192, 512]))
        c = int(16 * _RNG.integers(1, 33))
        out.append((i, nb, d, c))
    return out


FUSED = _fused_cases(12)
POOL = _pool_cases(8)
APPEND = _append_cases()


def _oracle_fused(case):
    H = to64(case.H)
    W = {k: to64(v) for k, v in case.W.items()}
    b = {k: to64(v) for k, v in case.biases.items()}
    if case.mode == "csa":
        return oracle.csa_compress(H, W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], b["Ba"], b["Bb"], case.m,
                                   case.cu_seqlens)
    return oracle.hca_compress(H, W["W_KV"], W["W_Z"], b["B"], case.m, case.cu_seqlens)


@pytest.mark.parametrize("i,mode,lengths,d,c,in_dtype", FUSED)
def test_fused_random_shape(gpu_device, i, mode, lengths, d, c, in_dtype):
    m = 4 if mode == "csa" else 128
    case = synth.compressor_case(mode, lengths, d, c, m, seed=100 + i, in_dtype=in_dtype, bias_std=0.5,
                                 device=gpu_device)
    b = case.biases
    Ba, Bb = (b["Ba"], b["Bb"]) if mode == "csa" else (b["B"], None)
    run = lambda od: sc.compress_fused(mode, case.H, case.Wt_cat, Ba, Bb, m, case.cu_seqlens, od)
    ref = _oracle_fused(case)
    f32, _ = run("f32")
    assert f32.shape == ref.shape
    err = max_abs_err(to64(f32), ref)
    print(f"case {i}: {mode} lengths={lengths} d={d} c={c} {in_dtype}: max abs err {err:.3e}")
    assert err <= 5e-5
    b16, _ = run("bf16")
    if ref.size:
        assert row_rel_err(to64(b16), ref).max() <= 2.0 ** -8
    q, s = run("fp8")
    if ref.size:
        fp8_codes_match_encoder(q.cpu().numpy(), s.cpu().double().numpy(), to64(f32))
        check_fp8(q, s, ref, 0.0, 5e-5)


@pytest.mark.parametrize("i,lengths,c,m_csa,m_hca", POOL)
def test_pool_random_shape(gpu_device, i, lengths, c, m_csa, m_hca):
    T = int(sum(lengths))
    pc = synth.pool_case(T, c, m_csa=m_csa, m_hca=m_hca, seed=200 + i, dtype="f32", bias_std=0.5,
                         lengths=lengths, z_std=2.0)
    st = {k: v.to(gpu_device) for k, v in pc.streams.items()}
    bi = {k: v.to(gpu_device) for k, v in pc.biases.items()}
    cu = pc.cu_seqlens
    s64 = {k: to64(v) for k, v in pc.streams.items()}
    b64 = {k: to64(v) for k, v in pc.biases.items()}
    out, _ = sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], bi["Ba"], bi["Bb"], m_csa, cu, "f32")
    ref = oracle.csa_pool(s64["Ca"], s64["Cb"], s64["Za"], s64["Zb"], b64["Ba"], b64["Bb"], m_csa, cu)
    assert out.shape == ref.shape
    assert max_abs_err(to64(out), ref) <= 1e-5
    outh, _ = sc.pool_hca(st["Ca"], st["Za"], bi["B"], m_hca, cu, "f32")
    refh = oracle.hca_pool(s64["Ca"], s64["Za"], b64["B"], m_hca, cu)
    assert outh.shape == refh.shape
    assert max_abs_err(to64(outh), refh) <= 1e-5


@pytest.mark.parametrize("i,nb,d,c", APPEND)
def test_append_random_shape(gpu_device, i, nb, d, c):
    """Three appends per sequence (12 tokens each): the entries equal the
    whole-sequence oracle's."""
    case = synth.compressor_case("csa", [12] * nb, d, c, 4, seed=300 + i, in_dtype="f32", bias_std=0.5,
                                 device=gpu_device)
    out, _ = _append_all(case, "f32", in_place=True)
    ref = _oracle_fused(case)
    assert out.shape == ref.shape
    err = max_abs_err(to64(out), ref)
    print(f"append case {i}: nb={nb} d={d} c={c}: max abs err {err:.3e}")
    assert err <= 5e-5
