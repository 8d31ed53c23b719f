"""Partial RoPE + mixed-precision store (seqcomp_rope_store) against the oracle.

The entries fed to both sides are the same fp32 (or bf16) values, so the
comparison isolates the store: positions are block centres plus a per-sequence
offset, the last r dimensions turn in adjacent pairs ("Ch 05 · HCA — 长上下文
的全景镜", section on partial RoPE) and are kept in bf16, the rest in fp8 with
a per-entry scale ("混合压缩注意力双方案解析", section 3).

Tolerances: scale relative 1e-6 (an fp32 max and one division); fp8 codes
decode to within one E4M3 step of the scaled value (the code is a rounding
decision taken in fp32 on the GPU and float64 in the oracle, so the two may
differ at a midpoint); the bf16 RoPE part within one bf16 step (2^-8
relative) plus 1e-6 absolute of the float64 rotation.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, e4m3_step

pytestmark = pytest.mark.gpu


def _check(cache, rows, X, pos, r, base=10000.0):
    nope, scale, rope = (t.cpu() for t in cache)
    codes_ref, s_ref, rope_ref = oracle.rope_mixed_store(X, pos, r, base)
    c = X.shape[1]
    s = scale.double().numpy()[rows]
    assert np.all(np.abs(s / s_ref - 1) <= 1e-6)
    if c - r > 0:
        dec = oracle.fp8_e4m3_decode(nope.numpy()[rows]) * s[:, None]
        want = X[:, : c - r]
        bound = e4m3_step(want / s_ref[:, None]) * s_ref[:, None] + 1e-12
        assert np.all(np.abs(dec - want) <= bound)
        same = np.mean(nope.numpy()[rows] == codes_ref)
        assert same >= 0.999, same
    if r > 0:
        got = rope.double().numpy()[rows]
        rot = oracle.rope_partial(X, pos, r, base)[:, c - r:]
        assert np.all(np.abs(got - rot) <= 2.0 ** -8 * np.abs(rot) + 1e-6)
        assert np.mean(got == rope_ref) >= 0.99


def test_rope_store_fp32_slots_and_offsets(gpu_device):
    lengths = [300, 7, 0, 1029, 64, 3]
    cu = synth.cu_from_lengths(lengths)
    m, c, r = 4, 512, 64
    E = int(sum(L // m for L in lengths))
    X = synth.normal((E, c), 1.0, (11, 1), "cpu", "f32").double().numpy()
    X[5] = 0.0                                            # an all-zero entry: scale 1
    pos0 = np.array([0, 17, 5, 1_000_000, 123456, 9])
    n_slots = E + 40
    slots = np.random.default_rng(0).permutation(n_slots)[:E]
    cache = sc.rope_cache(n_slots, c, r, gpu_device)
    cache[1].fill_(-7.0)
    sc.rope_store(torch.from_numpy(X).float().to(gpu_device), m, cu, cache, r, pos0=pos0, slots=slots)
    torch.cuda.synchronize()
    _check(cache, slots, X, oracle.entry_positions(cu, m, pos0), r)
    untouched = np.setdiff1d(np.arange(n_slots), slots)
    assert np.all(cache[1].cpu().numpy()[untouched] == -7.0)


@pytest.mark.parametrize("c,r,m", [(128, 64, 4), (64, 0, 128), (64, 64, 128), (256, 8, 1)])
def test_rope_store_bf16_shapes(gpu_device, c, r, m):
    lengths = [m * 70 + 1, m * 3, m]
    cu = synth.cu_from_lengths(lengths)
    E = int(sum(L // m for L in lengths))
    Xb = synth.normal((E, c), 2.0, (12, c), "cpu", "bf16")
    X = Xb.double().numpy()
    cache = sc.rope_cache(E, c, r, gpu_device)
    sc.rope_store(Xb.to(gpu_device), m, cu, cache, r)
    torch.cuda.synchronize()
    _check(cache, np.arange(E), X, oracle.entry_positions(cu, m), r)


def test_fused_then_store_matches_oracle(gpu_device):
    """Fused CSA entries (fp32 operands) stored with RoPE: the stored cache
    against the oracle's compressor followed by its mixed store."""
    lengths = [260, 45, 517]
    case = synth.compressor_case("csa", lengths, 128, 128, 4, seed=6, in_dtype="f32", bias_std=0.3,
                                 device=gpu_device)
    b = case.biases
    out, _ = sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, case.cu_seqlens, "f32")
    cache = sc.rope_cache(out.shape[0], 128, 64, gpu_device)
    sc.rope_store(out, 4, case.cu_seqlens, cache, 64)
    torch.cuda.synchronize()
    W = {k: to64(v) for k, v in case.W.items()}
    bb = {k: to64(v) for k, v in b.items()}
    ref = oracle.csa_compress(to64(case.H), W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], bb["Ba"], bb["Bb"], 4,
                              case.cu_seqlens)
    # the entries themselves differ from the oracle by the fused path's fp32 error (<= 2e-5): compare the
    # stored cache against the oracle store of the GPU's own entries, then the entries against the oracle
    _check(cache, np.arange(out.shape[0]), to64(out), oracle.entry_positions(case.cu_seqlens, 4), 64)
    assert np.max(np.abs(to64(out) - ref)) <= 2e-5


def test_rope_store_many_sequences(gpu_device):
    """70 sequences (past the 64 whose tiles the kernel looks up itself: the
    planner's table), ragged lengths with empty and short ones, random
    offsets: against the oracle store."""
    rng = np.random.default_rng(14)
    lengths = rng.integers(0, 700, size=70)
    lengths[[2, 30]] = 0
    lengths[[7, 50]] = 3
    cu = synth.cu_from_lengths(lengths)
    m, c, r = 4, 256, 64
    E = int(sum(L // m for L in lengths))
    X = synth.normal((E, c), 1.0, (14, 1), "cpu", "f32").double().numpy()
    pos0 = rng.integers(0, 100000, size=70)
    cache = sc.rope_cache(E, c, r, gpu_device)
    sc.rope_store(torch.from_numpy(X).float().to(gpu_device), m, cu, cache, r, pos0=pos0)
    torch.cuda.synchronize()
    _check(cache, np.arange(E), X, oracle.entry_positions(cu, m, pos0), r)


def test_rope_store_wide_entries(gpu_device):
    """c > 512 takes the chunked path: 1024 channels, 128 of them rotated."""
    lengths = [4 * 9, 4 * 70]
    cu = synth.cu_from_lengths(lengths)
    c, r = 1024, 128
    E = int(sum(L // 4 for L in lengths))
    X = synth.normal((E, c), 1.0, (13, 1), "cpu", "f32").double().numpy()
    cache = sc.rope_cache(E, c, r, gpu_device)
    sc.rope_store(torch.from_numpy(X).float().to(gpu_device), 4, cu, cache, r, pos0=[3, 40000])
    torch.cuda.synchronize()
    _check(cache, np.arange(E), X, oracle.entry_positions(cu, 4, [3, 40000]), r)
