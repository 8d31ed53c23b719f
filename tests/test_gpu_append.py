"""CSA decode append (seqcomp_csa_append) against the float64 oracle.

Appending the blocks of every sequence one call at a time, carrying the
b-stream state between calls, must give the entries of the whole-sequence
compressor ("序列压缩注意力", eq. attn-seqcomp-csa-softmax / -pool, with the
first block's b-rows masked: eq. attn-seqcomp-overlap-bound).  Tolerances as
for the fused path: fp32 max abs <= 2e-5 (fp32 dot products over d = 128),
bf16 per-row relative <= 2e-2, fp8 one E4M3 step on top of that.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, max_abs_err, row_rel_err, check_fp8

pytestmark = pytest.mark.gpu


def _oracle(case):
    W = {k: to64(v) for k, v in case.W.items()}
    b = {k: to64(v) for k, v in case.biases.items()}
    return oracle.csa_compress(to64(case.H), W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], b["Ba"], b["Bb"], 4,
                               case.cu_seqlens)


def _append_all(case, out_dtype, in_place):
    """Feed block k of every sequence that has one at step k; returns the
    entries in the packed order of the whole-sequence compressor."""
    cu = case.cu_seqlens
    nblk = np.diff(cu) // 4
    nseq = len(nblk)
    dev = case.H.device
    c = case.c
    state = sc.csa_empty_state(nseq, c, dev)
    starts = np.concatenate([[0], np.cumsum(nblk)])
    got = [None] * int(starts[-1])
    scales = [None] * int(starts[-1])
    b = case.biases
    for k in range(int(nblk.max(initial=0))):
        seqs = np.nonzero(nblk > k)[0]
        rows = np.concatenate([np.arange(cu[s] + 4 * k, cu[s] + 4 * k + 4) for s in seqs])
        H = case.H[torch.from_numpy(rows).to(dev)].contiguous()
        idx = torch.from_numpy(seqs).to(dev)
        st = state[idx].contiguous()
        out, scale, st2 = sc.csa_append(H, case.Wt_cat, b["Ba"], b["Bb"], st, out_dtype,
                                        state_out=st if in_place else None)
        if in_place:
            assert st2.data_ptr() == st.data_ptr()
        state[idx] = st2
        for r, s in enumerate(seqs):
            got[starts[s] + k] = out[r]
            if scale is not None:
                scales[starts[s] + k] = scale[r]
    torch.cuda.synchronize()
    out = torch.stack(got) if got else torch.empty((0, c), device=dev)
    sc_ = torch.stack(scales) if scales and scales[0] is not None else None
    return out, sc_


@pytest.mark.parametrize("lengths,c", [
    ([8, 4, 13, 40, 0, 3, 24], 80),                 # ragged block counts, tails, empty and short sequences
    ([4 * 3] * 70, 64),                              # 70 sequences: two tiles of 64 blocks per call
    ([8, 12, 4, 20], 1024),                         # c = 1024: 32 channel tiles of the small-batch form
])
def test_append_fp32_matches_whole_sequence(gpu_device, lengths, c):
    case = synth.compressor_case("csa", lengths, 128, c, 4, seed=3, in_dtype="f32", bias_std=0.3, device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "f32", in_place=False)
    assert out.shape == ref.shape
    assert max_abs_err(to64(out), ref) <= 2e-5


def test_append_bf16_in_place_and_fp8(gpu_device):
    """300 sequences (5 tiles per call), bf16 operands, state updated in place."""
    lengths = [4 * 2] * 250 + [4 * 3 + 1] * 50
    case = synth.compressor_case("csa", lengths, 256, 128, 4, seed=4, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "bf16", in_place=True)
    assert row_rel_err(to64(out), ref).max() <= 2e-2
    q, s = _append_all(case, "fp8", in_place=False)
    check_fp8(q, s, ref, 2e-2)


def test_append_split_k_full_depth(gpu_device):
    """64 sequences of two blocks at the full projection depth (d = 7168,
    bf16, c = 512): 2 x 16 tiles of 128 x 128, so each call splits K over 8
    workgroups per tile (14 slabs each) and a reduce kernel adds them; both
    appends against the oracle."""
    case = synth.compressor_case("csa", [8] * 64, 7168, 512, 4, seed=6, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "bf16", in_place=True)
    assert row_rel_err(to64(out), ref).max() <= 2e-2


def test_append_uneven_split_and_partial_channel_tile(gpu_device):
    """20 sequences, c = 160 (5 channel tiles of 32, every one full) at
    d = 7168: 5 tiles split 32 ways, 3 or 4 of the 112 K slabs each, then
    fp8 output through the same partials."""
    case = synth.compressor_case("csa", [8] * 20, 7168, 160, 4, seed=8, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "bf16", in_place=False)
    assert row_rel_err(to64(out), ref).max() <= 2e-2
    q, s = _append_all(case, "fp8", in_place=True)
    check_fp8(q, s, ref, 2e-2)


def test_append_unsplit_many_tiles(gpu_device):
    """520 single-block sequences with c = 1024 make 9 x 16 = 144 tiles of
    256 x 256: the big-tile kernel runs the K loop whole in each tile."""
    case = synth.compressor_case("csa", [4] * 520, 64, 1024, 4, seed=7, in_dtype="f32", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "f32", in_place=False)
    assert max_abs_err(to64(out), ref) <= 2e-5


def test_append_skinny_unsplit(gpu_device):
    """400 single-block sequences at c = 512: 7 x 8 big tiles are too few,
    13 x 16 = 208 tiles of 128 x 128 run unsplit and the tile kernel
    finishes the entries itself (its odd-k-step waves added through LDS)."""
    case = synth.compressor_case("csa", [4] * 400, 64, 512, 4, seed=10, in_dtype="f32", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "f32", in_place=True)
    assert max_abs_err(to64(out), ref) <= 2e-5


def test_append_big_tile_split(gpu_device):
    """1024 single-block sequences at c = 512: 16 x 8 = 128 big tiles, K split
    2 ways (both K slabs of d = 64 fp32), then the big-tile reduce."""
    case = synth.compressor_case("csa", [4] * 1024, 64, 512, 4, seed=11, in_dtype="f32", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "f32", in_place=False)
    assert max_abs_err(to64(out), ref) <= 2e-5


@pytest.mark.parametrize("nseq", [1, 2])
def test_append_few_sequences_full_depth(gpu_device, nseq):
    """One or two sequences (the one-launch kernel with a wave per weight
    row) at d = 7168, bf16 operands, c = 512: fp32 entries against the
    oracle at 1e-5 of each row's largest entry (products exact in fp32, sums
    over 7168 terms), then bf16 entries in place and fp8 entries."""
    case = synth.compressor_case("csa", [12] * nseq, 7168, 512, 4, seed=20 + nseq, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "f32", in_place=False)
    err = row_rel_err(to64(out), ref).max()
    print(f"nseq={nseq}: fp32 entries from bf16 operands, max row-relative error {err:.3e}")
    assert err <= 1e-5
    out, _ = _append_all(case, "bf16", in_place=True)
    assert row_rel_err(to64(out), ref).max() <= 2 ** -8
    q, s = _append_all(case, "fp8", in_place=False)
    check_fp8(q, s, ref, 2 ** -8)


@pytest.mark.parametrize("nseq,d,c", [(1, 8192, 48), (2, 8192, 16), (2, 4160, 32)])
def test_append_few_sequences_fp32_pieces(gpu_device, nseq, d, c):
    """fp32 operands: a row of d = 8192 is two 16 KiB pieces (the second one
    full), d = 4160 two pieces with a ragged second (64 of 1024 chunks);
    c = 16 is a grid of 8 workgroups."""
    case = synth.compressor_case("csa", [8] * nseq, d, c, 4, seed=30 + d + c, in_dtype="f32", bias_std=0.5,
                                 device=gpu_device)
    ref = _oracle(case)
    out, _ = _append_all(case, "f32", in_place=nseq == 2)
    err = max_abs_err(to64(out), ref)
    print(f"nseq={nseq} d={d} c={c}: max abs error {err:.3e}")
    assert err <= 2e-5


def test_append_agrees_with_fused(gpu_device):
    """One append of every sequence's second block, fed the state of its first
    block, equals entry 1 of the fused compressor over the two blocks."""
    nseq, d, c = 9, 128, 48
    case = synth.compressor_case("csa", [8] * nseq, d, c, 4, seed=5, in_dtype="f32", bias_std=0.3,
                                 device=gpu_device)
    b = case.biases
    fused, _ = sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, case.cu_seqlens, "f32")
    H = case.H.view(nseq, 2, 4, d)
    e0, _, st = sc.csa_append(H[:, 0].reshape(-1, d).contiguous(), case.Wt_cat, b["Ba"], b["Bb"], None, "f32")
    e1, _, _ = sc.csa_append(H[:, 1].reshape(-1, d).contiguous(), case.Wt_cat, b["Ba"], b["Bb"], st, "f32")
    f = to64(fused).reshape(nseq, 2, c)
    assert max_abs_err(to64(e0), f[:, 0]) <= 2e-5
    assert max_abs_err(to64(e1), f[:, 1]) <= 2e-5
