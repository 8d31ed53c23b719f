"""GPU parity of the projection and the fused compressor against the oracle.

Tolerances (written per test):
* fp32 operands (16x16x4 fp32 MFMA, fp32 accumulation over d <= 128): an
  fp32 dot product of length d errs by at most ~d * 2^-24 * sum |h w|, which
  is below 2e-5 for these shapes; entries are convex combinations of such
  values, so max abs <= 2e-5;
* the tiny CSA workload (fp32, d = 64): max abs <= 1e-5, its stated bar;
* bf16 operands (bf16 MFMA, fp32 accumulation): per-row relative <= 2e-2,
  and <= 2^-8 for the fused path (see BF16_OBSERVED);
* fp8 output: one E4M3 step on top of the bf16 path error (tests/helpers.py),
  and the encoder's codes equal to the oracle encoder's on the kernel's own
  fp32 entries except at rounding midpoints.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import (to64, max_abs_err, row_rel_err, check_fp8, fused_round_xcd_samples, oracle_entries, fp8_codes_match_encoder)

pytestmark = pytest.mark.gpu

# A bf16-operand entry is an fp32-accumulated value rounded once to bf16
# (relative 2^-9); the fp32 sums of exact bf16 products add ~1e-6.  The bf16
# paths are held to the stated 2e-2 per-row bar AND to this 2^-8 bound of the
# arithmetic itself, so that a logic error too small for 2e-2 (a dropped
# bias of std 0.02 moves entries by ~1%) still fails.
BF16_OBSERVED = 2.0 ** -8


def _W64(case):
    return {k: to64(v) for k, v in case.W.items()}


def _oracle_full(case):
    H = to64(case.H)
    W = _W64(case)
    b = {k: to64(v) for k, v in case.biases.items()}
    if case.mode == "csa":
        return oracle.csa_compress(H, W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], b["Ba"], b["Bb"], case.m,
                                   case.cu_seqlens)
    return oracle.hca_compress(H, W["W_KV"], W["W_Z"], b["B"], case.m, case.cu_seqlens)


def _run(case, out_dtype):
    b = case.biases
    if case.mode == "csa":
        return sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], case.m, case.cu_seqlens, out_dtype)
    return sc.compress_fused("hca", case.H, case.Wt_cat, b["B"], None, case.m, case.cu_seqlens, out_dtype)


# ------------------------------------------------------------------ project

@pytest.mark.parametrize("T,d,n_out", [(300, 128, 96), (64, 64, 128), (513, 192, 272)])
def test_project_fp32(gpu_device, T, d, n_out):
    """fp32 projection: max abs <= 2e-5 (fp32 accumulation over d <= 192)."""
    H = synth.normal((T, d), 1.0, (7, 1), gpu_device, "f32")
    Wt = synth.normal((n_out, d), 1.0 / np.sqrt(d), (7, 2), gpu_device, "f32")
    Y = sc.project(H, Wt, "f32")
    ref = oracle.project(to64(H), to64(Wt).T)
    assert max_abs_err(to64(Y), ref) <= 2e-5


def test_project_bf16_ragged(gpu_device):
    """bf16 projection, ragged T and N, bf16 and fp32 outputs: per-row relative <= 2e-2."""
    T, d, n_out = 1000, 512, 2048 + 16
    H = synth.normal((T, d), 1.0, (8, 1), gpu_device, "bf16")
    Wt = synth.normal((n_out, d), 1.0 / np.sqrt(d), (8, 2), gpu_device, "bf16")
    ref = oracle.project(to64(H), to64(Wt).T)
    for od in ("f32", "bf16"):
        Y = sc.project(H, Wt, od)
        rel = row_rel_err(to64(Y), ref)
        assert rel.max() <= 2e-2, (od, rel.max())
    Y = sc.project(H, Wt, "f32")
    assert row_rel_err(to64(Y), ref).max() <= 1e-5      # exact bf16 products, fp32 sums


@pytest.mark.parametrize("od", ["f32", "bf16"])
def test_project_into_padded_rows(gpu_device, od):
    """Y as the left columns of a wider buffer (row stride > n_out), ragged T
    and n_out: the padding columns and the rows past T keep their sentinel."""
    T, d, n_out, ld = 300, 128, 272, 272 + 56
    H = synth.normal((T, d), 1.0, (9, 1), gpu_device, "bf16")
    Wt = synth.normal((n_out, d), 1.0 / np.sqrt(d), (9, 2), gpu_device, "bf16")
    buf = torch.full((T + 5, ld), 7.0, dtype=torch.float32 if od == "f32" else torch.bfloat16, device=gpu_device)
    Y = sc.project(H, Wt, od, out=buf[:T, :n_out])
    ref = oracle.project(to64(H), to64(Wt).T)
    assert row_rel_err(to64(Y), ref).max() <= 2e-2
    assert bool((buf[:T, n_out:] == 7.0).all()) and bool((buf[T:] == 7.0).all())


# -------------------------------------------------------------- fused, fp32

def test_fused_csa_tiny_config(gpu_device):
    """CSA tiny workload (n=64, d=64, c=32, m=4 -> 16 entries, fp32 in and
    out): max abs <= 1e-5, the bar stated for this workload.  An fp32 dot
    product over d = 64 errs by ~1e-7 here; the observed error is printed."""
    cfg = synth.CONFIGS["csa_tiny"]
    case = synth.compressor_case("csa", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0, in_dtype="f32",
                                 bias_std=cfg["bias_std"], device=gpu_device)
    out, scale = _run(case, "f32")
    ref = _oracle_full(case)
    assert out.shape == (16, 32) and scale is None
    err = max_abs_err(to64(out), ref)
    print(f"csa_tiny: max abs err {err:.3e} (bar 1e-5)")
    assert err <= 1e-5


@pytest.mark.parametrize("mode,lengths,d,c", [
    ("csa", [700, 3, 260, 1025, 4], 128, 80),       # several tiles per sequence, partial N tile, halo fix-up
    ("csa", [256, 256, 512], 64, 64),                # tile-aligned sequences
    ("hca", [600, 100, 1000, 384], 128, 144),        # partial tiles, dropped tails, partial N tile
    ("hca", [128], 64, 16),
])
def test_fused_fp32_multitile(gpu_device, mode, lengths, d, c):
    """fp32 fused path over packed batches with ragged tiles: max abs <= 2e-5."""
    m = 4 if mode == "csa" else 128
    case = synth.compressor_case(mode, lengths, d, c, m, seed=3, in_dtype="f32", bias_std=0.5, device=gpu_device)
    out, _ = _run(case, "f32")
    ref = _oracle_full(case)
    assert out.shape == ref.shape
    assert max_abs_err(to64(out), ref) <= 2e-5


@pytest.mark.parametrize("mode,lengths,d,c", [
    ("csa", [700, 3, 260, 1025, 4], 128, 80),       # two K slabs, halo fix-up, partial N tile
    ("csa", [256, 256, 512], 64, 64),                # one K slab, tile-aligned sequences
    ("csa", [513, 1, 300], 320, 192),                # five K slabs, three N tiles
    ("hca", [600, 100, 1000, 384], 128, 144),        # partial tiles, dropped tails, partial N tile
    ("hca", [128, 256], 320, 32),
])
def test_fused_bf16_operands_multitile(gpu_device, mode, lengths, d, c):
    """bf16 operands, fp32 entries, packed batches with ragged tiles.  bf16
    products are exact in fp32 and the oracle takes the same bf16 values, so
    only the fp32 accumulation over d <= 320 differs: max abs <= 2e-5, as for
    fp32 operands (bias std 0.5, so a slip in the epilogue's bias or block
    bookkeeping cannot hide)."""
    m = 4 if mode == "csa" else 128
    case = synth.compressor_case(mode, lengths, d, c, m, seed=5, in_dtype="bf16", bias_std=0.5, device=gpu_device)
    out, _ = _run(case, "f32")
    ref = _oracle_full(case)
    assert out.shape == ref.shape
    err = max_abs_err(to64(out), ref)
    print(f"{mode} bf16 operands d={d} c={c}: max abs err {err:.3e}")
    assert err <= 2e-5


@pytest.mark.parametrize("mode,lengths", [("csa", [517, 260]), ("hca", [640, 300])])
def test_fused_wide_and_deep(gpu_device, mode, lengths):
    """c = 2048 channels (CSA: 32 N tiles; HCA: 16 channel slices of 128) and
    d = 8192 (128 K slabs), bf16 operands, fp32 entries.  Each projected
    value sums 8192 exact bf16 products in fp32; with unit-variance values
    the accumulation errs by ~2^-24 * sqrt(8192) ~ 5e-6 (observed 3-5e-6),
    so max abs <= 5e-5 holds with a tenfold margin while a slip in the bias or block bookkeeping (bias
    std 0.5) moves entries by ~0.1."""
    m = 4 if mode == "csa" else 128
    case = synth.compressor_case(mode, lengths, 8192, 2048, m, seed=9, in_dtype="bf16", bias_std=0.5,
                                 device=gpu_device)
    out, _ = _run(case, "f32")
    ref = _oracle_full(case)
    assert out.shape == ref.shape
    err = max_abs_err(to64(out), ref)
    print(f"{mode} c=2048 d=8192: max abs err {err:.3e}")
    assert err <= 5e-5


@pytest.mark.parametrize("T,d,n_out", [(300, 128, 96), (513, 320, 272), (64, 64, 512)])
def test_project_bf16_operands_f32_out(gpu_device, T, d, n_out):
    """bf16 projection with fp32 output against the float64 product of the same
    bf16 values: max abs <= 2e-5 (exact products, fp32 sums over d <= 320);
    ragged M and N tiles and one to five K slabs."""
    H = synth.normal((T, d), 1.0, (12, 1), gpu_device, "bf16")
    Wt = synth.normal((n_out, d), 1.0 / np.sqrt(d), (12, 2), gpu_device, "bf16")
    Y = sc.project(H, Wt, "f32")
    ref = oracle.project(to64(H), to64(Wt).T)
    assert Y.shape == (T, n_out)
    assert max_abs_err(to64(Y), ref) <= 2e-5


def test_fused_zero_entries(gpu_device):
    """A batch whose sequences are all shorter than m gives an empty result."""
    case = synth.compressor_case("hca", [100, 27], 64, 32, 128, in_dtype="f32", device=gpu_device)
    out, _ = _run(case, "bf16")
    assert out.shape == (0, 32)


# -------------------------------------------------------------- fused, bf16

@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_fused_bf16_matches_unfused(gpu_device, mode):
    """bf16 fused vs the oracle (all entries): per-row relative <= 2e-2 and
    <= 2^-8 observed; the unfused path (project to bf16, then pool on column
    slices; the bf16 rounding of the logits adds its own error): <= 2e-2."""
    lengths = [1000, 4, 777] if mode == "csa" else [1280, 200, 300]
    m = 4 if mode == "csa" else 128
    d, c = 256, 128
    case = synth.compressor_case(mode, lengths, d, c, m, seed=4, in_dtype="bf16", bias_std=0.3, device=gpu_device)
    ref = _oracle_full(case)
    out, _ = _run(case, "bf16")
    rel = row_rel_err(to64(out), ref)
    assert rel.max() <= 2e-2 and rel.max() <= BF16_OBSERVED
    Y = sc.project(case.H, case.Wt_cat, "bf16")
    b = case.biases
    if mode == "csa":
        un, _ = sc.pool_csa(Y[:, :c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:], b["Ba"], b["Bb"], m,
                            case.cu_seqlens, "bf16")
    else:
        un, _ = sc.pool_hca(Y[:, :c], Y[:, c:], b["B"], m, case.cu_seqlens, "bf16")
    assert row_rel_err(to64(un), ref).max() <= 2e-2


def _n_cu(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def test_csa_full_config_all_entries(gpu_device):
    """CSA full workload: n=8192, d=7168, c=512, m=4 -> 2048 entries, bf16.
    Every entry against the oracle (the launch is one persistent round of
    256 tiles): per-row relative <= 2e-2, and <= 2^-8 observed."""
    cfg = synth.CONFIGS["csa_full"]
    case = synth.compressor_case("csa", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0,
                                 in_dtype="bf16", bias_std=cfg["bias_std"], device=gpu_device)
    out, _ = _run(case, "bf16")
    assert out.shape == (2048, 512)
    ref = _oracle_full(case)
    rel = row_rel_err(to64(out), ref)
    print(f"csa_full: all 2048 entries, max per-row rel err {rel.max():.3e}")
    assert rel.max() <= 2e-2
    assert rel.max() <= BF16_OBSERVED


def test_hca_full_config_every_round_and_xcd(gpu_device):
    """HCA workload: n=131072, d=7168, c=512, m'=128 -> 1024 entries, bf16.
    Entries from every (persistent round, XCD) pair of the launch, and every
    entry of the first and last rounds' tiles: per-row relative <= 2e-2 and
    <= 2^-8 observed."""
    cfg = synth.CONFIGS["hca_full"]
    case = synth.compressor_case("hca", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0,
                                 in_dtype="bf16", bias_std=cfg["bias_std"], device=gpu_device)
    out, _ = _run(case, "bf16")
    assert out.shape == (1024, 512)
    idx = fused_round_xcd_samples(case.cu_seqlens, case.m, "hca", case.c, _n_cu(gpu_device), seed=10)
    ref = oracle_entries(case, idx)
    got = to64(out[torch.from_numpy(idx).to(gpu_device)])
    rel = row_rel_err(got, ref)
    print(f"hca_full: {idx.size} sampled entries, max per-row rel err {rel.max():.3e}")
    assert rel.max() <= 2e-2
    assert rel.max() <= BF16_OBSERVED


def test_varlen_fp8_config_every_round_and_xcd(gpu_device):
    """Batched variable-length workload: 32 sequences (lengths uniform in
    [4096, 65536] in steps of 128; seed 0 gives T = 968,960), d=7168, c=512,
    fused CSA (242,240 entries) and HCA (7,570 entries) with 1% of the Z
    channels scaled x30, fp8 E4M3 output with per-entry scales.  Entries from
    every (persistent round, XCD) pair of each launch, every tile boundary of
    the first and last rounds and every sequence's entry 0: scale within 2e-2
    and one E4M3 step on top of 2e-2 * max |ref|.  The same launch with fp32
    output must give codes identical to the oracle's encoder on those fp32
    entries (except at rounding midpoints)."""
    cfg = synth.CONFIGS["varlen_fp8"]
    lengths = synth.varlen_config_lengths(0)
    assert int(lengths.sum()) == 968960
    for mode, m in (("csa", cfg["m_csa"]), ("hca", cfg["m_hca"])):
        case = synth.compressor_case(mode, lengths, cfg["d"], cfg["c"], m, seed=0, in_dtype="bf16",
                                     bias_std=cfg["bias_std"], device=gpu_device,
                                     z_outlier_frac=cfg["z_outlier_frac"], z_outlier_scale=cfg["z_outlier_scale"],
                                     per_sequence_h=True)
        q, s = _run(case, "fp8")
        E = case.n_entries
        assert q.shape == (E, 512) and s.shape == (E,)
        counts = np.diff(case.cu_seqlens) // m
        starts = np.concatenate([[0], np.cumsum(counts)])[:-1]
        idx = np.union1d(fused_round_xcd_samples(case.cu_seqlens, m, mode, case.c, _n_cu(gpu_device), seed=11),
                         starts[counts > 0])
        ref = oracle_entries(case, idx)
        sel = torch.from_numpy(idx).to(gpu_device)
        srel, excess = check_fp8(q[sel], s[sel], ref, path_rel=2e-2)
        f32, _ = _run(case, "f32")
        n, mids = fp8_codes_match_encoder(q[sel].cpu().numpy(), s[sel].cpu().numpy(), to64(f32[sel]))
        rel = row_rel_err(to64(f32[sel]), ref)
        print(f"varlen {mode}: {idx.size} sampled entries; fp32 entries max per-row rel err {rel.max():.3e}; "
              f"fp8 scale rel err {srel:.3e}; {n} codes, {mids} at rounding midpoints")
        assert rel.max() <= 2e-2 and rel.max() <= BF16_OBSERVED
        del case, q, s, f32
        torch.cuda.empty_cache()


@pytest.mark.parametrize("mode,out_dtype", [("csa", "bf16"), ("csa", "fp8"), ("hca", "bf16")])
def test_planned_and_looked_up_tiles_agree(gpu_device, mode, out_dtype):
    """Batches of up to 64 sequences find their tiles from the offsets inside
    the kernels; larger ones take the planner's table.  70 sequences in one
    call (planner) give bit for bit the entries (and fp8 scales) of the same
    sequences in two calls of 64 and 6 (looked up): ragged lengths, empty
    and shorter-than-m sequences, tile-aligned ones."""
    m = 4 if mode == "csa" else 128
    rng = np.random.default_rng(70)
    lengths = rng.integers(0, 1600 if mode == "csa" else 3000, size=70)
    lengths[[3, 17]] = 0
    lengths[[5, 40]] = m - 1
    lengths[[8, 66]] = 512
    case = synth.compressor_case(mode, lengths, 64, 32, m, seed=71, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    b = case.biases
    Ba, Bb = (b["Ba"], b["Bb"]) if mode == "csa" else (b["B"], None)
    cu = np.asarray(case.cu_seqlens, dtype=np.int64)
    whole = sc.compress_fused(mode, case.H, case.Wt_cat, Ba, Bb, m, cu, out_dtype)
    parts = [sc.compress_fused(mode, case.H, case.Wt_cat, Ba, Bb, m, cu[:65], out_dtype),
             sc.compress_fused(mode, case.H[cu[64]:], case.Wt_cat, Ba, Bb, m, cu[64:] - cu[64], out_dtype)]
    assert torch.equal(whole[0], torch.cat([parts[0][0], parts[1][0]]))
    if out_dtype == "fp8":
        assert torch.equal(whole[1], torch.cat([parts[0][1], parts[1][1]]))
    if out_dtype == "bf16":
        assert row_rel_err(to64(whole[0]), _oracle_full(case)).max() <= BF16_OBSERVED


@pytest.mark.parametrize("mode,out_dtype", [("csa", "f32"), ("csa", "fp8"), ("hca", "bf16"), ("hca", "fp8")])
def test_sequence_results_independent_of_packing(gpu_device, mode, out_dtype):
    """No kernel communicates between workgroups (the CSA halo is merged by a
    separate launch), so the order in which the persistent grid visits tiles
    cannot change a result.  Tiles never cross sequences, so sequence A is cut
    into the same tiles whether it is packed alone or after other sequences,
    which moves its tiles to other workgroups, XCDs and rounds: its entries
    (and fp8 scales) must be identical bit for bit, and the pooling call's
    too."""
    m = 4 if mode == "csa" else 128
    d, c = 256, 128
    la = 3000 if mode == "csa" else 6400
    lengths_alone, lengths_packed = [la], [1000, 777, 1536, la, 300]
    cases = [synth.compressor_case(mode, L, d, c, m, seed=70, in_dtype="bf16", bias_std=0.3, device=gpu_device)
             for L in (lengths_alone, lengths_packed)]
    A_rows = slice(sum(lengths_packed[:3]), sum(lengths_packed[:4]))
    # the packed case's sequence A gets the alone case's rows and weights
    packed = cases[1]
    packed.H[A_rows] = cases[0].H
    packed.Wt_cat.copy_(cases[0].Wt_cat)
    for k in packed.biases:
        packed.biases[k].copy_(cases[0].biases[k])
    alone_out, alone_scale = _run(cases[0], out_dtype)
    packed_out, packed_scale = _run(packed, out_dtype)
    e0 = sum(L // m for L in lengths_packed[:3])
    E = la // m
    assert torch.equal(packed_out[e0:e0 + E], alone_out)
    if out_dtype == "fp8":
        assert torch.equal(packed_scale[e0:e0 + E], alone_scale)
    # the pooling call on the projected streams, same check
    Ys = [sc.project(cs.H, cs.Wt_cat, "bf16") for cs in (cases[0], packed)]
    b = cases[0].biases
    if mode == "csa":
        pools = [sc.pool_csa(Y[:, :c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:], b["Ba"], b["Bb"], m, cs.cu_seqlens,
                             "bf16")[0] for Y, cs in zip(Ys, (cases[0], packed))]
    else:
        pools = [sc.pool_hca(Y[:, :c], Y[:, c:], b["B"], m, cs.cu_seqlens, "bf16")[0]
                 for Y, cs in zip(Ys, (cases[0], packed))]
    assert torch.equal(pools[1][e0:e0 + E], pools[0])
