"""GPU parity of the projection and the fused compressor against the oracle.

Tolerances (written per test):
* fp32 operands (16x16x4 fp32 MFMA, fp32 accumulation over d <= 128): an
  fp32 dot product of length d errs by at most ~d * 2^-24 * sum |h w|, which
  is below 2e-5 for these shapes; entries are convex combinations of such
  values, so max abs <= 2e-5;
* bf16 operands (bf16 MFMA, fp32 accumulation): per-row relative <= 2e-2;
* fp8 output: one E4M3 step on top of the bf16 path error (tests/helpers.py).
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, max_abs_err, row_rel_err, check_fp8, sample_entries, entry_owner

pytestmark = pytest.mark.gpu


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


def _oracle_sampled(case, idx):
    """Oracle value of the packed entries `idx`, projecting only the rows each reads."""
    W = _W64(case)
    b = {k: to64(v) for k, v in case.biases.items()}
    seq, loc = entry_owner(case.cu_seqlens, case.m, idx)
    rows = []
    m = case.m
    for s, i in zip(seq, loc):
        t0 = int(case.cu_seqlens[s])
        if case.mode == "csa":
            lo = max(i - 1, 0) * m
            H = to64(case.H[t0 + lo:t0 + (i + 1) * m])
            k = i - lo // m
            rows.append(oracle.csa_compress_sequence(H, W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], b["Ba"], b["Bb"],
                                                     m, k, k + 1))
        else:
            H = to64(case.H[t0 + i * m:t0 + (i + 1) * m])
            rows.append(oracle.hca_compress_sequence(H, W["W_KV"], W["W_Z"], b["B"], m))
    return np.concatenate(rows)


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
    """CSA tiny workload (n=64, d=64, c=32, m=4 -> 16 entries, fp32): max abs <= 2e-5."""
    cfg = synth.CONFIGS["csa_tiny"]
    case = synth.compressor_case("csa", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0, in_dtype="f32",
                                 bias_std=cfg["bias_std"], device=gpu_device)
    out, scale = _run(case, "f32")
    ref = _oracle_full(case)
    assert out.shape == (16, 32) and scale is None
    assert max_abs_err(to64(out), ref) <= 2e-5


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


def test_fused_zero_entries(gpu_device):
    """A batch whose sequences are all shorter than m gives an empty result."""
    case = synth.compressor_case("hca", [100, 27], 64, 32, 128, in_dtype="f32", device=gpu_device)
    out, _ = _run(case, "bf16")
    assert out.shape == (0, 32)


# -------------------------------------------------------------- fused, bf16

@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_fused_bf16_matches_unfused(gpu_device, mode):
    """bf16 fused vs the oracle (all entries) and vs the unfused path
    (project, then pool on column slices): per-row relative <= 2e-2."""
    lengths = [1000, 4, 777] if mode == "csa" else [1280, 200, 300]
    m = 4 if mode == "csa" else 128
    d, c = 256, 128
    case = synth.compressor_case(mode, lengths, d, c, m, seed=4, in_dtype="bf16", bias_std=0.3, device=gpu_device)
    ref = _oracle_full(case)
    out, _ = _run(case, "bf16")
    assert row_rel_err(to64(out), ref).max() <= 2e-2
    Y = sc.project(case.H, case.Wt_cat, "bf16")
    b = case.biases
    if mode == "csa":
        un, _ = sc.pool_csa(Y[:, :c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:], b["Ba"], b["Bb"], m,
                            case.cu_seqlens, "bf16")
    else:
        un, _ = sc.pool_hca(Y[:, :c], Y[:, c:], b["B"], m, case.cu_seqlens, "bf16")
    assert row_rel_err(to64(un), ref).max() <= 2e-2


def test_csa_full_config_sampled(gpu_device):
    """CSA full workload: n=8192, d=7168, c=512, m=4 -> 2048 entries, bf16.
    Sampled entries (every tile boundary of the first tiles, first, last,
    random) against the oracle: per-row relative <= 2e-2."""
    cfg = synth.CONFIGS["csa_full"]
    case = synth.compressor_case("csa", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0,
                                 in_dtype="bf16", bias_std=cfg["bias_std"], device=gpu_device)
    out, _ = _run(case, "bf16")
    assert out.shape == (2048, 512)
    idx = sample_entries(2048, 24, seed=9, must=(0, 1, 31, 32, 63, 64, 65, 127, 128, 2047))
    ref = _oracle_sampled(case, idx)
    got = to64(out[torch.from_numpy(idx).to(gpu_device)])
    rel = row_rel_err(got, ref)
    assert rel.max() <= 2e-2, rel.max()


def test_hca_full_config_sampled(gpu_device):
    """HCA workload: n=131072, d=7168, c=512, m'=128 -> 1024 entries, bf16."""
    cfg = synth.CONFIGS["hca_full"]
    case = synth.compressor_case("hca", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0,
                                 in_dtype="bf16", bias_std=cfg["bias_std"], device=gpu_device)
    out, _ = _run(case, "bf16")
    assert out.shape == (1024, 512)
    idx = sample_entries(1024, 6, seed=10, must=(0, 1, 2, 1023))
    ref = _oracle_sampled(case, idx)
    got = to64(out[torch.from_numpy(idx).to(gpu_device)])
    assert row_rel_err(got, ref).max() <= 2e-2


def test_varlen_fp8_config_sampled(gpu_device):
    """Batched variable-length workload: 32 sequences (lengths uniform in
    [4096, 65536] in steps of 128; seed 0 gives T = 968,960), d=7168, c=512,
    fused CSA (242,240 entries) and HCA (7,570 entries) with 1% of the Z
    channels scaled x30, fp8 E4M3 output with per-entry scales.  Sampled
    entries (each sequence's entry 0 and its first tile boundary, random):
    scale within 2e-2 and one E4M3 step on top of 2e-2 * max |ref|."""
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
        must = list(starts) + (list(starts + 64) if mode == "csa" else [])   # entry 64: second tile of a sequence
        idx = sample_entries(E, 16, seed=11, must=must)
        ref = _oracle_sampled(case, idx)
        sel = torch.from_numpy(idx).to(gpu_device)
        check_fp8(q[sel], s[sel], ref, path_rel=2e-2)
        del case, q, s
        torch.cuda.empty_cache()
