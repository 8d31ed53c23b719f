"""GPU parity of the pooling-only calls against the float64 oracle.

Tolerances: fp32 in / fp32 out max abs <= 1e-5; bf16 paths per-row relative
<= 2e-2 (bf16 output adds at most half a bf16 step, 2^-9 relative); fp8 one
E4M3 step on top of the path error (see tests/helpers.py).
"""

import numpy as np
import pytest
import torch

import oracle
import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth
from helpers import to64, max_abs_err, row_rel_err, check_fp8, sample_entries, fp8_codes_match_encoder

pytestmark = pytest.mark.gpu


def _oracle_csa(case, cu):
    s = {k: to64(v) for k, v in case.streams.items()}
    return oracle.csa_pool(s["Ca"], s["Cb"], s["Za"], s["Zb"], to64(case.biases["Ba"]), to64(case.biases["Bb"]),
                           case.m_csa, cu)


def _oracle_hca(case, cu):
    s = {k: to64(v) for k, v in case.streams.items()}
    return oracle.hca_pool(s["Ca"], s["Za"], to64(case.biases["B"]), case.m_hca, cu)


def _dev(case, device):
    for k in case.streams:
        case.streams[k] = case.streams[k].to(device)
    for k in case.biases:
        case.biases[k] = case.biases[k].to(device)
    return case


@pytest.mark.parametrize("lengths,c,m_csa,m_hca", [
    ([64], 32, 4, 128),                          # tiny: fewer rows than one HCA block
    ([256 * 3 + 4 * 5 + 3], 48, 4, 128),          # several tiles, ragged tail, c/8 = 6 vectors
    ([5, 0, 3, 4, 257, 1000, 64, 129], 32, 4, 8), # packed batch: empty / shorter-than-m sequences
    ([1031], 16, 1, 1),                           # degenerate m = 1
    ([997], 64, 3, 5),                            # m that does not divide the tile
    ([2048 + 7], 512, 16, 256),                   # c = 512, larger m
    ([1500], 192, 4, 96),                         # c = 192: several HCA channel slices, m = 96
    ([700, 9, 300], 2048, 4, 128),                # c = 2048: four CSA slices of 512, 32 HCA slices
])
def test_pool_fp32_exact(gpu_device, lengths, c, m_csa, m_hca):
    """fp32 streams, fp32 output: max abs error <= 1e-5 against the oracle."""
    case = _dev(synth.pool_case(sum(lengths), c, m_csa=m_csa, m_hca=m_hca, seed=1, dtype="f32",
                                bias_std=0.5, lengths=lengths, z_std=2.0), gpu_device)
    cu = case.cu_seqlens
    st = case.streams
    out, scale = sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], case.biases["Ba"], case.biases["Bb"],
                             m_csa, cu, "f32")
    assert scale is None
    ref = _oracle_csa(case, cu)
    assert out.shape == ref.shape
    assert max_abs_err(to64(out), ref) <= 1e-5
    outh, _ = sc.pool_hca(st["Ca"], st["Za"], case.biases["B"], m_hca, cu, "f32")
    refh = _oracle_hca(case, cu)
    assert outh.shape == refh.shape
    assert max_abs_err(to64(outh), refh) <= 1e-5


def test_pool_bf16_and_fp8_outputs(gpu_device):
    """bf16 inputs; bf16 output within 2e-2 per row (observed ~2^-9), fp8 within one step."""
    lengths = [700, 1, 513]
    case = _dev(synth.pool_case(sum(lengths), 64, seed=2, dtype="bf16", lengths=lengths, bias_std=0.3),
                gpu_device)
    cu = case.cu_seqlens
    st = case.streams
    ref = _oracle_csa(case, cu)
    out, _ = sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], case.biases["Ba"], case.biases["Bb"], 4, cu, "bf16")
    rel = row_rel_err(to64(out), ref)
    assert rel.max() <= 2e-2 and rel.max() <= 2.0 ** -8
    q, s = sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], case.biases["Ba"], case.biases["Bb"], 4, cu, "fp8")
    check_fp8(q, s, ref, path_rel=0.0, path_abs=1e-5)
    refh = _oracle_hca(case, cu)
    qh, sh = sc.pool_hca(st["Ca"], st["Za"], case.biases["B"], 128, cu, "fp8")
    check_fp8(qh, sh, refh, path_rel=0.0, path_abs=1e-5)


def test_fp8_encoder_codes_match_oracle(gpu_device):
    """The fp8 encoder alone: fp32 streams pooled to fp32 and to fp8 by the
    same kernels; the codes must equal oracle.fp8_entry_quantize of the fp32
    entries exactly (except within 1e-6 relative of a rounding midpoint,
    where the two neighbours are allowed) and the scales must be within one
    fp32 ulp of max |x| / 448.  Entries span magnitudes 1e-3 to 1e3, one is
    all zero (scale 1, codes 0), and both CSA and HCA pooling are encoded."""
    n, c = 4 * 700, 96
    case = _dev(synth.pool_case(n, c, m_csa=4, m_hca=8, seed=7, dtype="f32", bias_std=0.5, z_std=2.0), gpu_device)
    st = case.streams
    mag = torch.from_numpy(10.0 ** np.random.default_rng(8).uniform(-3, 3, size=(n, 1))).float().to(gpu_device)
    for k in ("Ca", "Cb"):
        st[k] = (st[k] * mag).contiguous()
    st["Ca"][4 * 9:4 * 10] = 0.0          # entry 9 reads a-rows of block 9 and b-rows of block 8
    st["Cb"][4 * 8:4 * 9] = 0.0
    st["Ca"][8 * 5:8 * 6] = 0.0           # HCA (m' = 8) entry 5 is all zero
    b = case.biases
    for pool, args in (("csa", (st["Ca"], st["Cb"], st["Za"], st["Zb"], b["Ba"], b["Bb"], 4)),
                       ("hca", (st["Ca"], st["Za"], b["B"][:8].contiguous(), 8))):
        fn = sc.pool_csa if pool == "csa" else sc.pool_hca
        x, _ = fn(*args, None, "f32")
        q, s = fn(*args, None, "fp8")
        x64 = to64(x)
        zero = 9 if pool == "csa" else 5
        assert np.all(x64[zero] == 0) and float(s[zero]) == 1.0 and bool((q[zero] == 0).all())
        n_codes, mids = fp8_codes_match_encoder(q.cpu().numpy(), s.cpu().numpy(), x64)
        print(f"fp8 encoder ({pool} pool): {n_codes} codes identical to the oracle's, {mids} at rounding midpoints")


def test_pool_weights_sum_to_one(gpu_device):
    """Value streams of ones give entries of exactly one (weights sum to 1,
    entry 0 included), whatever the logits."""
    n, c = 1000, 32
    ones = torch.ones((n, c), dtype=torch.float32, device=gpu_device)
    Z = synth.normal((n, c), 5.0, (3, 1), gpu_device, "f32")
    Ba = synth.normal((4, c), 1.0, (3, 2), gpu_device, "f32")
    out, _ = sc.pool_csa(ones, ones, Z, Z, Ba, Ba, 4, None, "f32")
    assert torch.all(out == 1.0)
    out, _ = sc.pool_hca(ones, Z, synth.normal((128, c), 1.0, (3, 3), gpu_device, "f32"), 128, None, "f32")
    assert torch.all(out == 1.0)


def test_pool_zero_entries_and_slices(gpu_device):
    """n < m gives zero entries and no launch; streams may be column slices of
    one [T x 4c] projection output (ld_in = 4c)."""
    c = 32
    Y = synth.normal((3, 4 * c), 1.0, (4, 1), gpu_device, "f32")
    B = torch.zeros((4, c), device=gpu_device)
    out, _ = sc.pool_csa(Y[:, :c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:], B, B, 4, None, "f32")
    assert out.shape == (0, c)
    n = 1024 + 12
    Y = synth.normal((n, 4 * c), 1.0, (4, 2), gpu_device, "f32")
    Ba = synth.normal((4, c), 0.2, (4, 3), gpu_device, "f32")
    Bb = synth.normal((4, c), 0.2, (4, 4), gpu_device, "f32")
    out, _ = sc.pool_csa(Y[:, :c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:], Ba, Bb, 4, None, "f32")
    y = to64(Y)
    ref = oracle.csa_pool(y[:, :c], y[:, c:2 * c], y[:, 2 * c:3 * c], y[:, 3 * c:], to64(Ba), to64(Bb), 4)
    assert max_abs_err(to64(out), ref) <= 1e-5


def test_pool_long_context_full_size_sampled(gpu_device):
    """The long-context pooling workload at full size: four bf16 streams of
    1048576 x 512, CSA m=4 (262144 entries) and HCA m'=128 on (C^a, Z^a)
    (8192 entries); bf16 output.  Sampled entries (first, last, random)
    against the oracle, per-row relative <= 2e-2; plus the fp32 copy of the
    same streams at max abs <= 1e-5."""
    cfg = synth.CONFIGS["pool_long"]
    n, c = cfg["n"], cfg["c"]
    case = synth.pool_case(n, c, seed=0, dtype="bf16", device=gpu_device, bias_std=cfg["bias_std"])
    st, b = case.streams, case.biases
    cu = case.cu_seqlens
    out, _ = sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], b["Ba"], b["Bb"], 4, cu, "bf16")
    outh, _ = sc.pool_hca(st["Ca"], st["Za"], b["B"], 128, cu, "bf16")
    assert out.shape == (262144, c) and outh.shape == (8192, c)
    idx = sample_entries(262144, 256, seed=5, must=(0, 1, 3, 4, 63, 64, 2047, 2048, 262143))
    Ba, Bb = to64(b["Ba"]), to64(b["Bb"])
    got = to64(out[torch.from_numpy(idx).to(gpu_device)])
    for k, i in enumerate(idx):
        lo = max(i - 1, 0) * 4
        s = {nm: to64(st[nm][lo:(i + 1) * 4]) for nm in st}
        ref = oracle.csa_pool_sequence(s["Ca"], s["Cb"], s["Za"], s["Zb"], Ba, Bb, 4, i - lo // 4, i - lo // 4 + 1)
        assert row_rel_err(got[k:k + 1], ref).max() <= 2e-2, i
    idxh = sample_entries(8192, 16, seed=6, must=(0, 8191))
    # HCA entry i reads rows [128 i, 128 i + 127]
    goth = to64(outh[torch.from_numpy(idxh).to(gpu_device)])
    for k, i in enumerate(idxh):
        rows = slice(128 * i, 128 * (i + 1))
        ref = oracle.hca_pool_sequence(to64(st["Ca"][rows]), to64(st["Za"][rows]), to64(b["B"]), 128)
        assert row_rel_err(goth[k:k + 1], ref).max() <= 2e-2, i
    # fp32 copy of the same streams: <= 1e-5
    st32 = {k: v.float() for k, v in st.items()}
    del out, outh
    out32, _ = sc.pool_csa(st32["Ca"], st32["Cb"], st32["Za"], st32["Zb"], b["Ba"], b["Bb"], 4, cu, "f32")
    got = to64(out32[torch.from_numpy(idx).to(gpu_device)])
    for k, i in enumerate(idx):
        lo = max(i - 1, 0) * 4
        s = {nm: to64(st32[nm][lo:(i + 1) * 4]) for nm in st32}
        ref = oracle.csa_pool_sequence(s["Ca"], s["Cb"], s["Za"], s["Zb"], Ba, Bb, 4, i - lo // 4, i - lo // 4 + 1)
        assert max_abs_err(got[k:k + 1], ref) <= 1e-5, i


def test_offsets_of_equal_size_are_not_confused(gpu_device):
    """The binding keeps small device copies of the sequence offsets by
    content: two layouts with the same number of sequences, called in turn
    and then again, each give their own oracle result."""
    case = _dev(synth.pool_case(1200, 32, m_csa=4, m_hca=8, seed=2, dtype="f32", bias_std=0.5, z_std=2.0),
                gpu_device)
    st = case.streams
    layouts = [np.array([0, 400, 1200]), np.array([0, 804, 1200]), np.array([0, 400, 1200])]
    for cu in layouts:
        out, _ = sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], case.biases["Ba"], case.biases["Bb"], 4, cu,
                             "f32")
        ref = _oracle_csa(case, cu)
        assert out.shape == ref.shape
        assert max_abs_err(to64(out), ref) <= 1e-5
