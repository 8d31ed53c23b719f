"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test names what it pins and which page passage fixes the expected value.
A plausible mistake in the oracle (a dropped bias, a b-stream taken from the
wrong block, separate instead of joint normalisation, a missing boundary
mask, a missing max-subtraction, ceil instead of floor) fails at least one of
them; ``test_planted_mistakes_are_caught`` checks that claim on mutated copies.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import compressor as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- projection

def test_project_integer_exact():
    """eq. attn-seqcomp-csa-proj (序列压缩注意力): X = H W.  With small integers
    every float64 product and sum is exact, so the oracle must equal an
    integer triple loop bit for bit; a transposed operand changes the result."""
    rng = np.random.default_rng(1)
    H = rng.integers(-4, 5, size=(7, 5))
    W = rng.integers(-4, 5, size=(5, 3))
    ref = [[sum(int(H[i, k]) * int(W[k, j]) for k in range(5)) for j in range(3)] for i in range(7)]
    got = oracle.project(H.astype(float), W.astype(float))
    assert got.shape == (7, 3)
    assert np.array_equal(got, np.array(ref, dtype=float))
    with pytest.raises(ValueError):
        oracle.project(H.astype(float), W.T.astype(float))


# ------------------------------------------------------ exact rational pools

def _rational_csa_case(n, m, c, seed):
    """Z = ln k and B = ln b with positive integers, so exp(Z + B) = k * b."""
    rng = np.random.default_rng(seed)
    ka, kb = rng.integers(1, 10, size=(n, c)), rng.integers(1, 10, size=(n, c))
    ba, bb = rng.integers(1, 6, size=(m, c)), rng.integers(1, 6, size=(m, c))
    Ca, Cb = rng.integers(-9, 10, size=(n, c)), rng.integers(-9, 10, size=(n, c))
    return ka, kb, ba, bb, Ca, Cb


@pytest.mark.parametrize("n,m,c,seed", [(22, 4, 3, 0), (12, 4, 2, 1), (17, 3, 2, 2), (9, 2, 4, 3), (3, 4, 2, 4)])
def test_csa_pool_exact_rational(n, m, c, seed):
    """eq. attn-seqcomp-csa-softmax / -pool / -overlap-bound (序列压缩注意力).

    With exp(Z^a + B^a) = k^a b^a and exp(Z^b + B^b) = k^b b^b, entry i is the
    weighted mean sum(w C) / sum(w) over the a rows of block i and the b rows
    of block i-1 (joint normalisation), and over the a rows alone for i = 0.
    Evaluated in exact rationals."""
    ka, kb, ba, bb, Ca, Cb = _rational_csa_case(n, m, c, seed)
    got = oracle.csa_pool_sequence(Ca, Cb, np.log(ka), np.log(kb), np.log(ba), np.log(bb), m)
    E = n // m
    assert got.shape == (E, c)
    for i in range(E):
        for ch in range(c):
            num, den = Fraction(0), Fraction(0)
            for r in range(m):
                w = int(ka[m * i + r, ch]) * int(ba[r, ch])
                num += w * int(Ca[m * i + r, ch]); den += w
                if i >= 1:
                    w = int(kb[m * (i - 1) + r, ch]) * int(bb[r, ch])
                    num += w * int(Cb[m * (i - 1) + r, ch]); den += w
            ref = num / den
            assert abs(got[i, ch] - float(ref)) <= 1e-14 * max(1.0, abs(float(ref))), (i, ch)


@pytest.mark.parametrize("n,m,c,seed", [(29, 8, 3, 0), (128 * 2 + 5, 128, 2, 1), (7, 8, 2, 2)])
def test_hca_pool_exact_rational(n, m, c, seed):
    """eq. attn-seqcomp-hca (序列压缩注意力): entry i is the softmax-weighted mean
    of rows [m i, m(i+1)-1] of C with weights exp(Z + B) = k b; exact rationals."""
    rng = np.random.default_rng(seed)
    k = rng.integers(1, 10, size=(n, c)); b = rng.integers(1, 6, size=(m, c))
    C = rng.integers(-9, 10, size=(n, c))
    got = oracle.hca_pool_sequence(C, np.log(k), np.log(b), m)
    E = n // m
    assert got.shape == (E, c)
    for i in range(E):
        for ch in range(c):
            ws = [int(k[m * i + r, ch]) * int(b[r, ch]) for r in range(m)]
            ref = Fraction(sum(w * int(C[m * i + r, ch]) for r, w in enumerate(ws)), sum(ws))
            assert abs(got[i, ch] - float(ref)) <= 1e-14 * max(1.0, abs(float(ref)))


# ----------------------------------------------------------- closed forms

def _rand_streams(n, c, seed, zscale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, c)) * s for s in (1.0, 1.0, zscale, zscale)]


def test_weights_sum_to_one():
    """The softmax weights of a window sum to 1 ("Ch 05 · HCA" section 2: each
    segment's weights sum to 1, the entry is a convex combination): with
    every value row equal to 1 every entry is exactly 1, entry 0 included."""
    n, c, m = 40, 5, 4
    _, _, Za, Zb = _rand_streams(n, c, 3, 3.0)
    rng = np.random.default_rng(4)
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    ones = np.ones((n, c))
    assert np.allclose(oracle.csa_pool_sequence(ones, ones, Za, Zb, Ba, Bb, m), 1.0, atol=1e-15, rtol=0)
    assert np.allclose(oracle.hca_pool_sequence(ones, Za, rng.standard_normal((8, c)), 8), 1.0, atol=1e-15, rtol=0)


def test_mean_pool_special_case():
    """Constant Z with B = 0 turns the learned pooling into the plain segment
    mean ("Ch 04 · CSA" section 3 names the naive compressor: floor(n/m)
    segments, each a simple average).  CSA entry i >= 1 is the mean of its 2m
    rows, entry 0 the mean of its m a-rows; HCA is reshape(E, m, c).mean(1)."""
    n, c, m = 4 * 9 + 3, 6, 4
    Ca, Cb, _, _ = _rand_streams(n, c, 5)
    Z = np.full((n, c), 0.37)
    zero = np.zeros((m, c))
    got = oracle.csa_pool_sequence(Ca, Cb, Z, Z, zero, zero, m)
    E = n // m
    a = Ca[:E * m].reshape(E, m, c)
    b = Cb[:(E - 1) * m].reshape(E - 1, m, c)
    ref = np.empty((E, c))
    ref[0] = a[0].mean(axis=0)
    ref[1:] = np.concatenate([a[1:], b], axis=1).mean(axis=1)
    assert np.allclose(got, ref, atol=1e-14, rtol=0)
    mh = 8
    got_h = oracle.hca_pool_sequence(Ca, Z, np.zeros((mh, c)), mh)
    ref_h = Ca[:(n // mh) * mh].reshape(n // mh, mh, c).mean(axis=1)
    assert np.allclose(got_h, ref_h, atol=1e-14, rtol=0)


def test_entry0_is_pure_a_stream():
    """eq. attn-seqcomp-overlap-bound (序列压缩注意力): entry 0's b rows have
    logit -inf and vector 0, so entry 0 is the single-stream compression of
    block 0 with B^a and does not depend on any b input."""
    n, c, m = 24, 4, 4
    Ca, Cb, Za, Zb = _rand_streams(n, c, 6, 2.0)
    rng = np.random.default_rng(7)
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    base = oracle.csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m)
    pert = oracle.csa_pool_sequence(Ca, Cb + 5.0, Za, Zb - 3.0, Ba, Bb * 7.0, m)
    assert np.array_equal(base[0], pert[0])
    single = oracle.hca_pool_sequence(Ca[:m], Za[:m], Ba, m)
    assert np.allclose(base[0], single[0], atol=1e-15, rtol=0)


def _parse_worked_example():
    spec = {"map": {}}
    with open(os.path.join(GOLDEN, "csa_worked_example_n12_m4.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] in ("n", "m", "entries"):
                spec["count" if tok[0] == "entries" else tok[0]] = int(tok[1])
            elif tok[0] == "entry":
                i = int(tok[1])
                a = tuple(int(x) for x in tok[3].split(".."))
                b = None if tok[5] == "none" else tuple(int(x) for x in tok[5].split(".."))
                spec["map"][i] = (a, b)
            elif tok[0] == "token":
                spec["token"] = (int(tok[1]), int(tok[3]), int(tok[5]))
    return spec


def test_footprint_matches_worked_example():
    """"Ch 04 · CSA" section 3 worked example (golden fixture): with n = 12 and
    m = 4, entry 0 reads a-rows 0..3 only, entry 1 a 4..7 and b 0..3, entry 2
    a 8..11 and b 4..7; token 4 reaches entry 1 via a and entry 2 via b.
    Perturbing one input row must change exactly the entries listed."""
    spec = _parse_worked_example()
    n, m, c = spec["n"], spec["m"], 3
    Ca, Cb, Za, Zb = _rand_streams(n, c, 8)
    Ba, Bb = np.full((m, c), 0.1), np.full((m, c), -0.2)
    base = oracle.csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m)
    assert base.shape[0] == spec["count"] == len(spec["map"]) == 3

    def touched(stream, row):
        arrs = {"Ca": Ca.copy(), "Cb": Cb.copy(), "Za": Za.copy(), "Zb": Zb.copy()}
        arrs[stream][row] += 0.75
        out = oracle.csa_pool_sequence(arrs["Ca"], arrs["Cb"], arrs["Za"], arrs["Zb"], Ba, Bb, m)
        return {i for i in range(out.shape[0]) if not np.array_equal(out[i], base[i])}

    for row in range(n):
        exp_a = {i for i, (a, _) in spec["map"].items() if a[0] <= row <= a[1]}
        exp_b = {i for i, (_, b) in spec["map"].items() if b is not None and b[0] <= row <= b[1]}
        assert touched("Ca", row) == exp_a and touched("Za", row) == exp_a, row
        assert touched("Cb", row) == exp_b and touched("Zb", row) == exp_b, row
    tok, ea, eb = spec["token"]
    assert touched("Ca", tok) == {ea} and touched("Cb", tok) == {eb}


def _dense_window_pool(V, L, windows):
    """Brute force: per channel, an (E x rows) weight matrix from torch's float64
    softmax over each entry's window (other rows masked to -inf), times V."""
    E = len(windows)
    n, c = V.shape
    out = np.empty((E, c))
    Vt = torch.from_numpy(V)
    for ch in range(c):
        logit = torch.full((E, n), -math.inf, dtype=torch.float64)
        for i, rows in enumerate(windows):
            for (row, bias) in rows:
                logit[i, row] = float(L[row, ch]) + bias[ch]
        Wm = torch.softmax(logit, dim=1)
        out[:, ch] = (Wm @ Vt[:, ch]).numpy()
    return out


def test_brute_force_dense_formulation():
    """A second, independent formulation on tiny inputs: every entry as one row
    of a dense per-channel weight matrix (torch float64 softmax over the
    entry's window, all other rows masked) applied to the stacked streams
    [C^a; C^b].  Must agree with the oracle to 1e-12."""
    for (n, c, m, seed) in [(26, 3, 4, 9), (13, 2, 2, 10), (40, 2, 8, 11)]:
        Ca, Cb, Za, Zb = _rand_streams(n, c, seed, 2.5)
        rng = np.random.default_rng(seed + 100)
        Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
        E = n // m
        V = np.concatenate([Ca, Cb]); L = np.concatenate([Za, Zb])
        windows = []
        for i in range(E):
            rows = [(m * i + r, Ba[r]) for r in range(m)]
            if i >= 1:
                rows += [(n + m * (i - 1) + r, Bb[r]) for r in range(m)]
            windows.append(rows)
        ref = _dense_window_pool(V, L, windows)
        got = oracle.csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
        # HCA: one stream, windows of m rows with B.
        B = rng.standard_normal((m, c))
        ref_h = _dense_window_pool(Ca, Za, [[(m * i + r, B[r]) for r in range(m)] for i in range(E)])
        assert np.allclose(oracle.hca_pool_sequence(Ca, Za, B, m), ref_h, atol=1e-12, rtol=0)


def test_stride_m_kernel_2m_reduction():
    """"Ch 04 · CSA" section 3: the overlapped compressor acts like a learnable
    pooling with stride m and kernel 2m.  With one shared stream (C^a = C^b,
    Z^a = Z^b, B^a = B^b = B) entry i >= 1 is the softmax pool of rows
    [m(i-1), m(i+1)-1] with bias [B; B]; computed here by the dense
    brute-force formulation on a single stream."""
    n, c, m = 30, 3, 4
    C, _, Z, _ = _rand_streams(n, c, 12, 2.0)
    B = np.random.default_rng(13).standard_normal((m, c))
    got = oracle.csa_pool_sequence(C, C, Z, Z, B, B, m)
    E = n // m
    # a kernel of 2m rows over one stream; the row at position r of its block takes B[r]
    windows = [[(row, B[row % m]) for row in range(max(0, m * (i - 1)), m * (i + 1))] for i in range(E)]
    ref = _dense_window_pool(C, Z, windows)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)


def test_shift_invariance_and_overflow_safety():
    """Adding a per-channel constant to Z leaves a softmax unchanged.  +800 makes
    exp overflow float64 unless the maximum is subtracted first."""
    n, c, m = 32, 4, 4
    Ca, Cb, Za, Zb = _rand_streams(n, c, 14)
    rng = np.random.default_rng(15)
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    shift = 800.0 + np.arange(c)
    base = oracle.csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m)
    moved = oracle.csa_pool_sequence(Ca, Cb, Za + shift, Zb + shift, Ba, Bb, m)
    assert np.all(np.isfinite(moved))
    assert np.allclose(base, moved, atol=1e-11, rtol=0)
    B = rng.standard_normal((8, c))
    assert np.allclose(oracle.hca_pool_sequence(Ca, Za, B, 8), oracle.hca_pool_sequence(Ca, Za + shift, B, 8),
                       atol=1e-11, rtol=0)


def test_convex_hull():
    """Each entry is a convex combination of its window's vectors ("Ch 05 · HCA"
    section 2), so per channel it lies within their [min, max]."""
    n, c, m = 48, 5, 4
    Ca, Cb, Za, Zb = _rand_streams(n, c, 16, 4.0)
    rng = np.random.default_rng(17)
    out = oracle.csa_pool_sequence(Ca, Cb, Za, Zb, rng.standard_normal((m, c)), rng.standard_normal((m, c)), m)
    for i in range(n // m):
        vals = Ca[m * i:m * i + m] if i == 0 else np.concatenate([Ca[m * i:m * i + m], Cb[m * (i - 1):m * i]])
        assert np.all(out[i] >= vals.min(axis=0) - 1e-15) and np.all(out[i] <= vals.max(axis=0) + 1e-15)


def test_entry_counts_from_pages():
    """Entry counts the pages print (golden fixture) follow floor(n/m)."""
    with open(os.path.join(GOLDEN, "entry_counts.txt"), encoding="utf-8") as f:
        rows = [ln.split("#")[0].split() for ln in f if ln.split("#")[0].strip()]
    assert len(rows) >= 6
    for n, m, expected, tol in rows:
        assert abs(oracle.n_entries(int(n), int(m)) - int(expected)) <= int(tol), (n, m)
    assert oracle.n_entries(64, 4) == 16 and oracle.n_entries(8192, 4) == 2048
    assert oracle.n_entries(131072, 128) == 1024 and oracle.n_entries(127, 128) == 0


# ----------------------------------------------------------- batch / fused

def test_packed_batch_sequences_are_independent():
    """Sequences of a packed batch do not interact: the packed result is the
    concatenation of per-sequence results, and entry 0 of every sequence is
    its pure a-stream entry."""
    c, m = 3, 4
    lengths = [9, 4, 0, 17, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    n = int(cu[-1])
    Ca, Cb, Za, Zb = _rand_streams(n, c, 18)
    rng = np.random.default_rng(19)
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    packed = oracle.csa_pool(Ca, Cb, Za, Zb, Ba, Bb, m, cu)
    parts = [oracle.csa_pool_sequence(Ca[s:t], Cb[s:t], Za[s:t], Zb[s:t], Ba, Bb, m) for s, t in zip(cu[:-1], cu[1:])]
    assert packed.shape[0] == sum(L // m for L in lengths)
    assert np.array_equal(packed, np.concatenate(parts))
    # perturbing sequence 0's rows leaves later sequences untouched
    Cb2 = Cb.copy(); Cb2[:cu[1]] += 9.0
    packed2 = oracle.csa_pool(Ca, Cb2, Za, Zb, Ba, Bb, m, cu)
    k0 = lengths[0] // m
    assert np.array_equal(packed2[k0:], packed[k0:])
    B = rng.standard_normal((2, c))
    hp = oracle.hca_pool(Ca, Za, B, 2, cu)
    assert np.array_equal(hp, np.concatenate([oracle.hca_pool_sequence(Ca[s:t], Za[s:t], B, 2)
                                              for s, t in zip(cu[:-1], cu[1:])]))


def test_compress_is_project_then_pool_and_ranges_agree():
    """The compressor is the projection followed by the pooling; computing a
    sub-range of entries (projecting only the rows they read) gives the same
    entries as the full computation."""
    rng = np.random.default_rng(20)
    n, d, c, m = 50, 6, 3, 4
    H = rng.standard_normal((n, d))
    Ws = [rng.standard_normal((d, c)) for _ in range(4)]
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    full = oracle.csa_compress_sequence(H, *Ws, Ba, Bb, m)
    ref = oracle.csa_pool_sequence(H @ Ws[0], H @ Ws[1], H @ Ws[2], H @ Ws[3], Ba, Bb, m)
    assert np.allclose(full, ref, atol=1e-13, rtol=0)
    for e0, e1 in [(0, 1), (1, 4), (5, 12), (11, 12), (3, 3)]:
        part = oracle.csa_compress_sequence(H, *Ws, Ba, Bb, m, e0, e1)
        assert np.allclose(part, full[e0:e1], atol=1e-13, rtol=0)
    mh = 8
    B = rng.standard_normal((mh, c))
    fh = oracle.hca_compress_sequence(H, Ws[0], Ws[2], B, mh)
    assert np.allclose(fh, oracle.hca_pool_sequence(H @ Ws[0], H @ Ws[2], B, mh), atol=1e-13, rtol=0)
    assert np.allclose(oracle.hca_compress_sequence(H, Ws[0], Ws[2], B, mh, 2, 5), fh[2:5], atol=1e-13, rtol=0)


# -------------------------------------------------------------- encoders

def test_bf16_matches_torch_cast():
    """bfloat16 RNE: the oracle's rounding equals torch's float32 -> bfloat16
    cast (an independent library routine) on random values and on exact
    halfway points between neighbouring bf16 values."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    base = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    step = np.ldexp(1.0, np.frexp(np.abs(base))[1] - 8)
    mids = (base + 0.5 * step).astype(np.float32)               # exactly representable in fp32
    for v in (x, mids):
        ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
        assert np.array_equal(oracle.round_bf16(v.astype(np.float64)), ref)


def _all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.fp8_e4m3_decode(codes)
    return codes, vals


def test_fp8_decode_table_definition():
    """OCP E4M3FN: largest finite 448 (code 0x7E), smallest normal 2^-6
    (0x08), smallest subnormal 2^-9 (0x01), NaN at S.1111.111, no infinity."""
    codes, vals = _all_codes()
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    assert vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9 and vals[0x38] == 1.0
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.sum(np.isnan(vals)) == 2 and np.all(np.isfinite(vals[~np.isnan(vals)]))
    assert np.nanmax(vals) == 448.0
    # torch's own float8_e4m3fn decode agrees on every finite code
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    fin = ~np.isnan(vals)
    assert np.array_equal(tv[fin].astype(np.float64), vals[fin])


def test_fp8_encode_brute_force_nearest():
    """Encoding = nearest finite E4M3 value by exhaustive search over all 256
    codes, ties to the even code, magnitudes above 448 saturate."""
    codes, vals = _all_codes()
    fin = ~np.isnan(vals)
    fc, fv = codes[fin], vals[fin]
    rng = np.random.default_rng(22)
    x = np.concatenate([rng.standard_normal(3000) * 50, rng.uniform(-1e-2, 1e-2, 2000),
                        (fv[:, None] + np.array([[0.0]])).ravel(),
                        ((np.sort(np.unique(fv))[1:] + np.sort(np.unique(fv))[:-1]) / 2),   # midpoints
                        [500.0, -1e6, 449.0, 464.0, 480.0]])
    got = oracle.fp8_e4m3_encode(x)
    for xi, gi in zip(x, got):
        xs = min(max(xi, -448.0), 448.0)
        dist = np.abs(fv - xs)
        cand = fc[dist == dist.min()]
        if len(cand) > 1:   # tie: prefer the even mantissa; +0 / -0 follow the sign of x
            cand = [k for k in cand if (k & 1) == 0]
            if len(cand) > 1:
                cand = [k for k in cand if bool(k & 0x80) == bool(np.signbit(xs))]
        assert oracle.fp8_e4m3_decode(np.array([gi]))[0] == oracle.fp8_e4m3_decode(np.array([cand[0]]))[0], xi


def test_fp8_encode_matches_torch_in_range():
    """For |x| <= 448 torch's float32 -> float8_e4m3fn cast (RNE) is an
    independent reference for the codes."""
    rng = np.random.default_rng(23)
    x = np.clip(rng.standard_normal(50000) * np.exp(rng.uniform(-12, 6, 50000)), -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_e4m3_encode(x.astype(np.float64)), ref)


def test_fp8_entry_quantize_scale_rule():
    """Per-entry scale s_i = max |x_i| / 448: the largest magnitude of every
    non-zero entry encodes to +-448 exactly; an all-zero entry keeps scale 1."""
    rng = np.random.default_rng(24)
    X = rng.standard_normal((6, 16)) * np.array([[1e-3], [1.0], [30.0], [1e4], [0.0], [2.0]])
    codes, s = oracle.fp8_entry_quantize(X)
    assert s[4] == 1.0 and np.all(oracle.fp8_e4m3_decode(codes[4]) == 0)
    for i in (0, 1, 2, 3, 5):
        assert s[i] == np.abs(X[i]).max() / 448.0
        j = np.argmax(np.abs(X[i]))
        assert abs(oracle.fp8_e4m3_decode(codes[i, j:j + 1])[0]) == 448.0
        dec = oracle.fp8_e4m3_decode(codes[i]) * s[i]
        # one E4M3 step at the value's magnitude bounds the error (half a step for RNE)
        assert np.all(np.abs(dec - X[i]) <= 2.0 ** -4 * np.abs(X[i]) + 2.0 ** -10 * s[i])


# ----------------------------------------------------- the pins have teeth

def _mutant_pool_b_from_next_block(Ca, Cb, Za, Zb, Ba, Bb, m):
    n, c = Ca.shape
    E = n // m
    out = np.empty((E, c))
    for i in range(E):
        La = Za[m * i:m * i + m] + Ba
        if i + 1 < E:   # wrong: b rows of block i+1
            Lb = Zb[m * (i + 1):m * (i + 2)] + Bb; Vb = Cb[m * (i + 1):m * (i + 2)]
        else:
            Lb = np.full((m, c), -np.inf); Vb = np.zeros((m, c))
        L = np.concatenate([La, Lb]); V = np.concatenate([Ca[m * i:m * i + m], Vb])
        w = np.exp(L - L.max(0)); out[i] = (w * V).sum(0) / w.sum(0)
    return out


def _mutant_separate_normalisation(Ca, Cb, Za, Zb, Ba, Bb, m):
    n, c = Ca.shape
    E = n // m
    out = np.empty((E, c))
    for i in range(E):
        La = Za[m * i:m * i + m] + Ba; wa = np.exp(La - La.max(0)); out[i] = (wa * Ca[m * i:m * i + m]).sum(0) / wa.sum(0)
        if i:
            Lb = Zb[m * (i - 1):m * i] + Bb; wb = np.exp(Lb - Lb.max(0))
            out[i] += (wb * Cb[m * (i - 1):m * i]).sum(0) / wb.sum(0)
    return out


def _mutant_no_bias(Ca, Cb, Za, Zb, Ba, Bb, m):
    return oc.csa_pool_sequence(Ca, Cb, Za, Zb, 0 * Ba, 0 * Bb, m)


def _mutant_swapped_bias(Ca, Cb, Za, Zb, Ba, Bb, m):
    return oc.csa_pool_sequence(Ca, Cb, Za, Zb, Bb, Ba, m)


def _mutant_entry0_wraps(Ca, Cb, Za, Zb, Ba, Bb, m):
    # wrong boundary: entry 0 takes the LAST block's b rows (negative index wrap)
    out = oc.csa_pool_sequence(Ca, Cb, Za, Zb, Ba, Bb, m)
    n, c = Ca.shape
    E = n // m
    L = np.concatenate([Za[:m] + Ba, Zb[(E - 1) * m:E * m] + Bb]); V = np.concatenate([Ca[:m], Cb[(E - 1) * m:E * m]])
    w = np.exp(L - L.max(0)); out[0] = (w * V).sum(0) / w.sum(0)
    return out


@pytest.mark.parametrize("mutant", [_mutant_pool_b_from_next_block, _mutant_separate_normalisation,
                                    _mutant_no_bias, _mutant_swapped_bias, _mutant_entry0_wraps])
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    """Plant a plausible mistake in the oracle (on the CPU) and check that the
    exact rational pin rejects it."""
    monkeypatch.setattr(oracle, "csa_pool_sequence", mutant)
    with pytest.raises(AssertionError):
        test_csa_pool_exact_rational(22, 4, 3, 0)
