"""Pins of the oracle's packed-batch compressors, ``oracle.csa_compress`` and
``oracle.hca_compress`` (projection, then pooling, over a packed batch of
independent sequences).  These two functions are the reference of the fused
GPU tests and of the smoke check, so they are pinned here against facts that
do not come from the oracle:

* exact rational arithmetic: with zero logit weights and B = 0 every window
  is a plain mean ("Ch 04 · CSA" section 3, the simple-average special case),
  and with integer H and W the projected values are integers, so every entry
  is a rational number computed here with ``fractions.Fraction`` from an
  integer triple loop;
* a second, dense formulation over the whole packed batch: every entry is a
  row of a per-channel weight matrix (torch float64 softmax over the entry's
  window, all other packed rows masked), applied to the stacked projected
  streams, with the projection done by torch;
* the boundary rule of eq. attn-seqcomp-overlap-bound ("序列压缩注意力") for
  every sequence: entry 0 is the a-stream alone and depends on no b input;
* independence: perturbing one sequence's rows changes only its own
  entries, and only those whose windows read the rows;
* planted mistakes in the packed wrappers (windows crossing sequences, the
  tail dropped per batch instead of per sequence, sequences reordered) fail
  at least one of the above.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

LENGTHS = [9, 4, 0, 17, 3, 12, 1, 8]          # ragged: empty, shorter than m, tails


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _csa_inputs(lengths, d, c, m, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    H = rng.standard_normal((T, d))
    W = [rng.standard_normal((d, c)) * scale / math.sqrt(d) for _ in range(4)]
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    return H, W, Ba, Bb


def _windows_csa(cu, m):
    """Window of every packed entry as (stream, packed row, bias row) triples:
    a rows of block i and b rows of block i - 1 of the same sequence."""
    wins = []
    for s, t in zip(cu[:-1], cu[1:]):
        E = (t - s) // m
        for i in range(E):
            rows = [("a", s + m * i + r, r) for r in range(m)]
            if i >= 1:
                rows += [("b", s + m * (i - 1) + r, r) for r in range(m)]
            wins.append(rows)
    return wins


def _dense_packed(V, L, wins, T, c):
    """Per channel: (E x 2T) logits, -inf except each entry's window; torch
    float64 softmax over rows; times the stacked values [a-stream; b-stream]."""
    E = len(wins)
    out = np.zeros((E, c))
    if E == 0:
        return out
    for ch in range(c):
        logit = torch.full((E, V.shape[0]), -math.inf, dtype=torch.float64)
        for e, rows in enumerate(wins):
            for stream, row, r in rows:
                k = row if stream == "a" else T + row
                logit[e, k] = float(L[k, ch, r]) if L.ndim == 3 else float(L[k, ch])
        Wm = torch.softmax(logit, dim=1)
        out[:, ch] = (Wm @ torch.from_numpy(V[:, ch])).numpy()
    return out


# ---------------------------------------------------------------- dense form

def test_csa_compress_packed_dense_brute_force():
    """The packed CSA compressor equals a dense formulation written over the
    whole packed batch (torch projection, torch float64 softmax over each
    entry's masked window of [C^a; C^b]) to 1e-12: windows never cross a
    sequence, every sequence's entry 0 has no b rows, tails are dropped per
    sequence."""
    m, d, c = 4, 6, 3
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    H, W, Ba, Bb = _csa_inputs(LENGTHS, d, c, m, 30, scale=3.0)
    Ht = torch.from_numpy(H)
    Ca, Cb, Za, Zb = ((Ht @ torch.from_numpy(w)).numpy() for w in W)
    V = np.concatenate([Ca, Cb])
    wins = _windows_csa(cu, m)
    # logits with the bias of the row's position in its block: one plane per r
    L = np.empty((2 * T, c, m))
    for r in range(m):
        L[:T, :, r] = Za + Ba[r]
        L[T:, :, r] = Zb + Bb[r]
    ref = _dense_packed(V, L, wins, T, c)
    got = oracle.csa_compress(H, *W, Ba, Bb, m, cu)
    assert got.shape == (sum(L_ // m for L_ in LENGTHS), c)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)


def test_hca_compress_packed_dense_brute_force():
    """The packed HCA compressor equals the dense formulation over the packed
    batch (windows = the m' rows of each complete block of each sequence)."""
    m, d, c = 3, 5, 4
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    rng = np.random.default_rng(31)
    H = rng.standard_normal((T, d))
    W_KV, W_Z = rng.standard_normal((d, c)), rng.standard_normal((d, c)) * 2.0
    B = rng.standard_normal((m, c))
    Ht = torch.from_numpy(H)
    C = (Ht @ torch.from_numpy(W_KV)).numpy()
    Z = (Ht @ torch.from_numpy(W_Z)).numpy()
    wins = []
    for s, t in zip(cu[:-1], cu[1:]):
        for i in range((t - s) // m):
            wins.append([("a", s + m * i + r, r) for r in range(m)])
    L = np.empty((2 * T, c, m))
    for r in range(m):
        L[:T, :, r] = Z + B[r]
        L[T:, :, r] = -np.inf
    ref = _dense_packed(np.concatenate([C, C]), L, wins, T, c)
    got = oracle.hca_compress(H, W_KV, W_Z, B, m, cu)
    assert got.shape == (sum(L_ // m for L_ in LENGTHS), c)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)


# ------------------------------------------------------ exact rational means

def _int_mat(rng, shape, lo=-5, hi=6):
    return rng.integers(lo, hi, size=shape)


def test_csa_compress_packed_exact_mean():
    """Zero logit weights and zero biases make every weight equal, so CSA
    entry i >= 1 of a sequence is the mean of its m a-rows of C^a = H W^{KV_a}
    and its m b-rows of C^b = H W^{KV_b}; entry 0 the mean of its m a-rows.
    With integer H and W that is an exact rational, computed here from an
    integer triple loop."""
    m, d, c = 4, 3, 2
    rng = np.random.default_rng(32)
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    H = _int_mat(rng, (T, d))
    Wa, Wb = _int_mat(rng, (d, c)), _int_mat(rng, (d, c))
    zero_w, zero_b = np.zeros((d, c)), np.zeros((m, c))

    def proj(Wm, t, ch):
        return sum(int(H[t, k]) * int(Wm[k, ch]) for k in range(d))

    ref = []
    for s, t in zip(cu[:-1], cu[1:]):
        for i in range((t - s) // m):
            row = []
            for ch in range(c):
                vals = [proj(Wa, s + m * i + r, ch) for r in range(m)]
                if i >= 1:
                    vals += [proj(Wb, s + m * (i - 1) + r, ch) for r in range(m)]
                row.append(Fraction(sum(vals), len(vals)))
            ref.append(row)
    got = oracle.csa_compress(H.astype(float), Wa.astype(float), Wb.astype(float), zero_w, zero_w, zero_b, zero_b,
                              m, cu)
    assert got.shape == (len(ref), c)
    for e, row in enumerate(ref):
        for ch in range(c):
            assert abs(Fraction(float(got[e, ch])) - row[ch]) <= abs(row[ch]) * Fraction(1, 10 ** 14) + \
                Fraction(1, 10 ** 15), (e, ch)


def test_hca_compress_packed_exact_mean():
    """Zero logit weights and B = 0: each HCA entry is the mean of the m' rows
    of its block of C = H W^{KV}, in exact rationals (integer H and W)."""
    m, d, c = 4, 3, 2
    rng = np.random.default_rng(33)
    cu = _cu(LENGTHS)
    T = int(cu[-1])
    H = _int_mat(rng, (T, d))
    Wk = _int_mat(rng, (d, c))
    ref = []
    for s, t in zip(cu[:-1], cu[1:]):
        for i in range((t - s) // m):
            ref.append([Fraction(sum(sum(int(H[s + m * i + r, k]) * int(Wk[k, ch]) for k in range(d))
                                     for r in range(m)), m) for ch in range(c)])
    got = oracle.hca_compress(H.astype(float), Wk.astype(float), np.zeros((d, c)), np.zeros((m, c)), m, cu)
    assert got.shape == (len(ref), c)
    for e, row in enumerate(ref):
        for ch in range(c):
            assert abs(Fraction(float(got[e, ch])) - row[ch]) <= abs(row[ch]) * Fraction(1, 10 ** 14) + \
                Fraction(1, 10 ** 15), (e, ch)


# ------------------------------------------------- boundary and independence

def _entry_starts(cu, m):
    counts = np.diff(cu) // m
    return np.concatenate([[0], np.cumsum(counts)]), counts


def test_csa_compress_every_entry0_is_pure_a_stream():
    """eq. attn-seqcomp-overlap-bound ("序列压缩注意力") for every sequence of
    the batch: entry 0 equals the single-stream softmax pool of block 0 of the
    a-stream with B^a (the HCA formula with m' = m), and changing every
    b-stream input (W^{KV_b}, W^{Z_b}, B^b) leaves each sequence's entry 0
    bit-identical while it changes every other entry."""
    m, d, c = 4, 5, 3
    cu = _cu(LENGTHS)
    H, W, Ba, Bb = _csa_inputs(LENGTHS, d, c, m, 34, scale=2.0)
    base = oracle.csa_compress(H, *W, Ba, Bb, m, cu)
    rng = np.random.default_rng(35)
    pert = oracle.csa_compress(H, W[0], W[1] + rng.standard_normal(W[1].shape), W[2],
                               W[3] + rng.standard_normal(W[3].shape), Ba, Bb + 1.5, m, cu)
    starts, counts = _entry_starts(cu, m)
    first = {int(starts[b]) for b in range(len(LENGTHS)) if counts[b] > 0}
    assert first
    for e in range(base.shape[0]):
        if e in first:
            assert np.array_equal(base[e], pert[e]), e
        else:
            assert not np.allclose(base[e], pert[e], atol=1e-6, rtol=0), e
    for b in range(len(LENGTHS)):
        if counts[b]:
            s = int(cu[b])
            block0 = H[s:s + m]
            single = oracle.hca_pool_sequence(block0 @ W[0], block0 @ W[2], Ba, m)
            assert np.allclose(base[starts[b]], single[0], atol=1e-14, rtol=0), b


@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_compress_perturbing_one_sequence_touches_only_its_windows(mode):
    """Perturbing one H row of sequence b changes exactly the entries whose
    windows read that row (CSA: the entry of its block via the a-stream and
    the next entry of the same sequence via the b-stream; HCA: its block's
    entry; none for a row in the dropped tail), and every other entry of the
    packed batch stays bit-identical."""
    m = 4
    d, c = 5, 3
    cu = _cu(LENGTHS)
    H, W, Ba, Bb = _csa_inputs(LENGTHS, d, c, m, 36, scale=2.0)
    rng = np.random.default_rng(37)
    Bh = rng.standard_normal((m, c))

    def run(Hx):
        if mode == "csa":
            return oracle.csa_compress(Hx, *W, Ba, Bb, m, cu)
        return oracle.hca_compress(Hx, W[0], W[2], Bh, m, cu)

    base = run(H)
    starts, counts = _entry_starts(cu, m)
    for b in range(len(LENGTHS)):
        for j in range(LENGTHS[b]):
            Hp = H.copy()
            Hp[int(cu[b]) + j] += 0.5
            out = run(Hp)
            changed = {e for e in range(out.shape[0]) if not np.array_equal(out[e], base[e])}
            blk = j // m
            expect = set()
            if blk < counts[b]:
                expect.add(int(starts[b]) + blk)
                if mode == "csa" and blk + 1 < counts[b]:
                    expect.add(int(starts[b]) + blk + 1)
            assert changed == expect, (mode, b, j, changed, expect)


# ----------------------------------------------------- the pins have teeth

def _mutant_csa_ignores_cu(H, W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m, cu_seqlens=None):
    # wrong: the whole batch as one sequence (windows cross sequences)
    from oracle import compressor as oc
    return oc.csa_compress_sequence(H, W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m)


def _mutant_csa_b_crosses_sequences(H, W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m, cu_seqlens=None):
    # wrong: every sequence's entry 0 reads the previous sequence's last rows as its b block
    from oracle import compressor as oc
    cu = np.asarray(cu_seqlens)
    outs = []
    for s, t in zip(cu[:-1], cu[1:]):
        E = (t - s) // m
        if E == 0:
            continue
        lo = s - m if s >= m else s
        full = oc.csa_compress_sequence(H[lo:s + E * m], W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m)
        outs.append(full[-E:])
    return np.concatenate(outs) if outs else np.zeros((0, np.asarray(W_KVa).shape[1]))


def _mutant_csa_reversed_sequences(H, W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m, cu_seqlens=None):
    # wrong: packed output in reverse sequence order
    from oracle import compressor as oc
    cu = np.asarray(cu_seqlens)
    outs = [oc.csa_compress_sequence(H[s:t], W_KVa, W_KVb, W_Za, W_Zb, Ba, Bb, m) for s, t in zip(cu[:-1], cu[1:])]
    return np.concatenate(outs[::-1])


def _mutant_hca_tail_per_batch(H, W_KV, W_Z, B, m, cu_seqlens=None):
    # wrong: blocks taken over the packed rows, tail dropped once per batch
    from oracle import compressor as oc
    return oc.hca_compress_sequence(H, W_KV, W_Z, B, m)


@pytest.mark.parametrize("mutant,pin", [
    (_mutant_csa_ignores_cu, test_csa_compress_packed_dense_brute_force),
    (_mutant_csa_ignores_cu, test_csa_compress_packed_exact_mean),
    (_mutant_csa_b_crosses_sequences, test_csa_compress_packed_dense_brute_force),
    (_mutant_csa_b_crosses_sequences, test_csa_compress_every_entry0_is_pure_a_stream),
    (_mutant_csa_reversed_sequences, test_csa_compress_packed_exact_mean),
])
def test_planted_csa_packing_mistakes_are_caught(mutant, pin, monkeypatch):
    """A plausible mistake planted in the packed CSA wrapper fails the pin."""
    monkeypatch.setattr(oracle, "csa_compress", mutant)
    with pytest.raises(AssertionError):
        pin()


@pytest.mark.parametrize("pin", [test_hca_compress_packed_dense_brute_force, test_hca_compress_packed_exact_mean])
def test_planted_hca_packing_mistake_is_caught(pin, monkeypatch):
    """Blocks taken over the packed rows instead of per sequence fail the HCA pins."""
    monkeypatch.setattr(oracle, "hca_compress", _mutant_hca_tail_per_batch)
    with pytest.raises(AssertionError):
        pin()
