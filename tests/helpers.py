"""Shared test helpers: tolerance checks against the float64 oracle.

Tolerances (written out in every test that uses them):
* fp32 inputs and fp32 output on the pooling path: max |gpu - oracle| <= 1e-5;
* bf16 paths (bf16 GEMM operands or bf16 output): per entry row,
  max_ch |gpu - ref| / max_ch |ref| <= 2e-2;
* fp8 output: |s_gpu / s_ref - 1| <= 2e-2, and per element
  |decode(q_gpu) s_gpu - ref| <= ulp_E4M3(|ref| / s_ref) s_ref + base, where
  `base` is the error bound of the path without fp8 (2e-2 * max_ch |ref_i|
  for bf16 paths, 1e-5 for fp32 ones): one fp8 step on top of the path error.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max |got - ref| / max |ref|."""
    if got.size == 0:
        return np.zeros(0)
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return num / den


def e4m3_step(x: np.ndarray) -> np.ndarray:
    """Spacing of E4M3 values at magnitude x (scaled domain): 2^(floor(log2 x) - 3),
    2^-9 in the subnormal range."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -6)))
    return np.where(ax < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def check_fp8(codes: torch.Tensor, scale: torch.Tensor, ref: np.ndarray, path_rel: float, path_abs: float = 0.0):
    """Assert the fp8 tolerance; returns (max scale rel err, max excess)."""
    q = codes.cpu().numpy().astype(np.uint8)
    s = scale.cpu().double().numpy()
    amax = np.abs(ref).max(axis=1)
    s_ref = np.where(amax > 0, amax / oracle.FP8_E4M3_MAX, 1.0)
    srel = np.abs(s / s_ref - 1.0)
    assert np.all(srel <= 2e-2), f"scale rel err {srel.max()}"
    dec = oracle.fp8_e4m3_decode(q) * s[:, None]
    bound = e4m3_step(ref / s_ref[:, None]) * s_ref[:, None] + path_rel * amax[:, None] + path_abs
    excess = np.abs(dec - ref) - bound
    assert np.all(excess <= 0), f"fp8 error exceeds bound by {excess.max()} at {np.unravel_index(np.argmax(excess), excess.shape)}"
    return float(srel.max()), float(excess.max())


def sample_entries(E: int, k: int, seed: int = 0, must=()) -> np.ndarray:
    """Sorted sample of k entry indices in [0, E) plus the `must` ones (clipped)."""
    rng = np.random.default_rng(seed)
    picks = set(int(x) for x in must if 0 <= x < E)
    if E > 0:
        picks.update(int(x) for x in rng.choice(E, size=min(k, E), replace=False))
    return np.array(sorted(picks), dtype=np.int64)


def entry_owner(cu: np.ndarray, m: int, idx: np.ndarray):
    """Map packed entry indices to (sequence, local entry)."""
    counts = np.diff(cu) // m
    starts = np.concatenate([[0], np.cumsum(counts)])
    seq = np.searchsorted(starts, idx, side="right") - 1
    return seq, idx - starts[seq]


# ------------------------------------------------------------ indexer checks

U32 = 2.0 ** -24   # fp32 unit roundoff


def indexer_score_bound(Q, w, K, u=U32):
    """Per-query a priori bound on |fp32 score - exact score| over all keys:
    200 u max_s sum_h |w_h| sum_i |q_hi K_si|.  A dot product of 128 bf16
    products (exact in fp32) takes at most 127 roundings, the weighted head
    sum at most 66 (fused multiply-adds, two partial sums, one exchange add),
    so the error is below (gamma_127 + gamma_66 + gamma_127 gamma_66) B
    < 200 u B, with B = sum_h |w_h| sum_i |q_hi K_si|."""
    Q, w, K = np.abs(Q), np.abs(w), np.abs(K)
    T, H, c = Q.shape
    B = np.einsum("th,ths->ts", w, (Q.reshape(T * H, c) @ K.T).reshape(T, H, -1))
    return 200.0 * u * (B.max(axis=1) if B.shape[1] else np.zeros(T))


def check_topk_valid(idx, sc, I, nv, k, beta):
    """A selection is valid when scores differ from the oracle's by <= beta:
    indices distinct, increasing and visible, min(k, visible) of them; returned
    scores within beta of the oracle's; every key above the oracle's k-th
    score + 2 beta selected and none below the k-th - 2 beta."""
    idx = np.asarray(idx, dtype=np.int64)
    for t in range(idx.shape[0]):
        v = int(nv[t])
        n = min(k, v)
        sel = idx[t, :n]
        assert np.all(idx[t, n:] == -1), t
        assert np.all(np.diff(sel) > 0) and (n == 0 or (sel[0] >= 0 and sel[-1] < v)), t
        if sc is not None:
            assert np.all(np.isneginf(sc[t, n:])), t
            err = np.abs(sc[t, :n] - I[t, sel])
            assert np.all(err <= beta[t]), (t, err.max(), beta[t])
        if v > k:
            row = I[t, :v]
            kth = np.sort(row)[::-1][k - 1]
            must = np.nonzero(row > kth + 2 * beta[t])[0]
            never = np.nonzero(row < kth - 2 * beta[t])[0]
            s = set(sel.tolist())
            assert all(int(x) in s for x in must), t
            assert not any(int(x) in s for x in never), t


# ------------------------------------------------- shared-KV attention checks

def mqa_abs_weighted(Q, KV, nv, scale, k_sink=None, v_sink=None):
    """sum_s alpha_s |v_s| per output element (float64), the scale of the
    error the bf16 rounding of the probabilities can cause."""
    absv = np.abs(KV)
    vs = None if v_sink is None else np.abs(v_sink)
    T, H, c = Q.shape
    out = np.zeros((T, H, c))
    for t in range(T):
        K = KV[: int(nv[t])]
        V = absv[: int(nv[t])]
        if k_sink is not None:
            K = np.vstack([k_sink[None], K])
            V = np.vstack([(np.zeros(c) if v_sink is None else vs)[None], V])
        if K.shape[0] == 0:
            continue
        lg = scale * (Q[t] @ K.T)
        e = np.exp(lg - lg.max(1, keepdims=True))
        out[t] = (e / e.sum(1, keepdims=True)) @ V
    return out


def check_mqa(out, ref, absw, out_dtype, lse=None, ref_lse=None):
    """|gpu - ref| <= 2^-7 sum_s alpha_s |v_s| (+ 2^-8 |ref| for bf16 output):
    each probability is rounded to bf16 (relative 2^-9) before the value
    product, with a 4x margin; the log-sum-exp within 1e-4 absolute."""
    tol = 2.0 ** -7 * absw + (2.0 ** -8 * np.abs(ref) if out_dtype == "bf16" else 0.0) + 1e-6
    err = np.abs(out - ref)
    assert np.all(err <= tol), f"max excess {np.max(err - tol)} at {np.unravel_index(np.argmax(err - tol), err.shape)}"
    if lse is not None:
        both_inf = np.isneginf(lse) & np.isneginf(ref_lse)
        with np.errstate(invalid="ignore"):                  # -inf - -inf where nothing is visible
            close = np.abs(lse - ref_lse) <= 1e-4
        assert np.all(both_inf | close), np.nanmax(np.where(both_inf, 0.0, np.abs(lse - ref_lse)))


# ------------------------------------------ fused kernel schedule (host mirror)

FUSED_TILE_ROWS = 256      # rows (tokens) per M tile of the fused kernels


def fused_tiles(cu, m: int):
    """Tile table of the fused kernels, as the planner writes it: every
    sequence's complete blocks cut into tiles of 256 rows, in sequence order.
    Returns a list of (row_start, n_rows, entry_start, first_of_sequence)."""
    tiles, ent = [], 0
    for s, t in zip(cu[:-1], cu[1:]):
        rows = (int(t - s) // m) * m
        for j, r0 in enumerate(range(0, rows, FUSED_TILE_ROWS)):
            n = min(FUSED_TILE_ROWS, rows - r0)
            tiles.append((int(s) + r0, n, ent + r0 // m, j == 0))
        ent += rows // m
    return tiles


def fused_n_tiles_n(mode: str, c: int) -> int:
    """N tiles per M tile: 64 channels x 4 streams (CSA), 128 x 2 (HCA)."""
    return -(-c // (64 if mode == "csa" else 128))


def fused_round_xcd_samples(cu, m: int, mode: str, c: int, n_cu: int, seed: int = 0) -> np.ndarray:
    """Packed entry indices that place at least one check in every
    (persistent round, XCD) pair of the fused kernel's grid, plus every tile
    boundary (a tile's first and last entry, and the entry before it) of the
    first and the last round.

    The grid has P = min(G, n_cu) workgroups over G = tiles x N tiles logical
    tiles; round k covers logical tiles [k P, (k + 1) P).  Workgroup w runs on
    XCD w mod 8, and XCD x owns the contiguous range of q + (x < r) logical
    tiles starting at x q + min(x, r) of each round (q = P // 8, r = P % 8);
    logical tile L is M tile L // n_nt."""
    tiles = fused_tiles(cu, m)
    n_nt = fused_n_tiles_n(mode, c)
    G = len(tiles) * n_nt
    if G == 0:
        return np.zeros(0, dtype=np.int64)
    P = min(G, n_cu)
    q, r = P // 8, P % 8
    rounds = -(-G // P)
    rng = np.random.default_rng(seed)
    picks = set()
    for k in range(rounds):
        for x in range(8):
            lo = k * P + x * q + min(x, r)
            hi = min(lo + q + (1 if x < r else 0), G)
            if lo >= hi:
                continue
            _, n_rows, e0, _ = tiles[int(rng.integers(lo, hi)) // n_nt]
            picks.add(e0 + int(rng.integers(0, n_rows // m)))
    for k in {0, rounds - 1}:
        for mt in sorted({L // n_nt for L in range(k * P, min((k + 1) * P, G))}):
            _, n_rows, e0, _ = tiles[mt]
            picks.update({e0, e0 + n_rows // m - 1})
            if e0 > 0:
                picks.add(e0 - 1)
    return np.array(sorted(picks), dtype=np.int64)


def oracle_entries(case, idx, rows_per_chunk: int = 8192) -> np.ndarray:
    """Oracle value of the packed entries `idx` of a compressor case,
    projecting only the rows each entry reads.  The rows of many entries are
    gathered into one matrix per chunk, projected with ``oracle.project``
    (one product per stream) and pooled window by window with
    ``oracle.csa_pool_sequence`` / ``oracle.hca_pool_sequence`` -- the same
    composition as ``oracle.csa_compress_sequence``."""
    idx = np.asarray(idx, dtype=np.int64)
    m, c = case.m, case.c
    csa = case.mode == "csa"
    W = {k: to64(v) for k, v in case.W.items()}
    b = {k: to64(v) for k, v in case.biases.items()}
    seq, loc = entry_owner(case.cu_seqlens, m, idx)
    out = np.empty((idx.size, c))
    per_chunk = max(1, rows_per_chunk // (2 * m if csa else m))
    dev = case.H.device
    for j0 in range(0, idx.size, per_chunk):
        rows, spans = [], []
        for s, i in zip(seq[j0:j0 + per_chunk], loc[j0:j0 + per_chunk]):
            t0 = int(case.cu_seqlens[s])
            lo = max(int(i) - 1, 0) * m if csa else int(i) * m
            hi = (int(i) + 1) * m
            spans.append((len(rows), hi - lo, int(i) - lo // m))
            rows.extend(range(t0 + lo, t0 + hi))
        Hs = to64(case.H[torch.as_tensor(rows, dtype=torch.int64, device=dev)])
        if csa:
            P = [oracle.project(Hs, W[k]) for k in ("W_KVa", "W_KVb", "W_Za", "W_Zb")]
            for j, (p0, n, k) in enumerate(spans):
                win = [x[p0:p0 + n] for x in P]
                out[j0 + j] = oracle.csa_pool_sequence(*win, b["Ba"], b["Bb"], m, k, k + 1)[0]
        else:
            C, Z = oracle.project(Hs, W["W_KV"]), oracle.project(Hs, W["W_Z"])
            for j, (p0, n, _) in enumerate(spans):
                out[j0 + j] = oracle.hca_pool_sequence(C[p0:p0 + n], Z[p0:p0 + n], b["B"], m)[0]
    return out


def fp8_codes_match_encoder(codes, scale, x32, rel_mid: float = 1e-6):
    """The fp8 encoder alone against the oracle's: `x32` are the fp32 entries
    the same kernels produced (float64 copy), `codes` / `scale` the encoded
    output.  The scale must be within one fp32 ulp of max |x| / 448 (1 for an
    all-zero entry) and every code must equal oracle.fp8_entry_quantize's,
    except where x / s lies within `rel_mid` (relative) of a rounding midpoint
    between two neighbouring E4M3 values: there the two codes may be those
    neighbours (fp32 rounding of s and of x / s moves the quotient by about
    1e-7 relative).  Returns (number of codes, number of midpoint cases)."""
    q = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scale, dtype=np.float64)
    ref_q, ref_s = oracle.fp8_entry_quantize(x32)
    ulp = np.spacing(np.abs(ref_s).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(s - ref_s) <= ulp), f"scale off by {np.max(np.abs(s - ref_s) / ulp)} ulp"
    bad = np.nonzero(q != ref_q)
    mid_cases = 0
    if bad[0].size:
        y = x32[bad] / ref_s[bad[0]]
        v_gpu = oracle.fp8_e4m3_decode(q[bad])
        v_ref = oracle.fp8_e4m3_decode(ref_q[bad])
        mid = 0.5 * (v_gpu + v_ref)
        step = e4m3_step(np.minimum(np.abs(v_gpu), np.abs(v_ref)))
        neighbours = np.abs(v_gpu - v_ref) <= step * (1 + 1e-12)
        near_mid = np.abs(y - mid) <= rel_mid * np.abs(mid)
        ok = neighbours & near_mid
        assert np.all(ok), (f"{int((~ok).sum())} codes differ away from a rounding midpoint, e.g. x/s="
                            f"{y[~ok][:4]} gpu={v_gpu[~ok][:4]} ref={v_ref[~ok][:4]}")
        mid_cases = int(bad[0].size)
    return int(q.size), mid_cases
