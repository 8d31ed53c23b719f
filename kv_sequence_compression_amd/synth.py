"""Seeded synthetic inputs for the compressor (no compressor arithmetic here).

This module only draws random tensors and lays them out; it computes nothing
of the method.  Both the HIP path and the float64 oracle consume the tensors
it returns, so they see identical values.

Recipe (shapes are the DeepSeek-V4 shapes the pages use: d = 7168, c = 512,
m = 4 for CSA, m' = 128 for HCA, ~1M tokens):

* every tensor has its own stream keyed by (seed, tensor_id[, sub_id]), so
  draws do not depend on order;
* on the CPU the stream is ``numpy.random.default_rng([seed, tensor_id, ...])``
  drawing float32 standard normals; on a GPU it is a
  ``torch.Generator(device)`` seeded with a 63-bit mix of the same key (fast
  for the 14 GB hidden-state tensors).  The two devices give different but
  equally distributed values; a test always feeds the oracle the very tensor
  the GPU consumed;
* a value is drawn as float32 ``N(0, 1) * std`` and then rounded to the
  storage dtype (bf16 by round-to-nearest-even, via torch's cast);
* "N(0, 1/d)" for a weight means variance 1/d (std 1/sqrt(d)), so a
  projected logit is ~N(0, 1); bias "N(0, s)" means std s.

Tensor ids: H=1, W_KVa=2, W_KVb=3, W_Za=4, W_Zb=5, B^a=6, B^b=7, W_KV=8,
W_Z=9, B=10, lengths=11, outlier channels=12, C^a=13, C^b=14, Z^a=15,
Z^b=16, indexer queries q^I=17, head weights w^I=18, indexer keys=19,
attention queries=20, attended entries=21, sink key=22, sink value=23.

Lightning-indexer inputs (64 heads of 128 dims, the pages' n_h^I and c^I):
queries and keys bf16 N(0, 1), head weights fp32 N(0, 1) (learned weights
of either sign); or, for exact comparisons, small integers in [-3, 3] (every
product and sum is then an integer well below 2^24, exact in fp32).  A query
at position p of its sequence sees the compressed entries whose blocks of m
tokens are complete, floor((p + 1) / m).

Shared-KV attention inputs (128 heads of 512 dims, the pages' n_h and c):
queries bf16 N(0, q_std^2), entries bf16 N(0, 1) (one vector per entry, key
and value), sink key and value bf16 N(0, 1); the logit scale is 1/sqrt(512),
so q_std sets how peaked the attention is.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

TID = dict(H=1, W_KVa=2, W_KVb=3, W_Za=4, W_Zb=5, Ba=6, Bb=7, W_KV=8, W_Z=9, B=10,
           lengths=11, outliers=12, Ca=13, Cb=14, Za=15, Zb=16, Qidx=17, Widx=18, Kidx=19,
           Qatt=20, KVatt=21, Ksink=22, Vsink=23)

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _key_to_int(key) -> int:
    """Deterministic 63-bit integer from a tuple of small ints (SplitMix64 mix)."""
    x = 0x9E3779B97F4A7C15
    for k in key:
        x = (x ^ (int(k) + 0x632BE59BD9B4E019)) & 0xFFFFFFFFFFFFFFFF
        x = (x * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        x ^= x >> 31
    return x & 0x7FFFFFFFFFFFFFFF


def normal(shape, std: float, key, device="cpu", dtype="f32") -> torch.Tensor:
    """Seeded N(0, std^2) tensor of `shape`, stored as `dtype` on `device`."""
    shape = tuple(int(s) for s in shape)
    dev = torch.device(device)
    if dev.type == "cpu":
        rng = np.random.default_rng(list(key))
        x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
        if std != 1.0:
            x.mul_(np.float32(std))
        return x.to(_TORCH_DTYPES[dtype])
    g = torch.Generator(device=dev)
    g.manual_seed(_key_to_int(key))
    out = torch.empty(shape, dtype=_TORCH_DTYPES[dtype], device=dev)
    # Draw in float32 row chunks so a 14 GB bf16 tensor needs no 28 GB float32 temporary.
    rows = shape[0] if shape else 1
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    chunk = max(1, (1 << 28) // max(per_row, 1))
    flat = out.view(rows, per_row) if shape else out.view(1, 1)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        tmp = torch.randn((r1 - r0, per_row), generator=g, dtype=torch.float32, device=dev)
        if std != 1.0:
            tmp.mul_(std)
        flat[r0:r1].copy_(tmp)
    return out


def varlen_lengths(seed: int, batch: int, lo: int, hi: int, multiple: int) -> np.ndarray:
    """Sequence lengths uniform in [lo, hi], in steps of `multiple`."""
    rng = np.random.default_rng([seed, TID["lengths"]])
    k = rng.integers(lo // multiple, hi // multiple + 1, size=batch)
    return (k * multiple).astype(np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    """Prefix offsets [0, L0, L0+L1, ...] (int64) of a packed batch."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    return cu


@dataclass
class CompressorCase:
    """Inputs of one compressor call.

    Wt_cat is [S*c x d] (rows = output channels, K contiguous): CSA stacks
    the transposes of W_KVa | W_KVb | W_Za | W_Zb, HCA those of W_KV | W_Z.
    ``W`` holds each page-layout matrix (d x c) as a view of Wt_cat.
    """
    mode: str
    m: int
    d: int
    c: int
    cu_seqlens: np.ndarray
    H: torch.Tensor
    Wt_cat: torch.Tensor
    biases: dict
    in_dtype: str
    W: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_entries(self) -> int:
        L = np.diff(self.cu_seqlens)
        return int((L // self.m).sum())


def compressor_case(mode: str, lengths, d: int, c: int, m: int, *, seed: int = 0,
                    in_dtype: str = "bf16", bias_std: float = 0.02, device="cpu",
                    w_device=None, z_outlier_frac: float = 0.0, z_outlier_scale: float = 30.0,
                    per_sequence_h: bool = False, H: torch.Tensor | None = None) -> CompressorCase:
    """Draw H, the stacked weights and the biases for one compressor call.

    `z_outlier_frac` of the Z-weight columns (channels) are multiplied by
    `z_outlier_scale`, so those channels' logits are ~N(0, scale^2) on every
    row (the softmax-stability stress of the batched workload).  An existing
    `H` (T x d) may be passed to share hidden states between calls.
    """
    assert mode in ("csa", "hca")
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    w_device = device if w_device is None else w_device
    if H is not None:
        if tuple(H.shape) != (T, d):
            raise ValueError("H does not match the lengths and d")
    elif per_sequence_h:
        H = torch.empty((T, d), dtype=_TORCH_DTYPES[in_dtype], device=device)
        for b in range(lengths.size):
            H[cu[b]:cu[b + 1]] = normal((int(lengths[b]), d), 1.0, (seed, TID["H"], b), device, in_dtype)
    else:
        H = normal((T, d), 1.0, (seed, TID["H"]), device, in_dtype)
    names = ("W_KVa", "W_KVb", "W_Za", "W_Zb") if mode == "csa" else ("W_KV", "W_Z")
    wstd = 1.0 / np.sqrt(d)
    blocks = []
    for nm in names:
        w = normal((c, d), wstd, (seed, TID[nm]), w_device, "f32")
        if nm.startswith("W_Z") and z_outlier_frac > 0:
            k = max(1, int(round(z_outlier_frac * c)))
            rng = np.random.default_rng([seed, TID["outliers"], TID[nm]])
            ch = torch.from_numpy(np.sort(rng.choice(c, size=k, replace=False))).to(w.device)
            w[ch] *= z_outlier_scale
        blocks.append(w.to(_TORCH_DTYPES[in_dtype]))
    Wt_cat = torch.cat(blocks, dim=0).contiguous()
    W = {nm: Wt_cat[i * c:(i + 1) * c].T for i, nm in enumerate(names)}
    if mode == "csa":
        biases = {"Ba": normal((m, c), bias_std, (seed, TID["Ba"]), w_device, "f32"),
                  "Bb": normal((m, c), bias_std, (seed, TID["Bb"]), w_device, "f32")}
    else:
        biases = {"B": normal((m, c), bias_std, (seed, TID["B"]), w_device, "f32")}
    return CompressorCase(mode, m, d, c, cu, H, Wt_cat, biases, in_dtype, W)


@dataclass
class PoolCase:
    """Pre-projected streams for the pooling-only calls (rows x c each)."""
    cu_seqlens: np.ndarray
    streams: dict        # Ca, Cb, Za, Zb
    biases: dict         # Ba, Bb (m_csa x c), B (m_hca x c)
    m_csa: int
    m_hca: int


def pool_case(n: int, c: int, *, m_csa: int = 4, m_hca: int = 128, seed: int = 0,
              dtype: str = "bf16", bias_std: float = 0.02, device="cpu",
              z_std: float = 1.0, lengths=None) -> PoolCase:
    """Independent N(0,1) streams C^a, C^b (std 1) and Z^a, Z^b (std z_std)."""
    cu = cu_from_lengths([n] if lengths is None else lengths)
    T = int(cu[-1])
    streams = {
        "Ca": normal((T, c), 1.0, (seed, TID["Ca"]), device, dtype),
        "Cb": normal((T, c), 1.0, (seed, TID["Cb"]), device, dtype),
        "Za": normal((T, c), z_std, (seed, TID["Za"]), device, dtype),
        "Zb": normal((T, c), z_std, (seed, TID["Zb"]), device, dtype),
    }
    biases = {
        "Ba": normal((m_csa, c), bias_std, (seed, TID["Ba"]), device, "f32"),
        "Bb": normal((m_csa, c), bias_std, (seed, TID["Bb"]), device, "f32"),
        "B": normal((m_hca, c), bias_std, (seed, TID["B"]), device, "f32"),
    }
    return PoolCase(cu, streams, biases, m_csa, m_hca)


# The five workloads (seed 0 everywhere).
CONFIGS = {
    # CSA tiny: n=64, d=64, c=32, m=4 -> 16 entries; fp32 in, fp32 out; biases std 0.1.
    "csa_tiny": dict(kind="fused", mode="csa", lengths=[64], d=64, c=32, m=4,
                     in_dtype="f32", out_dtype="f32", bias_std=0.1),
    # CSA full: n=8192, d=7168, c=512, m=4 -> 2048 entries; bf16 in/out.
    "csa_full": dict(kind="fused", mode="csa", lengths=[8192], d=7168, c=512, m=4,
                     in_dtype="bf16", out_dtype="bf16", bias_std=0.02),
    # HCA: n=131072, d=7168, c=512, m'=128 -> 1024 entries; bf16 in/out.
    "hca_full": dict(kind="fused", mode="hca", lengths=[131072], d=7168, c=512, m=128,
                     in_dtype="bf16", out_dtype="bf16", bias_std=0.02),
    # Pool-only long context: four bf16 streams of 1048576 x 512; CSA m=4 -> 262144
    # entries, HCA m'=128 on (C^a, Z^a) -> 8192 entries.
    "pool_long": dict(kind="pool", n=1 << 20, c=512, m_csa=4, m_hca=128,
                      dtype="bf16", out_dtype="bf16", bias_std=0.02),
    # Batched variable-length fused CSA + HCA: 32 sequences, lengths uniform in
    # [4096, 65536] in steps of 128, fp8 E4M3 entries with per-entry fp32 scales,
    # 1% of the Z channels scaled x30.
    "varlen_fp8": dict(kind="fused2", batch=32, len_lo=4096, len_hi=65536, len_mult=128,
                       d=7168, c=512, m_csa=4, m_hca=128, in_dtype="bf16",
                       out_dtype="fp8", bias_std=0.02, z_outlier_frac=0.01,
                       z_outlier_scale=30.0),
    # Lightning indexer at 1M context: one sequence of 2^20 tokens -> 262144
    # compressed indexer keys (m = 4); its last 4096 tokens query them
    # (causal: floor((p + 1) / 4) visible), k = 1024.
    "indexer_1m": dict(kind="indexer", n_tokens=1 << 20, m=4, n_queries=4096, k=1024),
    # HCA dense attention at 1M context: 2^20 tokens -> 8192 HCA entries
    # (m' = 128); the last 4096 tokens attend (causal: floor((p + 1) / 128)
    # visible), 128 heads x 512, with an attention sink; bf16 out.
    "hca_mqa_1m": dict(kind="mqa", n_tokens=1 << 20, m=128, n_queries=4096, q_std=1.0),
}


def varlen_config_lengths(seed: int = 0) -> np.ndarray:
    cfg = CONFIGS["varlen_fp8"]
    return varlen_lengths(seed, cfg["batch"], cfg["len_lo"], cfg["len_hi"], cfg["len_mult"])


# ------------------------------------------------------------ indexer inputs

INDEXER_HEADS = 64     # n_h^I
INDEXER_DIM = 128      # c^I


def integers(shape, lo: int, hi: int, key, device="cpu", dtype="bf16") -> torch.Tensor:
    """Seeded uniform integers in [lo, hi] stored as `dtype` (exact in bf16
    for |v| <= 256)."""
    rng = np.random.default_rng(list(key))
    x = torch.from_numpy(rng.integers(lo, hi + 1, size=tuple(int(v) for v in shape)).astype(np.float32))
    return x.to(_TORCH_DTYPES[dtype]).to(device)


@dataclass
class IndexerCase:
    q: torch.Tensor            # [T x 64 x 128] bf16
    w: torch.Tensor            # [T x 64] fp32
    keys: torch.Tensor         # [N x 128] bf16
    cu_q: np.ndarray
    cu_k: np.ndarray


def indexer_case(q_lengths, k_lengths, *, seed: int = 0, device="cpu", integer: bool = False) -> IndexerCase:
    """Queries, head weights and compressed indexer keys of a packed batch:
    sequence b has q_lengths[b] queries and k_lengths[b] keys."""
    T, N = int(np.sum(q_lengths)), int(np.sum(k_lengths))
    H, D = INDEXER_HEADS, INDEXER_DIM
    if integer:
        q = integers((T, H, D), -3, 3, (seed, TID["Qidx"]), device)
        w = integers((T, H), -3, 3, (seed, TID["Widx"]), device, "f32")
        keys = integers((N, D), -3, 3, (seed, TID["Kidx"]), device)
    else:
        q = normal((T, H, D), 1.0, (seed, TID["Qidx"]), device, "bf16")
        w = normal((T, H), 1.0, (seed, TID["Widx"]), device, "f32")
        keys = normal((N, D), 1.0, (seed, TID["Kidx"]), device, "bf16")
    return IndexerCase(q, w, keys, cu_from_lengths(q_lengths), cu_from_lengths(k_lengths))


def causal_visible(positions, m: int) -> np.ndarray:
    """Entries visible to queries at `positions`: complete blocks of m tokens."""
    return ((np.asarray(positions, dtype=np.int64) + 1) // m).astype(np.int32)


MQA_HEADS = 128        # n_h
MQA_DIM = 512          # c


@dataclass
class MqaCase:
    q: torch.Tensor            # [T x 128 x 512] bf16
    kv: torch.Tensor           # [N x 512] bf16
    k_sink: torch.Tensor       # [512] bf16
    v_sink: torch.Tensor       # [512] bf16
    cu_q: np.ndarray
    cu_k: np.ndarray


def mqa_case(q_lengths, k_lengths, *, seed: int = 0, device="cpu", q_std: float = 1.0) -> MqaCase:
    """Queries, entries and a sink for shared-KV attention over a packed batch:
    sequence b has q_lengths[b] queries and k_lengths[b] entries."""
    T, N = int(np.sum(q_lengths)), int(np.sum(k_lengths))
    q = normal((T, MQA_HEADS, MQA_DIM), q_std, (seed, TID["Qatt"]), device, "bf16")
    kv = normal((N, MQA_DIM), 1.0, (seed, TID["KVatt"]), device, "bf16")
    ks = normal((MQA_DIM,), 1.0, (seed, TID["Ksink"]), device, "bf16")
    vs = normal((MQA_DIM,), 1.0, (seed, TID["Vsink"]), device, "bf16")
    return MqaCase(q, kv, ks, vs, cu_from_lengths(q_lengths), cu_from_lengths(k_lengths))
