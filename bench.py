#!/usr/bin/env python3
"""Throughput of the token-level KV compressor on one MI355X.

One step = one pass of the whole compressor hot path over one batch:
the batched variable-length workload (32 sequences, lengths uniform in
[4096, 65536] in steps of 128 -> T = 968,960 tokens at seed 0; d = 7168,
c = 512) through the fused CSA compressor (m = 4, 242,240 entries) and the
fused HCA compressor (m' = 128, 7,570 entries), fp8 E4M3 entries with
per-entry scales.  Inputs are synthetic (seeded normals), resident in HBM
before timing starts.

Prints ONE JSON line (rank 0).  `value` is compressed entries/s of the step
(CSA + HCA entries); tokens/s counts each input token once.  Also reported:
* roofline of the dominant kernel (the fused CSA call: MFMA-bound; its
  FLOPs are 2 * T * d * 4c per launch), timed with HIP events on the
  library's stream over the timed region;
* the pooling-only path on the long-context streams (four bf16 streams of
  2^20 x 512; CSA m=4 and HCA m'=128), HBM-bound;
* cpu_baseline: the float64 oracle on a bounded sample of the same workload
  (the first 262144 tokens of the batch), on this host's cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed entries/s and tokens/s at n=1M; % bf16 MFMA peak / % HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
        from kv_sequence_compression_amd.build import source_digest
        entry = rec["kernels"][kernel_key]
        if entry.get("source_digest") != source_digest():
            return None
        return float(entry["bytes_per_launch"])
    except (OSError, KeyError, ValueError, ImportError):
        return None


def _progress(msg: str):
    """One line per finished phase on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _blas_threads() -> int:
    """Threads of the BLAS pool numpy uses (the oracle's only parallel part)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def cpu_baseline(case_csa, case_hca, sample_tokens: int):
    """The float64 oracle, as it stands, on the first `sample_tokens` tokens
    (whole sequences first, the last one truncated to a multiple of 128)."""
    import torch
    import oracle
    threads = _blas_threads()
    cu = case_csa.cu_seqlens
    H = case_csa.H[:sample_tokens].to("cpu", torch.float64).numpy()
    W = {k: v.to("cpu", torch.float64).numpy() for k, v in case_csa.W.items()}
    Wh = {k: v.to("cpu", torch.float64).numpy() for k, v in case_hca.W.items()}
    b = {k: v.to("cpu", torch.float64).numpy() for k, v in case_csa.biases.items()}
    bh = case_hca.biases["B"].to("cpu", torch.float64).numpy()
    seqs = []
    for s, t in zip(cu[:-1], cu[1:]):
        if s >= sample_tokens:
            break
        seqs.append((int(s), int(min(t, sample_tokens))))
    entries = 0
    t0 = time.perf_counter()
    for s, t in seqs:
        Hs = H[s:t]
        e_c = oracle.csa_compress_sequence(Hs, W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], b["Ba"], b["Bb"], 4)
        e_h = oracle.hca_compress_sequence(Hs, Wh["W_KV"], Wh["W_Z"], bh, 128)
        oracle.fp8_entry_quantize(e_c)
        oracle.fp8_entry_quantize(e_h)
        entries += e_c.shape[0] + e_h.shape[0]
    dt = time.perf_counter() - t0
    tokens = sum(t - s for s, t in seqs)
    return {"value": entries / dt, "unit": "entries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {tokens} tokens of the batch ({len(seqs)} sequence(s)); float64 numpy oracle; "
                      f"{dt:.2f} s; {tokens / dt:.1f} tokens/s"}


def indexer_keys(sc, synth, torch, csa, lengths, steps):
    """The indexer-key compressor: the same fused CSA operator at c^I = 128
    over the same packed hidden states (its own weights and biases)."""
    cI = 128
    d = csa.H.shape[1]
    ik = synth.compressor_case("csa", lengths, d, cI, 4, seed=1, in_dtype="bf16", bias_std=0.02, device=csa.H.device,
                               H=csa.H)
    b = ik.biases
    call = lambda: sc.compress_fused("csa", ik.H, ik.Wt_cat, b["Ba"], b["Bb"], 4, ik.cu_seqlens, "bf16")
    call()
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    T = int(ik.H.shape[0])
    flops = 2.0 * T * d * 4 * cI
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"indexer keys: fused CSA m=4, c=128 over the same T={T} tokens, d={d}, bf16 out",
            "ms": ms, "entries_per_s": ik.n_entries / (ms * 1e-3), "tflops": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS}


def decode_append(sc, torch, csa, batches, steps):
    """Decode-time CSA append: nb sequences each complete one block of 4
    tokens (rows taken from the packed hidden states); the b-stream state is
    carried in place."""
    d = csa.H.shape[1]
    c = csa.c
    b = csa.biases
    res = {}
    for nb in batches:
        H = csa.H[: 4 * nb]
        state = sc.csa_empty_state(nb, c, H.device)
        call = lambda: sc.csa_append(H, csa.Wt_cat, b["Ba"], b["Bb"], state, "bf16", state_out=state)
        call()
        torch.cuda.synchronize()
        ev = _events(torch, 2)
        ev[0].record()
        for _ in range(steps):
            call()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        flops = 2.0 * 4 * nb * d * 4 * c
        wbytes = 4 * c * d * 2 + 4 * nb * d * 2          # weights + new hidden rows
        res[f"nb={nb}"] = {"us": ms * 1e3, "entries_per_s": nb / (ms * 1e-3),
                           "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "hbm_frac": wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return {"workload": f"CSA decode append, m=4, d={d}, c={c}: one new block per sequence, bf16 out, "
                        "state updated in place", "batches": res}


def rope_store(sc, torch, csa, steps):
    """Partial RoPE (last 64 dims) + bf16/fp8 mixed store of the fp32 CSA
    entries of the batch into a cache, one row per entry."""
    b = csa.biases
    ent, _ = sc.compress_fused("csa", csa.H, csa.Wt_cat, b["Ba"], b["Bb"], 4, csa.cu_seqlens, "f32")
    E, c = ent.shape
    r = 64
    cache = sc.rope_cache(E, c, r, ent.device)
    call = lambda: sc.rope_store(ent, 4, csa.cu_seqlens, cache, r)
    call()
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    nbytes = E * c * 4 + E * ((c - r) + 4 + 2 * r)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del ent, cache
    torch.cuda.empty_cache()
    return {"workload": f"RoPE store of the varlen CSA entries: E={E}, c={c}, r={r}, fp32 in, fp8+bf16 out",
            "us": ms * 1e3, "entries_per_s": E / (ms * 1e-3), "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}


def lightning_indexer(sc, synth, torch, steps, cpu_queries=2):
    """Lightning indexer at 1M context: 262144 compressed indexer keys
    (2^20 tokens, m = 4), the sequence's last 4096 tokens as queries (causal
    visibility), 64 heads x 128 dims bf16, fp32 head weights; k = 1024 and
    512.  MFMA-bound: 2 * 64 * 128 flops per visible (query, key) pair."""
    cfg = synth.CONFIGS["indexer_1m"]
    n_tok, T, m = cfg["n_tokens"], cfg["n_queries"], cfg["m"]
    dev = torch.device("cuda:0")
    case = synth.indexer_case([T], [n_tok // m], seed=0, device=dev)
    nv = synth.causal_visible(np.arange(n_tok - T, n_tok), m)
    pairs = float(nv.astype(np.float64).sum())
    flops = 2.0 * synth.INDEXER_HEADS * synth.INDEXER_DIM * pairs
    res = {"workload": f"indexer_1m: {n_tok // m} keys (n={n_tok}, m={m}), the last {T} tokens query with causal "
                       f"visibility, 64 heads x 128 bf16, fp32 head weights; ReLU scores + top-k",
           "flops_per_call": flops}
    for k in (cfg["k"], 512):
        call = lambda: sc.indexer_topk(case.q, case.w, case.keys, k, case.cu_q, case.cu_k, nv)
        call()
        torch.cuda.synchronize()
        ev = _events(torch, 2)
        ev[0].record()
        for _ in range(steps):
            call()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        tf = flops / (ms * 1e-3) / 1e12
        res[f"k={k}"] = {"ms": ms, "queries_per_s": T / (ms * 1e-3), "tflops": tf,
                         "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": tf / PEAK_BF16_TFLOPS, "traffic": _traffic("indexer_1m_topk"),
                                      "kernel": "indexer call (planner + indexer_topk_kernel)"}}
    # the float64 oracle on a few of the same queries, this host's cores
    import oracle
    rows = np.arange(T - cpu_queries, T)
    Q = case.q[-cpu_queries:].double().cpu().numpy()
    w = case.w[-cpu_queries:].double().cpu().numpy()
    K = case.keys.double().cpu().numpy()
    t0 = time.perf_counter()
    I = oracle.index_scores(Q, w, K, n_valid=nv[rows])
    oracle.top_k(I, cfg["k"])
    dt = time.perf_counter() - t0
    res["cpu_oracle"] = {"queries_per_s": cpu_queries / dt, "sample": f"{cpu_queries} queries x {n_tok // m} keys, "
                         f"k={cfg['k']}", "cores": _blas_threads(), "kind": "oracle"}
    del case
    torch.cuda.empty_cache()
    return res


def hca_attention(sc, synth, torch, steps, cpu_queries=2):
    """Dense shared-KV MQA with an attention sink over the HCA entries at 1M
    context: 8192 entries (2^20 tokens, m' = 128), the sequence's last 4096
    tokens as queries (causal visibility), 128 heads x 512 bf16, bf16 out.
    MFMA-bound: 4 * 128 * 512 flops per visible (query, entry) pair (scores
    and values)."""
    cfg = synth.CONFIGS["hca_mqa_1m"]
    n_tok, T, m = cfg["n_tokens"], cfg["n_queries"], cfg["m"]
    dev = torch.device("cuda:0")
    case = synth.mqa_case([T], [n_tok // m], seed=0, device=dev, q_std=cfg["q_std"])
    nv = synth.causal_visible(np.arange(n_tok - T, n_tok), m)
    pairs = float(nv.astype(np.float64).sum())
    flops = 4.0 * synth.MQA_HEADS * synth.MQA_DIM * pairs
    call = lambda: sc.shared_kv_mqa(case.q, case.kv, case.cu_q, case.cu_k, nv, case.k_sink, case.v_sink, None,
                                    "bf16")
    call()
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": f"hca_mqa_1m: {n_tok // m} entries (n={n_tok}, m'={m}), the last {T} tokens attend with "
                       "causal visibility, 128 heads x 512 bf16, attention sink with value, bf16 out",
           "flops_per_call": flops, "ms": ms, "queries_per_s": T / (ms * 1e-3), "tflops": tf,
           "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / PEAK_BF16_TFLOPS, "traffic": _traffic("hca_mqa_1m"),
                        "kernel": "attention call (planner + mqa_sink_kernel)"}}
    import oracle
    rows = np.arange(T - cpu_queries, T)
    Q = case.q[-cpu_queries:].double().cpu().numpy()
    KV = case.kv.double().cpu().numpy()
    ks = case.k_sink.double().cpu().numpy()
    vs = case.v_sink.double().cpu().numpy()
    t0 = time.perf_counter()
    oracle.shared_kv_mqa(Q, KV, nv[rows], 1.0 / np.sqrt(synth.MQA_DIM), ks, vs)
    dt = time.perf_counter() - t0
    res["cpu_oracle"] = {"queries_per_s": cpu_queries / dt, "sample": f"{cpu_queries} queries x {n_tok // m} entries",
                         "cores": _blas_threads(), "kind": "oracle"}
    del case
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--pool-steps", type=int, default=20)
    ap.add_argument("--cpu-sample-tokens", type=int, default=262144)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pool", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the indexer-key compressor, decode-append, RoPE-store, lightning-indexer and "
                         "HCA-attention measurements")
    ap.add_argument("--profile-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (torch copy kernel): the known-size reference that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this compressor build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_sequence_compression_amd as sc
    from kv_sequence_compression_amd import synth

    dev = torch.device("cuda:0")
    if args.profile_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = synth.CONFIGS["varlen_fp8"]
    lengths = synth.varlen_config_lengths(0)
    T = int(lengths.sum())
    d, c = cfg["d"], cfg["c"]
    common = dict(seed=0, in_dtype="bf16", bias_std=cfg["bias_std"], device=dev,
                  z_outlier_frac=cfg["z_outlier_frac"], z_outlier_scale=cfg["z_outlier_scale"])
    csa = synth.compressor_case("csa", lengths, d, c, cfg["m_csa"], per_sequence_h=True, **common)
    hca = synth.compressor_case("hca", lengths, d, c, cfg["m_hca"], H=csa.H, **common)   # same hidden states
    E_csa, E_hca = csa.n_entries, hca.n_entries
    bc, bh = csa.biases, hca.biases

    def step():
        sc.compress_fused("csa", csa.H, csa.Wt_cat, bc["Ba"], bc["Bb"], 4, csa.cu_seqlens, "fp8")
        sc.compress_fused("hca", hca.H, hca.Wt_cat, bh["B"], None, 128, hca.cu_seqlens, "fp8")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = _events(torch, 3 * args.steps)
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[3 * k].record()
        sc.compress_fused("csa", csa.H, csa.Wt_cat, bc["Ba"], bc["Bb"], 4, csa.cu_seqlens, "fp8")
        ev[3 * k + 1].record()
        sc.compress_fused("hca", hca.H, hca.Wt_cat, bh["B"], None, 128, hca.cu_seqlens, "fp8")
        ev[3 * k + 2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    csa_ms = float(np.mean([ev[3 * k].elapsed_time(ev[3 * k + 1]) for k in range(args.steps)]))
    hca_ms = float(np.mean([ev[3 * k + 1].elapsed_time(ev[3 * k + 2]) for k in range(args.steps)]))
    ms_step = wall * 1e3 / args.steps
    flops_csa = 2.0 * T * d * 4 * c
    flops_hca = 2.0 * T * d * 2 * c
    achieved = flops_csa / (csa_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": (E_csa + E_hca) / (ms_step * 1e-3),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "varlen_fp8: fused CSA (m=4) + fused HCA (m'=128) over 32 packed sequences, "
                               f"T={T}, d={d}, c={c}, fp8 E4M3 entries + per-entry fp32 scales",
                   "tokens": T, "entries_csa": E_csa, "entries_hca": E_hca, "seq_lengths": "U[4096,65536] step 128"},
        "tokens_per_s": T / (ms_step * 1e-3),
        "kernels_ms": {"fused_csa_call": csa_ms, "fused_hca_call": hca_ms},
        "hca_roofline_frac": flops_hca / (hca_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": _traffic("fused_csa_varlen"),
                     "kernel": "fused CSA call (tile kernel + planner + halo fix-up + fp8 encoder)",
                     "algorithmic_flops_per_launch": flops_csa},
    }
    _progress("compressor step timed")
    if not args.no_pool:
        pc = synth.pool_case(1 << 20, 512, seed=0, dtype="bf16", device=dev, bias_std=0.02)
        st, pb = pc.streams, pc.biases
        n = 1 << 20
        for _ in range(2):
            sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], pb["Ba"], pb["Bb"], 4, pc.cu_seqlens, "bf16")
            sc.pool_hca(st["Ca"], st["Za"], pb["B"], 128, pc.cu_seqlens, "bf16")
        torch.cuda.synchronize()
        pe = _events(torch, 3 * args.pool_steps)
        for k in range(args.pool_steps):
            pe[3 * k].record()
            sc.pool_csa(st["Ca"], st["Cb"], st["Za"], st["Zb"], pb["Ba"], pb["Bb"], 4, pc.cu_seqlens, "bf16")
            pe[3 * k + 1].record()
            sc.pool_hca(st["Ca"], st["Za"], pb["B"], 128, pc.cu_seqlens, "bf16")
            pe[3 * k + 2].record()
        torch.cuda.synchronize()
        pcsa = float(np.mean([pe[3 * k].elapsed_time(pe[3 * k + 1]) for k in range(args.pool_steps)]))
        phca = float(np.mean([pe[3 * k + 1].elapsed_time(pe[3 * k + 2]) for k in range(args.pool_steps)]))
        bytes_csa = 4 * n * 512 * 2 + (n // 4) * 512 * 2
        bytes_hca = 2 * n * 512 * 2 + (n // 128) * 512 * 2
        gbs_csa = bytes_csa / (pcsa * 1e-3) / 1e9
        out["pool_only"] = {
            "workload": "pool_long: four bf16 streams of 1048576 x 512; CSA m=4 -> 262144 entries, "
                        "HCA m'=128 on (C^a, Z^a) -> 8192 entries; bf16 out",
            "csa_ms": pcsa, "hca_ms": phca,
            "csa_entries_per_s": (n // 4) / (pcsa * 1e-3), "csa_tokens_per_s": n / (pcsa * 1e-3),
            "hca_entries_per_s": (n // 128) / (phca * 1e-3), "hca_tokens_per_s": n / (phca * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs_csa, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs_csa / PEAK_HBM_GBS, "traffic": _traffic("pool_csa_long"),
                         "kernel": "CSA pooling call", "algorithmic_bytes_per_launch": bytes_csa},
            "hca_roofline_frac": bytes_hca / (phca * 1e-3) / 1e9 / PEAK_HBM_GBS,
        }
        del pc, st
        torch.cuda.empty_cache()

    if not args.no_pool:
        _progress("pooling-only path measured")
    if not args.no_extras:
        out["indexer_keys"] = indexer_keys(sc, synth, torch, csa, lengths, args.steps)
        _progress("indexer-key compressor measured")
        out["decode_append"] = decode_append(sc, torch, csa, (64, 1024, 4096), args.steps)
        _progress("decode append measured")
        out["rope_store"] = rope_store(sc, torch, csa, args.steps)
        _progress("RoPE store measured")
        out["lightning_indexer"] = lightning_indexer(sc, synth, torch, args.steps)
        _progress("lightning indexer measured")
        out["hca_attention"] = hca_attention(sc, synth, torch, args.steps)
        _progress("HCA attention measured")

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(csa, hca, args.cpu_sample_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
