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
* csa_full (one sequence of 8192 tokens, 2048 entries) and hca_full (one
  sequence of 131072 tokens, 1024 entries), each with its own roofline, the
  projection alone and the unfused project-then-pool path beside it;
* the pooling-only path on the long-context streams (four bf16 streams of
  2^20 x 512; CSA m=4 and HCA m'=128), HBM-bound;
* the next-row kernels (indexer keys, decode append, RoPE store, lightning
  indexer, HCA dense attention);
* device: the GPU's properties and a measured 1 GiB device-to-device copy
  rate, beside the published peaks the fractions use;
* cpu_baseline: the float64 oracle on a bounded sample of the same workload
  (the first 262144 tokens of the batch) on this host's cores, the same on
  one core, and per workload (tiny, csa_full, hca_full, pooling) with all
  cores and with one; the host CPU model is recorded.

--legs selects measurements (e.g. for a profiler run of one kernel).
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
    None when the summary is missing or was taken on other sources of that
    kernel."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
        from kv_sequence_compression_amd.build import KERNEL_SOURCES, source_digest
        entry = rec["kernels"][kernel_key]
        if entry.get("source_digest") != source_digest(KERNEL_SOURCES[entry["sources"]]):
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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_cores() -> int:
    """Cores this process may run on (its affinity set), else os.cpu_count()."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _time_calls(torch, calls, steps: int, warmup: int = 2):
    """Median, minimum and mean time (ms) of one call, each call bracketed by
    HIP events on the current stream (the stream the library launches on).
    `calls` is one callable or a list that is cycled through (rotating input
    sets)."""
    calls = calls if isinstance(calls, (list, tuple)) else [calls]
    for k in range(max(warmup, len(calls))):
        calls[k % len(calls)]()
    torch.cuda.synchronize()
    ev = _events(torch, 2 * steps)
    for k in range(steps):
        ev[2 * k].record()
        calls[k % len(calls)]()
        ev[2 * k + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(steps)])
    return float(np.median(t)), float(t.min()), float(t.mean())


def _time_settled(torch, named, steps: int, warm_ms: float = 150.0):
    """{name: (median, minimum, mean) ms of one call} for several candidate
    paths, each timed in its steady state: it first runs alone for at least
    `warm_ms` (under a sustained matrix-core load the clock settles over
    ~100 ms, and settles differently after different work, so a path timed
    right after a short warm-up, or after another path, would be timed on a
    clock set by something else), then `steps` consecutive calls are timed.
    Each value is a callable or a list cycled through (rotating input sets)."""
    out = {}
    for n, c in named.items():
        seq = c if isinstance(c, (list, tuple)) else [c]
        t0 = time.perf_counter()
        k = 0
        while k < 2 or (time.perf_counter() - t0) * 1e3 < warm_ms:
            seq[k % len(seq)]()
            k += 1
            if k % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = _events(torch, 2 * steps)
        for j in range(steps):
            ev[2 * j].record()
            seq[(k + j) % len(seq)]()
            ev[2 * j + 1].record()
        torch.cuda.synchronize()
        t = np.array([ev[2 * j].elapsed_time(ev[2 * j + 1]) for j in range(steps)])
        out[n] = (float(np.median(t)), float(t.min()), float(t.mean()))
    return out


def device_record(torch, dev):
    """The device's properties and a measured plain device-to-device copy of
    1 GiB (torch copy: 1 GiB read + 1 GiB written), beside the published
    peaks the roofline fractions use."""
    p = torch.cuda.get_device_properties(dev)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    med, mn, _ = _time_calls(torch, lambda: dst.copy_(src), 9)
    del src, dst
    torch.cuda.empty_cache()
    rec = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "memory_gib": round(p.total_memory / 2 ** 30, 1),
           "copy_1gib": {"ms_median": med, "gbs_read_plus_write": 2 * 2 ** 30 / (med * 1e-3) / 1e9,
                         "frac_of_hbm_peak": 2 * 2 ** 30 / (med * 1e-3) / 1e9 / PEAK_HBM_GBS},
           "peaks": {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}}
    for attr in ("clock_rate", "L2_cache_size"):
        if hasattr(p, attr):
            rec[attr] = getattr(p, attr)
    return rec


def _mfma_roofline(flops: float, ms: float, kernel: str, traffic_key=None):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / PEAK_BF16_TFLOPS, "traffic": _traffic(traffic_key) if traffic_key else None,
            "kernel": kernel, "algorithmic_flops_per_launch": flops}


def _oracle_rate(fn, threads):
    """Seconds of fn() with the BLAS pool limited to `threads` (None: as is)."""
    from threadpoolctl import threadpool_limits
    if threads is None:
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0


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


def _f64(torch, t):
    return t.detach().to("cpu", torch.float64).numpy()


def csa_full_leg(sc, synth, torch, steps, cpu: bool):
    """CSA full workload: one sequence of 8192 tokens, d = 7168, c = 512,
    m = 4 -> 2048 entries, bf16 out.  Its hidden states (117 MB) would sit in
    the 256 MB last-level cache between calls, so three input sets are
    rotated; the weights are the same for every call, as in use.  Also timed:
    the projection alone (Y = H Wt^T, 8192 x 2048 bf16) and the unfused path
    (that projection, then CSA pooling of its column slices)."""
    cfg = synth.CONFIGS["csa_full"]
    dev = torch.device("cuda:0")
    T, d, c, m = cfg["lengths"][0], cfg["d"], cfg["c"], cfg["m"]
    case = synth.compressor_case("csa", cfg["lengths"], d, c, m, seed=0, in_dtype="bf16", bias_std=cfg["bias_std"],
                                 device=dev)
    Hs = [case.H] + [synth.normal((T, d), 1.0, (k, synth.TID["H"]), dev, "bf16") for k in (1, 2)]
    b = case.biases
    fused = [lambda H=H: sc.compress_fused("csa", H, case.Wt_cat, b["Ba"], b["Bb"], m, case.cu_seqlens, "bf16")
             for H in Hs]
    Y = torch.empty((T, 4 * c), dtype=torch.bfloat16, device=dev)
    proj = [lambda H=H: sc.project(H, case.Wt_cat, "bf16", out=Y) for H in Hs]

    def unfused_call(H):
        sc.project(H, case.Wt_cat, "bf16", out=Y)
        sc.pool_csa(Y[:, :c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:], b["Ba"], b["Bb"], m, case.cu_seqlens,
                    "bf16")
    unfused = [lambda H=H: unfused_call(H) for H in Hs]
    # yardstick: torch.mm (hipBLASLt) on the same product, weights as a
    # contiguous [d x 4c] matrix, output to a preallocated buffer
    Wdn = case.Wt_cat.t().contiguous()
    Yr = torch.empty((T, 4 * c), dtype=torch.bfloat16, device=dev)
    blas = [lambda H=H: torch.mm(H, Wdn, out=Yr) for H in Hs]
    r = _time_settled(torch, {"fused": fused, "proj": proj, "unfused": unfused, "blas": blas}, steps)
    (med, mn, mean), (pmed, pmn, _), (umed, umn, _), (bmed, bmn, _) = r["fused"], r["proj"], r["unfused"], r["blas"]
    flops = 2.0 * T * d * 4 * c
    E = T // m
    res = {"workload": f"csa_full: one sequence, n={T}, d={d}, c={c}, m={m} -> {E} entries, bf16 in/out "
                       "(3 rotating hidden-state sets)",
           "timing": f"each path alone for >= 150 ms, then {steps} consecutive calls timed with HIP events",
           "ms_median": med, "ms_min": mn, "entries_per_s": E / (med * 1e-3), "tokens_per_s": T / (med * 1e-3),
           "roofline": _mfma_roofline(flops, med, "fused CSA call (planner + tile kernel + halo fix-up)",
                                      "fused_csa_full"),
           "project_alone": {"ms_median": pmed, "ms_min": pmn,
                             "roofline": _mfma_roofline(flops, pmed, "seqcomp_project, 8192 x 2048 bf16 out",
                                                        "project_csa_full")},
           "unfused": {"ms_median": umed, "ms_min": umn, "entries_per_s": E / (umed * 1e-3),
                       "fused_speedup": umed / med,
                       "path": "seqcomp_project to bf16 [T x 4c], then seqcomp_pool_csa on its column slices"},
           "hipblaslt_mm": {"ms_median": bmed, "ms_min": bmn,
                            "roofline": _mfma_roofline(flops, bmed, "torch.mm (hipBLASLt), the same product")}}
    if cpu:
        import oracle
        ne = 256                                            # first 256 entries: 1024 tokens
        H = _f64(torch, case.H[:ne * m])
        W = {k: _f64(torch, v) for k, v in case.W.items()}
        bb = {k: _f64(torch, v) for k, v in b.items()}
        run = lambda: oracle.csa_compress_sequence(H, W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], bb["Ba"],
                                                   bb["Bb"], m)
        res["cpu_oracle"] = _oracle_legs(run, ne, ne * m, f"first {ne} entries ({ne * m} tokens)")
    del case, Hs, Y, Yr, Wdn
    torch.cuda.empty_cache()
    return res


def hca_full_leg(sc, synth, torch, steps, cpu: bool):
    """HCA workload: one sequence of 131072 tokens, d = 7168, c = 512,
    m' = 128 -> 1024 entries, bf16 out (hidden states 1.9 GB, far past the
    last-level cache).  Also the projection alone and the unfused path."""
    cfg = synth.CONFIGS["hca_full"]
    dev = torch.device("cuda:0")
    T, d, c, m = cfg["lengths"][0], cfg["d"], cfg["c"], cfg["m"]
    case = synth.compressor_case("hca", cfg["lengths"], d, c, m, seed=0, in_dtype="bf16", bias_std=cfg["bias_std"],
                                 device=dev)
    B = case.biases["B"]
    fused = lambda: sc.compress_fused("hca", case.H, case.Wt_cat, B, None, m, case.cu_seqlens, "bf16")
    Y = torch.empty((T, 2 * c), dtype=torch.bfloat16, device=dev)
    proj = lambda: sc.project(case.H, case.Wt_cat, "bf16", out=Y)

    def unfused():
        proj()
        sc.pool_hca(Y[:, :c], Y[:, c:], B, m, case.cu_seqlens, "bf16")
    Wdn = case.Wt_cat.t().contiguous()
    Yr = torch.empty((T, 2 * c), dtype=torch.bfloat16, device=dev)
    blas = lambda: torch.mm(case.H, Wdn, out=Yr)
    r = _time_settled(torch, {"fused": fused, "proj": proj, "unfused": unfused, "blas": blas}, steps)
    (med, mn, _), (pmed, pmn, _), (umed, umn, _), (bmed, bmn, _) = r["fused"], r["proj"], r["unfused"], r["blas"]
    flops = 2.0 * T * d * 2 * c
    E = T // m
    res = {"workload": f"hca_full: one sequence, n={T}, d={d}, c={c}, m'={m} -> {E} entries, bf16 in/out",
           "timing": f"each path alone for >= 150 ms, then {steps} consecutive calls timed with HIP events",
           "ms_median": med, "ms_min": mn, "entries_per_s": E / (med * 1e-3), "tokens_per_s": T / (med * 1e-3),
           "roofline": _mfma_roofline(flops, med, "fused HCA call (planner + tile kernel)", "fused_hca_full"),
           "project_alone": {"ms_median": pmed, "ms_min": pmn,
                             "roofline": _mfma_roofline(flops, pmed, "seqcomp_project, 131072 x 1024 bf16 out",
                                                        "project_hca_full")},
           "unfused": {"ms_median": umed, "ms_min": umn, "entries_per_s": E / (umed * 1e-3),
                       "fused_speedup": umed / med,
                       "path": "seqcomp_project to bf16 [T x 2c], then seqcomp_pool_hca on its column slices"},
           "hipblaslt_mm": {"ms_median": bmed, "ms_min": bmn,
                            "roofline": _mfma_roofline(flops, bmed, "torch.mm (hipBLASLt), the same product")}}
    if cpu:
        import oracle
        ne = 16                                             # first 16 entries: 2048 tokens
        H = _f64(torch, case.H[:ne * m])
        W = {k: _f64(torch, v) for k, v in case.W.items()}
        Bh = _f64(torch, B)
        run = lambda: oracle.hca_compress_sequence(H, W["W_KV"], W["W_Z"], Bh, m)
        res["cpu_oracle"] = _oracle_legs(run, ne, ne * m, f"first {ne} entries ({ne * m} tokens)")
    del case, Y, Yr, Wdn
    torch.cuda.empty_cache()
    return res


def _oracle_legs(run, entries: int, tokens: int, sample: str):
    """The oracle on a sample, with every thread of its BLAS pool (the host
    cores this process is given) and with one."""
    out = {"kind": "oracle", "sample": sample, "cpu_model": _cpu_model()}
    for name, threads in (("all_cores", None), ("one_core", 1)):
        dt = _oracle_rate(run, threads)
        out[name] = {"cores": _blas_threads() if threads is None else threads, "seconds": dt,
                     "entries_per_s": entries / dt, "tokens_per_s": tokens / dt}
    return out


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


def decode_append(sc, torch, csa, batches, steps, reps=5):
    """Decode-time CSA append: nb sequences each complete one block of 4
    tokens (rows taken from the packed hidden states); the b-stream state is
    carried in place.  `us` is the device time of one call: `steps` calls
    captured in a HIP graph, replayed `reps` times between two events (the
    library launches kernels only: no copies, fills or synchronisations).
    `us_eager` is the rate of the same calls made one by one from Python,
    binding overhead included.  `hipblaslt_mm_us` times torch.mm on the
    projection alone (same rows and weights, bf16 out) the same way: a
    yardstick for the skinny product, with no pooling or state."""
    d = csa.H.shape[1]
    c = csa.c
    b = csa.biases
    res = {}
    Wdn = csa.Wt_cat.t().contiguous()
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
        eager_ms = ev[0].elapsed_time(ev[1]) / steps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                call()
        g.replay()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / (reps * steps)
        del g
        # yardstick: torch.mm (hipBLASLt) on the projection alone, same
        # graph-replay timing, no pooling
        Yr = torch.empty((4 * nb, 4 * c), dtype=torch.bfloat16, device=H.device)
        blas = lambda: torch.mm(H, Wdn, out=Yr)
        blas()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                blas()
        g.replay()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        blas_ms = ev[0].elapsed_time(ev[1]) / (reps * steps)
        del g
        flops = 2.0 * 4 * nb * d * 4 * c
        wbytes = 4 * c * d * 2 + 4 * nb * d * 2          # weights + new hidden rows
        res[f"nb={nb}"] = {"us": ms * 1e3, "us_eager": eager_ms * 1e3, "hipblaslt_mm_us": blas_ms * 1e3,
                           "entries_per_s": nb / (ms * 1e-3),
                           "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "hbm_frac": wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return {"workload": f"CSA decode append, m=4, d={d}, c={c}: one new block per sequence, bf16 out, "
                        "state updated in place", "timing": "device time per call from HIP graph replay; "
                        "us_eager: one Python call after another", "batches": res}


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


LEGS = ("step", "csa_full", "hca_full", "pool", "indexer_keys", "decode_append", "rope_store", "lightning_indexer",
        "hca_attention")


def mfma_ceiling(torch, reps: int = 3, iters: int = 57344):
    """Sustained rate of the bf16 matrix cores with no data movement (the
    measurement-only seqcomp_probe_mfma: 16 independent 32x32x16 MFMA chains
    per wave on random bf16 operands in registers, one wave per SIMD, ~20 ms
    per call): the power-limited ceiling of the instruction the tile kernels
    use."""
    import ctypes
    path = os.path.join(ROOT, "kv_sequence_compression_amd", "libseqcomp_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.seqcomp_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    data = torch.randn((cus * 256 * 128,), dtype=torch.bfloat16, device=dev)
    sink = torch.empty((cus * 256,), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda: fn(ctypes.c_void_p(data.data_ptr()), iters, ctypes.c_void_p(sink.data_ptr()), stream)
    med, mn, mean = _time_calls(torch, call, reps, warmup=1)
    flops = float(iters) * 16 * 32768 * 4 * cus
    tf = flops / (med * 1e-3) / 1e12
    del data, sink
    return {"tflops": tf, "frac": tf / PEAK_BF16_TFLOPS, "ms": med,
            "probe": "kv_sequence_compression_amd/probe/ceilings.hip (seqcomp_probe_mfma)"}


def pool_ceiling(torch, st, n, steps, bytes_csa, csa_ms):
    """The CSA pooling call's memory traffic with no arithmetic (the
    measurement-only stream_mix probe): the same rows read in the same order
    with non-temporal loads, with and without the 1 KiB output row per entry.
    The read+write rate is the ceiling the pooling call is held against."""
    import ctypes
    path = os.path.join(ROOT, "kv_sequence_compression_amd", "libseqcomp_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.seqcomp_probe_stream_mix
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    dst = torch.empty((n // 4, 512), dtype=torch.bfloat16, device=st["Ca"].device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [ctypes.c_void_p(st[k].data_ptr()) for k in ("Ca", "Cb", "Za", "Zb")]
    res = {}
    for name, write, nbytes in (("read_only", 0, 4 * n * 1024), ("read_write", 1, bytes_csa)):
        call = lambda: fn(*ptrs, n // 4, ctypes.c_void_p(dst.data_ptr()), write, stream)
        _, _, mean = _time_calls(torch, call, steps)
        res[name] = {"ms": mean, "tbs": nbytes / (mean * 1e-3) / 1e12}
    res["pool_csa_over_read_write"] = res["read_write"]["ms"] / csa_ms
    res["probe"] = "kv_sequence_compression_amd/probe/ceilings.hip (seqcomp_probe_stream_mix)"
    del dst
    return res


def tiny_cpu_oracle(synth, torch):
    """The oracle on the whole tiny CSA workload (n = 64, d = 64, c = 32,
    m = 4), repeated for a measurable time."""
    import oracle
    cfg = synth.CONFIGS["csa_tiny"]
    case = synth.compressor_case("csa", cfg["lengths"], cfg["d"], cfg["c"], cfg["m"], seed=0, in_dtype="f32",
                                 bias_std=cfg["bias_std"], device="cpu")
    H = _f64(torch, case.H)
    W = {k: _f64(torch, v) for k, v in case.W.items()}
    b = {k: _f64(torch, v) for k, v in case.biases.items()}
    reps = 200

    def run():
        for _ in range(reps):
            oracle.csa_compress(H, W["W_KVa"], W["W_KVb"], W["W_Za"], W["W_Zb"], b["Ba"], b["Bb"], 4, case.cu_seqlens)
    return _oracle_legs(run, 16 * reps, 64 * reps, f"the whole workload (16 entries) x {reps}")


def pool_cpu_oracle(torch, pc):
    """The oracle's pooling on the first 4096 CSA entries (16384 rows) and the
    first 128 HCA entries (16384 rows) of the long-context streams."""
    import oracle
    rows = 16384
    st = {k: _f64(torch, v[:rows]) for k, v in pc.streams.items()}
    b = {k: _f64(torch, v) for k, v in pc.biases.items()}
    csa = _oracle_legs(lambda: oracle.csa_pool_sequence(st["Ca"], st["Cb"], st["Za"], st["Zb"], b["Ba"], b["Bb"], 4),
                       rows // 4, rows, f"first {rows // 4} CSA entries ({rows} rows of 4 streams)")
    hca = _oracle_legs(lambda: oracle.hca_pool_sequence(st["Ca"], st["Za"], b["B"], 128),
                       rows // 128, rows, f"first {rows // 128} HCA entries ({rows} rows of 2 streams)")
    return {"csa": csa, "hca": hca}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps first: the clock settles over ~100 ms of sustained matrix-core load")
    ap.add_argument("--pool-steps", type=int, default=20)
    ap.add_argument("--cpu-sample-tokens", type=int, default=262144)
    ap.add_argument("--cpu-one-core-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated measurements to run (default: all): " + ", ".join(LEGS))
    ap.add_argument("--no-pool", action="store_true", help="same as leaving 'pool' out of --legs")
    ap.add_argument("--no-extras", action="store_true",
                    help="leave out the indexer-key compressor, decode-append, RoPE-store, lightning-indexer and "
                         "HCA-attention measurements")
    ap.add_argument("--profile-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (torch copy kernel): the known-size reference that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this compressor build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    legs = [x for x in args.legs.split(",") if x]
    unknown = set(legs) - set(LEGS)
    if unknown:
        print(f"unknown legs: {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)
    if args.no_pool:
        legs = [x for x in legs if x != "pool"]
    if args.no_extras:
        legs = [x for x in legs if x not in ("indexer_keys", "decode_append", "rope_store", "lightning_indexer",
                                             "hca_attention")]
    cpu = not args.no_cpu_baseline

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
    out = {"metric": METRIC, "value": None, "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "varlen_fp8: fused CSA (m=4) + fused HCA (m'=128) over 32 packed sequences, "
                                  f"T={T}, d={d}, c={c}, fp8 E4M3 entries + per-entry fp32 scales",
                      "tokens": T, "seq_lengths": "U[4096,65536] step 128"}}
    out["device"] = device_record(torch, dev)
    need_varlen = any(x in legs for x in ("step", "indexer_keys", "decode_append", "rope_store"))
    if need_varlen:
        common = dict(seed=0, in_dtype="bf16", bias_std=cfg["bias_std"], device=dev,
                      z_outlier_frac=cfg["z_outlier_frac"], z_outlier_scale=cfg["z_outlier_scale"])
        csa = synth.compressor_case("csa", lengths, d, c, cfg["m_csa"], per_sequence_h=True, **common)
        hca = synth.compressor_case("hca", lengths, d, c, cfg["m_hca"], H=csa.H, **common)   # same hidden states
        E_csa, E_hca = csa.n_entries, hca.n_entries
        bc, bh = csa.biases, hca.biases
        out["config"].update({"entries_csa": E_csa, "entries_hca": E_hca})

    if "step" in legs:
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
        out.update({
            "value": (E_csa + E_hca) / (ms_step * 1e-3),
            "ms_per_step": ms_step,
            "tokens_per_s": T / (ms_step * 1e-3),
            "kernels_ms": {"fused_csa_call": csa_ms, "fused_hca_call": hca_ms},
            "hca_roofline_frac": flops_hca / (hca_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "roofline": _mfma_roofline(flops_csa, csa_ms,
                                       "fused CSA call (tile kernel + planner + halo fix-up + fp8 encoder)",
                                       "fused_csa_varlen"),
        })
        _progress("compressor step timed")
    if "csa_full" in legs:
        out["csa_full"] = csa_full_leg(sc, synth, torch, max(args.steps, 20), cpu)
        _progress("CSA full workload measured")
    if "hca_full" in legs:
        out["hca_full"] = hca_full_leg(sc, synth, torch, max(args.steps, 10), cpu)
        _progress("HCA workload measured")
    if any(x in legs for x in ("step", "csa_full", "hca_full")):
        ceil = mfma_ceiling(torch)
        if ceil is not None:
            out["mfma_ceiling"] = ceil
            for key in ("roofline", "csa_full", "hca_full"):
                r = out.get(key)
                r = r.get("roofline", r) if isinstance(r, dict) and key != "roofline" else r
                if isinstance(r, dict) and "achieved" in r:
                    r["frac_of_mfma_ceiling"] = r["achieved"] / ceil["tflops"]
            _progress("matrix-core ceiling measured")
    if "pool" in legs:
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
        gbs_hca = bytes_hca / (phca * 1e-3) / 1e9
        out["pool_only"] = {
            "workload": "pool_long: four bf16 streams of 1048576 x 512; CSA m=4 -> 262144 entries, "
                        "HCA m'=128 on (C^a, Z^a) -> 8192 entries; bf16 out",
            "csa_ms": pcsa, "hca_ms": phca,
            "csa_entries_per_s": (n // 4) / (pcsa * 1e-3), "csa_tokens_per_s": n / (pcsa * 1e-3),
            "hca_entries_per_s": (n // 128) / (phca * 1e-3), "hca_tokens_per_s": n / (phca * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs_csa, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs_csa / PEAK_HBM_GBS, "traffic": _traffic("pool_csa_long"),
                         "kernel": "CSA pooling call", "algorithmic_bytes_per_launch": bytes_csa},
            "hca_roofline": {"bound": "hbm", "achieved": gbs_hca, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": gbs_hca / PEAK_HBM_GBS, "traffic": _traffic("pool_hca_long"),
                             "kernel": "HCA pooling call", "algorithmic_bytes_per_launch": bytes_hca},
            "hca_roofline_frac": gbs_hca / PEAK_HBM_GBS,
        }
        out["pool_only"]["ceiling"] = pool_ceiling(torch, st, n, args.pool_steps, bytes_csa, pcsa)
        if cpu:
            out["pool_only"]["cpu_oracle"] = pool_cpu_oracle(torch, pc)
        del pc, st
        torch.cuda.empty_cache()
        _progress("pooling-only path measured")
    if "indexer_keys" in legs:
        out["indexer_keys"] = indexer_keys(sc, synth, torch, csa, lengths, args.steps)
        _progress("indexer-key compressor measured")
    if "decode_append" in legs:
        out["decode_append"] = decode_append(sc, torch, csa, (1, 64, 256, 512, 1024, 4096), args.steps)
        _progress("decode append measured")
    if "rope_store" in legs:
        out["rope_store"] = rope_store(sc, torch, csa, args.steps)
        _progress("RoPE store measured")
    if "lightning_indexer" in legs:
        out["lightning_indexer"] = lightning_indexer(sc, synth, torch, args.steps)
        _progress("lightning indexer measured")
    if "hca_attention" in legs:
        out["hca_attention"] = hca_attention(sc, synth, torch, args.steps)
        _progress("HCA attention measured")

    if cpu and "step" in legs:
        base = cpu_baseline(csa, hca, args.cpu_sample_tokens)
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = cpu_baseline(csa, hca, args.cpu_one_core_tokens)
        base["one_core"] = one
        base["cpu_model"] = _cpu_model()
        base["host_cores"] = _host_cores()
        base["csa_tiny"] = tiny_cpu_oracle(synth, torch)
        out["cpu_baseline"] = base
        _progress("oracle baselines timed")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
