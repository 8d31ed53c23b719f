"""The compressor's calls under HIP graph capture (serving loops, captured
decode steps): each graph is replayed several times, with eager work and
synchronisations between the replays, and every replay must equal the eager
result bit for bit (the same kernels on the same inputs).  The library
launches kernels only -- no copies, fills or allocations inside a call -- so
a captured call replays as it ran."""

import gc
import weakref

import numpy as np
import pytest
import torch

import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth

pytestmark = pytest.mark.gpu


def _replays(g, check, n=3):
    for i in range(n):
        noise = torch.randn(1 << 20, device="cuda")          # eager work between replays
        (noise * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        check(i)


@pytest.mark.parametrize("mode,out_dtype,noalloc", [("csa", "fp8", False), ("hca", "bf16", False),
                                                    ("csa", "bf16", True), ("hca", "fp8", True)])
def test_fused_call_captured(gpu_device, mode, out_dtype, noalloc):
    m = 4 if mode == "csa" else 128
    case = synth.compressor_case(mode, [1500, 7, 2300], 256, 128, m, seed=50, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    b = case.biases
    Ba, Bb = (b["Ba"], b["Bb"]) if mode == "csa" else (b["B"], None)
    call = sc.compress_fused_noalloc if noalloc else sc.compress_fused
    s = torch.cuda.Stream(gpu_device)
    with torch.cuda.stream(s):
        ref, ref_scale = call(mode, case.H, case.Wt_cat, Ba, Bb, m, case.cu_seqlens, out_dtype)   # also warms the
    s.synchronize()                                                                               # offsets' copy
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out, scale = call(mode, case.H, case.Wt_cat, Ba, Bb, m, case.cu_seqlens, out_dtype)

    def check(i):
        assert torch.equal(out, ref), f"replay {i}"
        if ref_scale is not None:
            assert torch.equal(scale, ref_scale), f"replay {i}"
    _replays(g, check)


def test_decode_append_captured(gpu_device):
    """Three appends per replay, the state carried in place: every replay
    starts from the same saved state and must give the eager entries and
    final state."""
    d, c, nb = 512, 128, 40
    case = synth.compressor_case("csa", [4 * nb * 3], d, c, 4, seed=51, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    b = case.biases
    Hs = [case.H[k * 4 * nb:(k + 1) * 4 * nb] for k in range(3)]
    s = torch.cuda.Stream(gpu_device)
    with torch.cuda.stream(s):
        state = sc.csa_empty_state(nb, c, gpu_device)
        ref = [sc.csa_append(H, case.Wt_cat, b["Ba"], b["Bb"], state, "bf16", state_out=state)[0] for H in Hs]
        ref_state = state.clone()
        state0 = sc.csa_empty_state(nb, c, gpu_device)
        state.copy_(state0)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = [sc.csa_append(H, case.Wt_cat, b["Ba"], b["Bb"], state, "bf16", state_out=state)[0] for H in Hs]

    def check(i):
        for k in range(3):
            assert torch.equal(outs[k], ref[k]), f"replay {i}, append {k}"
        assert torch.equal(state, ref_state), f"replay {i}"
        state.copy_(state0)                                   # the next replay starts from the empty state
        torch.cuda.synchronize()
    _replays(g, check)


def test_capture_refuses_an_uncached_host_copy(gpu_device):
    """Offsets that were never copied on the capturing stream are refused
    with a clear error instead of capturing a copy from a temporary buffer."""
    case = synth.compressor_case("hca", [1024], 128, 32, 128, seed=52, in_dtype="bf16", device=gpu_device)
    s = torch.cuda.Stream(gpu_device)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="graph capture"):
        with torch.cuda.graph(g, stream=s):
            sc.compress_fused("hca", case.H, case.Wt_cat, case.biases["B"], None, 128, [0, 1024 - 128, 1024],
                              "bf16")


def test_captured_offsets_outlive_cache_eviction(gpu_device):
    """The device copy of the offsets that a captured call reads stays
    allocated after the binding's cache has evicted it (more than its 64
    layouts seen since), so the allocator cannot hand that memory to another
    tensor; replays after the flood still equal the eager result.  The copy's
    survival is checked before any replay."""
    case = synth.compressor_case("csa", [900, 260], 128, 64, 4, seed=53, in_dtype="bf16", bias_std=0.3,
                                 device=gpu_device)
    b = case.biases
    s = torch.cuda.Stream(gpu_device)
    with torch.cuda.stream(s):
        ref, _ = sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, case.cu_seqlens, "bf16")
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out, _ = sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, case.cu_seqlens, "bf16")
    host = np.ascontiguousarray(np.asarray(case.cu_seqlens, dtype=np.int64))
    with torch.cuda.stream(s):
        captured = weakref.ref(sc._to_device(host, torch.int64, gpu_device))   # the cached copy the graph reads
        for k in range(100):                                                   # evict it from the cache
            sc._to_device(np.array([0, 4 * (k + 1), 4 * (k + 2)], dtype=np.int64), torch.int64, gpu_device)
    s.synchronize()
    gc.collect()
    assert captured() is not None, "the captured offsets' device copy was freed"

    def check(i):
        assert torch.equal(out, ref), f"replay {i}"
    _replays(g, check)
