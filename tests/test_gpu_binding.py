"""Argument checks of the Python binding that need device tensors: mixed
host and device inputs, offsets past the rows given, an entry count that
disagrees with the offsets.  Each call raises before any kernel launch."""

import numpy as np
import pytest
import torch

import kv_sequence_compression_amd as sc
from kv_sequence_compression_amd import synth

pytestmark = pytest.mark.gpu


def test_fused_rejects_mixed_devices_and_short_inputs(gpu_device):
    case = synth.compressor_case("csa", [300], 64, 32, 4, seed=60, in_dtype="bf16", device=gpu_device)
    b = case.biases
    with pytest.raises(ValueError, match="Bb must be on a GPU"):
        sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"].cpu(), 4, None)
    with pytest.raises(ValueError, match="past the 300 rows"):
        sc.compress_fused("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, [0, 200, 400])
    with pytest.raises(ValueError, match="past the 300 rows"):
        sc.compress_fused_noalloc("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, [0, 304])
    with pytest.raises(ValueError, match="out must have shape"):
        sc.compress_fused_noalloc("csa", case.H, case.Wt_cat, b["Ba"], b["Bb"], 4, None, "bf16",
                                  out=torch.empty((74, 32), dtype=torch.bfloat16, device=gpu_device))
    Y = sc.project(case.H, case.Wt_cat, "bf16")
    with pytest.raises(ValueError, match="past the 300 rows"):
        sc.pool_csa(Y[:, :32], Y[:, 32:64], Y[:, 64:96], Y[:, 96:], b["Ba"], b["Bb"], 4, [0, 301])


def test_rope_and_attention_reject_mismatched_counts(gpu_device):
    ent = torch.zeros((10, 128), dtype=torch.float32, device=gpu_device)
    cache = sc.rope_cache(16, 128, 64, gpu_device)
    with pytest.raises(ValueError, match="give 11 entries"):
        sc.rope_store(ent, 4, [0, 44], cache, 64)
    with pytest.raises(ValueError, match="one cache row per entry"):
        sc.rope_store(ent, 4, [0, 40], cache, 64, slots=np.arange(9))
    with pytest.raises(ValueError, match="one position per sequence"):
        sc.rope_store(ent, 4, [0, 40], cache, 64, pos0=[1, 2])
    q = torch.zeros((4, 128, 512), dtype=torch.bfloat16, device=gpu_device)
    kv = torch.zeros((20, 512), dtype=torch.bfloat16, device=gpu_device)
    with pytest.raises(ValueError, match="cu_k reaches row 21"):
        sc.shared_kv_mqa(q, kv, [0, 4], [0, 21])
    with pytest.raises(ValueError, match="one count per query"):
        sc.shared_kv_mqa(q, kv, n_valid=[20, 20, 20])
    qi = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device=gpu_device)
    w = torch.zeros((4, 64), dtype=torch.float32, device=gpu_device)
    keys = torch.zeros((20, 128), dtype=torch.bfloat16, device=gpu_device)
    with pytest.raises(ValueError, match="cu_q reaches row 5"):
        sc.indexer_topk(qi, w, keys, 8, [0, 5], [0, 20])
