"""Float64 CPU oracle for the token-level KV sequence compressor.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
helper with the HIP library under ``kv_sequence_compression_amd/``.

Sources (web pages, cited by title and equation/table label):

* "序列压缩注意力" (sequence-compressed attention) -- eq. attn-seqcomp-csa-proj,
  eq. attn-seqcomp-csa-softmax, eq. attn-seqcomp-csa-pool,
  eq. attn-seqcomp-overlap-bound, eq. attn-seqcomp-hca,
  table tbl-attn-seqcomp-overlap.
* "Ch 04 · CSA — 长上下文的快通道" -- section 3 (token-level compressor,
  the 12-token worked example) and section 4 (lightning indexer).
* "Ch 05 · HCA — 长上下文的全景镜" -- section 2 (HCA compression formula and
  the dense attention over the entries), the section on partial RoPE and the
  attention sink.
* "混合压缩注意力双方案解析：CSA与HCA技术对比与选型指南" -- section 3
  (mixed-precision storage).

Every function is pinned (``tests/test_oracle_*pins.py``) against facts that
do not come from the oracle itself (exact rational arithmetic, closed forms,
the worked example, library routines for the special cases).  No function
here is "parity unpinned".
"""

from .compressor import (  # noqa: F401
    n_entries,
    project,
    csa_pool_sequence,
    hca_pool_sequence,
    csa_pool,
    hca_pool,
    csa_compress_sequence,
    hca_compress_sequence,
    csa_compress,
    hca_compress,
)
from .encode import (  # noqa: F401
    round_bf16,
    fp8_e4m3_decode,
    fp8_e4m3_encode,
    fp8_entry_quantize,
    FP8_E4M3_MAX,
)
from .rope_store import (  # noqa: F401
    entry_positions,
    rope_partial,
    rope_mixed_store,
)
from .indexer import (  # noqa: F401
    index_scores,
    top_k,
)
from .mqa import (  # noqa: F401
    shared_kv_mqa,
)
