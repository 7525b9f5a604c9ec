"""Float64 CPU oracle of the compressed sparse attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or helper with the HIP library; the two meet only through the seeded
inputs of the ``synth`` package.

Pages cited (by title, section and figure):

* [V4] "DeepSeek-V4: エージェントが実際に使える100万トークンのコンテキスト"
  (Japanese translation of the DeepSeek-V4 blog post), section
  "ハイブリッド注意：CSAとHCA" and its figures 3 (CSA) and 4 (HCA).
* [V4.1] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
  (wiki digest of the V4.1-Flash technical report), sections
  "アーキテクチャ" (CED, CSA2, Hierarchical Sparse Indexer, FP4 main KV
  cache), Figures 4 and 5, and "推論カーネル".

Every function implements the plain definition, step by step, in float64,
from the byte-level inputs.  Where the pages leave a point open the
docstring names the reading taken.  Parity of the final numbers is pinned
by invariants, closed forms, library routines and brute force in
``tests/test_oracle_*.py``; the absolute values of the outputs follow the
readings, which the pages do not fix numerically (no worked example is
printed on any page).
"""

from .formats import (  # noqa: F401
    bf16_to_f64,
    f32_to_bf16,
    e4m3_to_f64,
    e2m1_to_f64,
    e8m0_to_f64,
    mxfp4_encode,
    mxfp4_decode,
    mxfp8_encode,
    mxfp8_decode,
    E2M1_VALUES,
    E4M3_VALUES,
)
from .csa import (  # noqa: F401
    visible_count,
    pool_block,
    compress,
    compress_hidden,
    decode_entries,
    index_scores,
    topk_select,
    index_topk,
    attention,
    rope_rotate,
    sparse_attention,
    dense_attention,
    csa2_pair,
    block_pool,
    hier_pair,
    csa2_stack,
    swa_encode,
    swa_decode,
    FULL,
    REINDEX,
    REUSE,
    CAND_AUTO,
    CAND_SCAN,
    CAND_SELECTION,
    CAND_POOL,
)
