"""CPU oracle for the SpargeAttn hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, numpy-fp64 implementation of what the GPU library computes.  Only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product path (``block_sparse_quantized_amd``) never imports,
links or calls anything in this package, and this package shares no code with it
(no kernels, headers, helpers or constant tables).

Citations name the page and the section they follow.  Page legend:
  [topgit]     "SpargeAttn: accelerate LLM inference without training" (topgit.dev)
  [readme]     "Sparge Attention" (GitHub README mirror, git.1-hub.cn)
  [chapterpal] "SpargeAttention: Accurate and Training-free Sparse Attention
               Accelerating Any Model Inference" (chapterpal.com summary)
  [gittools]   "SpargeAttention" (Chinese README mirror, gittoolsai.com)
  [abstract]   the paper abstract on codewithpapers.app

Parity status: every function is pinned by tests under ``tests/`` marked
``not gpu`` (closed forms, library routines, brute force, invariants), except the
ones listed as "parity unpinned" in their docstrings: the exact Hilbert variant is
a convention pinned only by its curve properties and by agreement of two
independent implementations (forward here, inverse in the library).
"""

from .sparge_oracle import (  # noqa: F401
    BQ,
    BK,
    num_blocks,
    block_valid,
    block_stats,
    pooled_scores,
    keep_count,
    select_row,
    predict_mask,
    predict_mask_all,
    kept_lists,
    attend_group,
    attend_head,
    attend_rows,
    quantize_blocks,
    smooth_k,
    smooth_k_blocks,
    k_block_means,
    Q_QUANT_ROWS,
    int8_qk_inputs,
    attend_head_int8_sim,
    row_softmax,
    OracleParams,
)
from .hilbert_ref import hilbert_cell_order, hilbert_index_to_axes  # noqa: F401
