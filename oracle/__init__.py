"""Plain fp64 CPU oracle for the long-context sparse prefill path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library and does not
import it.

Every function is a direct, slow, readable statement of what the pages define,
computed in float64 with numpy (a matrix product, a sort, exp/log are the only
library primitives used).  Sources are cited by page and section:

* [Qwen2.5-1M explainer] "論文解説: Qwen2.5-1M — 100万トークンコンテキストを実現する
  長文脈LLMの設計と推論最適化" (0h-n0.github.io), sections 推論フレームワーク /
  Length Extrapolation (DCA, YaRN attention scaling), 疎アテンション
  (vertical-slash), Chunked Prefill (last-64 estimate, attention recall,
  sparsity refinement) and "アルゴリズム: DCAと疎アテンションの統合"
  (continuous positions for selection, DCA positions for attention).
* [long-context blog] "大規模モデル長文脈最適化実践：RoPE拡張から100万トークン推論へ"
  (toolsku.com), sections "RoPE原理の復習" (relative-position property) and
  "YaRN実装" (parameter names beta_fast / beta_slow / original_max_pos).
* [architecture overview] deepseekmodel.com long-context architecture page,
  §2.2 (PI / NTK / YaRN), §2.4 code (inv_freq, rotate_half convention),
  §3.2 (blocked attention with online softmax), §4.1 (attention sinks and
  the sliding window), §4.2 (vertical-slash and the other head patterns),
  §4.3 (selection of whole key blocks).

Pinned by the ``-m "not gpu"`` tests (brute force, closed forms, invariants,
hand-worked values).  Readings taken where the pages are silent or garbled
are stated next to the code they affect.  The YaRN frequency ramp between
beta_slow and beta_fast (the pages' snippet is garbled) is pinned by its end
points, its band sizes and three pairs worked by hand inside the ramp.
"""

from .rope import (bf16_round, bf16_round64, fp16_round64, rope_inv_freq, yarn_inv_freq,
                   yarn_mscale, softmax_scale, rope_rotate, rope_apply)
from .dca import (dca_position_maps, dca_chunk_of, query_positions,
                  relative_positions)
from .attention import (KeyContext, attention_logits, dense_causal_rows,
                        critical_set, sparse_rows, attention_recall)
from .estimate import estimate_scores, select_top, select_pattern
from .refine import refine_budgets, refine_sizes
from .patterns import a_shape_set, a_shape_lists, choose_candidates
from .blocksparse import (BLOCK, block_scores, select_blocks, block_key_set,
                          block_sparse_rows)

__all__ = [
    "bf16_round", "bf16_round64", "fp16_round64", "rope_inv_freq", "yarn_inv_freq", "yarn_mscale",
    "softmax_scale", "rope_rotate", "rope_apply",
    "dca_position_maps", "dca_chunk_of", "query_positions",
    "relative_positions",
    "KeyContext", "attention_logits", "dense_causal_rows", "critical_set",
    "sparse_rows", "attention_recall",
    "estimate_scores", "select_top", "select_pattern",
    "refine_budgets", "refine_sizes",
    "a_shape_set", "a_shape_lists", "choose_candidates",
    "BLOCK", "block_scores", "select_blocks", "block_key_set", "block_sparse_rows",
]
