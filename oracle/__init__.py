"""Float64 CPU oracle for the Gemma-4-style local/global attention block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
GPU product path (``global_gqa_rope_amd``) never imports it, and this package
imports nothing from the product path: the two share no code.

Everything here is plain numpy in float64, written from the definitions on the
source pages (all about the "Gemma 4 Technical Report"):

* QKNorm: per-head RMSNorm on q and k ("Gemma 4 Technical Report" notes,
  §2 Model Architecture; "Gemma 4 技术报告摘要", table "1. 预训练 Recipe", row 架构).
* RoPE on local layers and p-RoPE (p = 0.25) on global layers, base 10k / 1M
  ("Gemma 4 Technical Report" notes, §2 "Long-context efficiency";
  "Gemma 4多模态大模型架构详解", section "p-RoPE（低频剪枝旋转位置编码）").
* K = V in global layers: the keys are reused as the values
  ("Gemma 4多模态大模型架构详解", section "K=V").
* Grouped-query attention, 2 query heads per KV head on local layers and 8 on
  global layers, global head dim doubled to 512
  ("Gemma 4多模态大模型架构详解", section "分组查询注意力";
  "Gemma 4 架構與多模態拆解" talk notes, chapter "Grouped query attention").
* Sliding-window causal attention on local layers, full causal attention on
  global layers ("Gemma 4多模态大模型架构详解", section "交错层（局部与全局注意力）").

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, special cases that reduce to a library routine, and brute force on
tiny inputs.  No function here is "parity unpinned"; the only unpinned item is
agreement with real trained Gemma 4 layers, for which the pages give no worked
numbers.
"""

from .attention import (  # noqa: F401
    OracleLayer,
    cache_bytes_per_token,
    decode_from_cache,
    decode_from_prerotated_cache,
    decode_multi_from_cache,
    dequantize_rows,
    expected_caches_after_append,
    expected_caches_after_prefill,
    masked_softmax_attention,
    prefill,
    prerotated_heads,
    qk_norm,
    quantize_rows,
    ring_positions,
    rope_frequencies,
    rotate,
    rotated_pairs,
)
