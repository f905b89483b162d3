"""MI355X (gfx950) sparse-attention indexer path.

Seven calls, each a thin binding of the C ABI in include/pagescore.h:

  nvfp4_index_k_dequant  -- gather NVFP4 index-K pages into contiguous E4M3 pages
  indexer_score_decode   -- fused NVFP4 dequant + per-page decode scores
  indexer_score_prefill  -- lightning-indexer scores summed over heads
  indexer_score_prefill_ragged -- the same over a ragged batch, causally masked,
                            rows filled with -inf past their visible keys
  topk16_select          -- exact top-16 column ids per score row
  indexer_prefill_topk16 -- the top-16 of every prefill score row without the
                            score matrix (workspace from prefill_topk16_workspace)
  mxfp8_e4m3_quantize    -- MXFP8 (E4M3 + E8M0) quantization of bf16 rows, the
                            step after the sparse attention

The kernels are hand-written HIP in csrc/, built by page_scoring_top_amd/build.py.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    PageScoreError,
    PreparedCall,
    indexer_score_decode,
    indexer_score_prefill,
    indexer_prefill_topk16,
    indexer_score_prefill_ragged,
    mxfp8_e4m3_quantize,
    nvfp4_index_k_dequant,
    prefill_topk16_workspace,
    prefill_topk16_workspace_bytes,
    prepare,
    topk16_select,
)

__all__ = ["nvfp4_index_k_dequant", "indexer_score_decode", "indexer_score_prefill",
           "indexer_score_prefill_ragged", "indexer_prefill_topk16", "prefill_topk16_workspace",
           "prefill_topk16_workspace_bytes",
           "topk16_select", "mxfp8_e4m3_quantize", "prepare", "PreparedCall", "PageScoreError", "LIB_PATH"]
