"""CPU oracle for paged sliding-window KV attention (test infrastructure).

This package is the slow, plain reference the device path is checked against.
It is test infrastructure, not part of the product: only the tests, the
package smoke check and the bench's CPU-baseline leg may import or run it.
It shares no code with the HIP path and imports nothing from it.

Contents
  page_cache  the page pool, free list, the three page streams (scale,
              sliding window, special), the visible page table and the
              single-level rollback, exactly as written in the readings of
              the pages listed in the module docstring.
  windowed    windowed inference: restart every window of kept units, the
              last units of a window shared with the next.
  fp8         FP8 (E4M3) KV pages: per-(token, head) power-of-two row
              scales, round-to-nearest-even quantisation and dequantisation.
  subset      page-subset visible tables (per-layer random page sampling)
              with the splitmix64 generator written out.
  attention   softmax attention in float64 over gathered pages, a dense
              reference over tokens selected straight from the frame history,
              a brute-force scalar version for tiny shapes, and the merge of
              partial (output, log-sum-exp) pairs.

Every function names the passage of the pages it follows.  Page titles used
in citations:
  "LingBot-Map Paged KV Cache" (a Chinese-language article, sections 1-7)
  "vLLM-Omni RFC #2727: Reconstruction Engine" (sections 1-3.6)
"""
from .page_cache import (  # noqa: F401
    OracleCache, OracleConfig, OutOfPages, NoUndo, FRAME_ALIGNED, CONTIGUOUS,
    is_keyframe, required_pages,
)
from .attention import (  # noqa: F401
    attention_f64, brute_attention, merge_partials, bf16_bits_to_f64, to_f64,
    dense_history_attention,
)
from .subset import splitmix64, subset_table, subset_keep_count  # noqa: F401,E402
from .windowed import OracleWindowed  # noqa: F401,E402
from .fp8 import E4M3_MAX, dequantize_rows, e4m3_decode, e4m3_encode, quantize_rows, row_exponent  # noqa: F401,E402
