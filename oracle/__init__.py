"""CPU oracle for fused RoPE causal prefill attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously correct
definition that the GPU library is checked against.  Only the test suite, the
smoke check in ``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the C-ABI library and its Python
binding) never imports, calls or links anything here, and this package never
imports the product path: the two share no code, tables or constants.

Pages cited (by title and section):

* "手写内核实现6倍prefill加速：边缘LLM推理的内存与计算协同优化"
  (www.0539edu.com/news/6082052), §2.2, §3.1 -- RoPE as a complex multiply
  fused into the Q·Kᵀ dot, cos/sin tables indexed by position.
* the 2kiu.com/news/6082051 retelling of the same engine (HTML title
  "企业官网建设流程全解析"), §2.1, §3.3, §4.2 -- blocked attention with no
  S×S matrix, int16 fixed-point RoPE tables, the RoPE table script.
* the MNN-on-K3 blog (zhaode.wang/blog/2026/mnn-k3-riscv), §六 -- fused
  attention as blocked online softmax (QK, online softmax, PV in one pass).
* the XNet-DNN article (www.szyisi.cn/article/817147.html), §三.3
  FlashAttention-2 -- online softmax, deferred rescale.
* "手写内核实现6倍prefill加速" §2.2 and §3.2 again for the KV cache: new
  tokens' K/V copied into free slots, an index map from logical position to
  physical slot (``kv_cache.py``).
* the 2kiu.com retelling, §3.3, and the MNN-on-K3 blog, §四, for the
  per-token dynamic int16 quantisation of float Q/K (``quantize.py``).
* the 2kiu.com retelling, §3.3, for the fixed-point softmax: exp as 16
  straight-line segments on [-8, 8] and a division-free reciprocal
  (``pwl_softmax.py``).

The blocked online softmax of those pages reaches, in exact arithmetic, the
plain causal softmax-attention result; so this oracle is that plain
definition: explicit RoPE, the full causal score matrix, a two-pass softmax.

Parity pins (tests/test_oracle_pins.py, tests/test_oracle_cache_pins.py,
tests/test_oracle_quant_pins.py, tests/test_oracle_pwl_pins.py) cover every
function here; none is
"parity unpinned".  Two *inputs* are readings rather than derivations and are
documented as such with the workloads: the int16 ``score_scale`` and the
per-head scale recipe of the long-prompt workload.
"""

from .attention import (
    rope_inv_freq,
    rope_cos_sin,
    rope_rotate,
    causal_probs,
    attention,
    attention_rows,
)
from .kv_cache import (
    ring_index_map,
    paged_index_map,
    kv_cache_update,
    gather_logical,
    attention_cached,
    attention_cached_rows,
    attention_i16_cached,
)
from .quantize import (
    quantize_rows_i16,
    attention_i16_quantized,
    attention_i16_quantized_rows,
)
from .pwl_softmax import (
    pwl_exp,
    newton_reciprocal,
    pwl_softmax_rows,
    attention_i16_pwl,
)
from .fixed_point import (
    rope_table_q14,
    rope_rotate_i16,
    scores_i32,
    attention_i16,
    attention_i16_rows,
)

__all__ = [
    "rope_inv_freq",
    "rope_cos_sin",
    "rope_rotate",
    "causal_probs",
    "attention",
    "attention_rows",
    "rope_table_q14",
    "rope_rotate_i16",
    "scores_i32",
    "attention_i16",
    "attention_i16_rows",
    "ring_index_map",
    "paged_index_map",
    "kv_cache_update",
    "gather_logical",
    "attention_cached",
    "attention_cached_rows",
    "attention_i16_cached",
    "quantize_rows_i16",
    "attention_i16_quantized",
    "attention_i16_quantized_rows",
    "pwl_exp",
    "newton_reciprocal",
    "pwl_softmax_rows",
    "attention_i16_pwl",
]
