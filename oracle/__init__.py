"""CPU float64 oracle of one Qwen3/Qwen3-VL text decoder layer's causal prefill.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition that the GPU path is checked against. Only the test suite, the
smoke check and the bench's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and this package imports
nothing from the product path.

Every function works in float64 on host numpy arrays. Matrix products use
numpy's matmul as a library primitive; nothing is blocked, fused or reordered
beyond the definitions the docstrings cite.

Sources (web pages, cited by title and item):
  * cortiq-engine 0.8.21, ``qwen3te.rs`` (Qwen3-VL as a prompt encoder):
    module doc, ``rms_norm_into``, ``silu``, ``norm_rope``, the per-pair
    causal attention loop and ``attention_gemm``, ``mrope_positions``,
    ``encode_with_images``.
  * hf2q 0.1.1, ``qwen3vl_text/forward.rs``: module doc (per-layer graph of
    the peer reference, final norm and LM head), the DeepStack residual
    injection (Phase D), ``forward_text_prefill_logits_last`` (model.py).
  * inferencelayer 0.2.3, ``vision.rs``: ``mrope_positions`` (M-RoPE
    positions), ``act_inplace`` (SiLU), ``rope_tables_2d`` and the vision block's
    ``attention`` (vision.py).
  * cortiq-engine 0.8.51, ``onevision2.rs``: three-axis vision rope tables, the
    adjacent-lane rotation and bidirectional ``attend`` (vision.py).
  * hf2q 0.1.1, ``qwen3vl_text/forward.rs``: the module doc's note on the deferred KV
    cache (decode.py: the cache a prefill leaves, one decode step); the Q4_0 FFN weights
    (quant.py).
  * cortiq-engine 0.8.21, ``qwen3te.rs``: ``q8_exact_matmat`` (quant.py: int8 rows with a
    row scale).

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests
against closed forms, invariants, textbook formulations and brute force; no
function is left unpinned.
"""

from .qwen3_layer import (  # noqa: F401
    causal_gqa_attention,
    layer_prefill,
    layer_prefill_rows,
    linear,
    mrope_axes,
    mrope_positions,
    qk_norm_mrope,
    rms_norm,
    rope_inv_freq,
    silu,
    stack_prefill,
    swiglu_ffn,
)
from .decode import decode_attention, layer_decode, prefill_kv  # noqa: F401,E402
from .quant import dequant, dequant_q4_0, dequant_q8_row  # noqa: F401,E402
from .model import embed_tokens, lm_head_last, model_prefill_logits_last  # noqa: F401,E402
from .vision import (  # noqa: F401,E402
    bidirectional_attention,
    merge_block_positions,
    rope_adjacent,
    rope_split_half,
    rope_tables_2d,
    rope_tables_3axis,
)
