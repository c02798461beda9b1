"""MI355X (gfx950) prefill of Qwen3/Qwen3-VL text decoder layers (and of the whole text model
to its last position's logits), the KV cache a prefill leaves and one decode step over it, with
dense or weight-only quantized (Q4_0, int8-row) projections.

The computation runs in libqwen3_prefill.so (hand-written HIP kernels behind a C ABI, see
include/qwen3_prefill.h). This package is the thin Python binding: it passes torch device
pointers and the current HIP stream to the library and does no arithmetic of its own.
"""

from .ops import (  # noqa: F401
    LayerSpec,
    Qwen3Error,
    apply_rope_tables,
    decode_attention_workspace_bytes,
    dequantize_matrix,
    gqa_bidirectional_attention,
    gqa_causal_attention,
    gqa_decode_attention,
    gqa_decode_attention_noalloc,
    kv_cache_alloc,
    kv_cache_write,
    layer_decode,
    layer_decode_quant,
    layer_decode_workspace_bytes,
    layer_prefill,
    layer_prefill_kv,
    layer_prefill_quant,
    layer_quant_workspace_bytes,
    layer_workspace_bytes,
    mfma_probe,
    model_decode_logits,
    model_decode_workspace_bytes,
    model_prefill_logits_last,
    model_workspace_bytes,
    qk_norm_mrope,
    rms_norm_rows,
    swiglu_ffn,
    tile_layer_weights,
    tile_weights,
    timing_collect,
    timing_enable,
    vision_rope_tables,
)
