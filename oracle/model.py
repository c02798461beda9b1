"""Float64 definition of the whole-model text prefill returning the last position's logits.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests, the smoke
check and the bench's CPU-baseline leg, never by the product path.

Source: hf2q 0.1.1, ``qwen3vl_text/forward.rs`` -- the module doc (per-layer graph, then
"Final": output RMSNorm and the LM head, which is the token embedding table when the
embeddings are tied) and ``forward_text_prefill_logits_last`` (token embedding lookup;
the decoder layers in order, with DeepStack slab ``il`` added after layer ``il`` for
``il < n_deepstack_layers``; final RMSNorm and LM head on the last position only;
errors for an empty prompt and out-of-range token ids).
"""

import numpy as np

from .qwen3_layer import layer_prefill_rows, linear, rms_norm, stack_prefill


def embed_tokens(tokens, table):
    """Row ``tokens[s]`` of the [vocab, H] embedding table for every position s
    (``forward_text_prefill_logits_last``, step 1: embedding lookup)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    table = np.asarray(table, dtype=np.float64)
    if tokens.ndim != 1 or tokens.size == 0:
        raise ValueError("empty token list")
    if tokens.min() < 0 or tokens.max() >= table.shape[0]:
        raise ValueError("token id out of range")
    return table[tokens]


def lm_head_last(h_last, output_norm, lm_head, eps):
    """Logits of one position: RMSNorm with ``output_norm``, then the LM head
    [vocab, H] in nn.Linear layout (module doc, "Final")."""
    return linear(rms_norm(np.asarray(h_last, dtype=np.float64)[None, :], output_norm, eps), lm_head)[0]


def model_prefill_logits_last(tokens, token_embd, layers, output_norm, lm_head, cfg, pos,
                              ds_rows=None, ds_per_layer=None):
    """Logits [vocab] of the last prompt position. ``lm_head`` None means tied embeddings
    (the LM head is ``token_embd``); ``ds_per_layer[il]`` is added after layer il (only the
    first ``len(ds_per_layer)`` layers receive one). The last layer is evaluated on the
    last row only (the definition restricted to the row the logits need)."""
    x = embed_tokens(tokens, token_embd)
    s = x.shape[0]
    head = token_embd if lm_head is None else lm_head
    if not layers:
        return lm_head_last(x[-1], output_norm, head, cfg.eps)
    n_ds = 0 if ds_per_layer is None else len(ds_per_layer)
    h = stack_prefill(x, layers[:-1], cfg, pos, ds_rows, ds_per_layer)
    li = len(layers) - 1
    ds_last = ds_per_layer[li] if li < n_ds else None
    last = layer_prefill_rows(h, layers[-1], cfg, pos, np.array([s - 1]), ds_rows, ds_last)
    return lm_head_last(last[0], output_norm, head, cfg.eps)
