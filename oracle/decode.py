"""Float64 definitions of the key/value cache a prefill leaves behind and of one decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests, the smoke
check and the bench's CPU-baseline leg, never by the product path.

Source: hf2q 0.1.1, ``qwen3vl_text/forward.rs`` -- the module doc's note on why there is no
KV cache yet and point 4 of ``forward_text_prefill_logits_last``'s notes: prefill walks the
whole sequence, a generation loop would at first prefill ``prompt + decoded`` again for every
new token, and keeping the keys and values for incremental decode is the later step. These
functions define that step as its plainest reading: the cache holds, per position and KV
head, the key after the per-head RMSNorm and the rotation (k') and the value (v) exactly as
the causal layer forms them; a decode step runs the layer on one new token whose query
attends to every cached key and to its own. By causality its output equals the last row
of the prefill over the longer sequence, which is what the pins check.
"""

import numpy as np

from .qwen3_layer import layer_prefill_rows, linear, qk_norm_mrope, rms_norm, silu

F64 = np.float64


def prefill_kv(x, w, cfg, pos):
    """(y [S, H], k' [S, nkv, hd], v [S, nkv, hd]) of one layer's causal prefill: the output
    rows and the cache entries of every prompt position."""
    s = np.asarray(x).shape[0]
    taps = {}
    y = layer_prefill_rows(x, w, cfg, pos, np.arange(s), taps=taps)
    return y, taps["k"], taps["v"]


def decode_attention(q, k_cache, v_cache):
    """Attention of one query row per head over every cached key.

    q: [nh, hd]; k_cache, v_cache: [L, nkv, hd] (the new token's own key and value
    included). Head h reads KV head h // (nh / nkv); weights are
    softmax(q_h . k_j / sqrt(hd)) over all L keys. Returns [nh, hd].
    """
    q, kc, vc = np.asarray(q, F64), np.asarray(k_cache, F64), np.asarray(v_cache, F64)
    nh, hd = q.shape
    group = nh // kc.shape[1]
    out = np.empty((nh, hd), dtype=F64)
    for h in range(nh):
        g = h // group
        z = kc[:, g, :] @ q[h] / np.sqrt(hd)
        p = np.exp(z - z.max())
        out[h] = (p / p.sum()) @ vc[:, g, :]
    return out


def layer_decode(x_new, w, cfg, pos_new, k_cache, v_cache):
    """One new token through the layer, the earlier positions read from the cache.

    x_new: [H]; pos_new: the token's (t, h, w) positions; k_cache, v_cache: [L, nkv, hd]
    of positions 0..L-1. Returns (y [H], k'_new [nkv, hd], v_new [nkv, hd]): the layer's
    output row and the entries the token appends to the cache at row L.
    """
    nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    x = np.asarray(x_new, F64)[None, :]
    pos = np.asarray(pos_new, dtype=np.int64).reshape(3, 1)
    xn = rms_norm(x, w["attn_norm"], cfg.eps)
    q = linear(xn, w["wq"]).reshape(1, nh, hd)
    k = linear(xn, w["wk"]).reshape(1, nkv, hd)
    v = linear(xn, w["wv"]).reshape(1, nkv, hd)
    q = qk_norm_mrope(q, w["q_norm"], cfg.eps, pos, cfg.theta, cfg.sections)
    k = qk_norm_mrope(k, w["k_norm"], cfg.eps, pos, cfg.theta, cfg.sections)
    kc = np.concatenate([np.asarray(k_cache, F64).reshape(-1, nkv, hd), k], axis=0)
    vc = np.concatenate([np.asarray(v_cache, F64).reshape(-1, nkv, hd), v], axis=0)
    o = decode_attention(q[0], kc, vc).reshape(1, nh * hd)
    y1 = x + linear(o, w["wo"])
    yn = rms_norm(y1, w["ffn_norm"], cfg.eps)
    y2 = y1 + linear(silu(linear(yn, w["w_gate"])) * linear(yn, w["w_up"]), w["w_down"])
    return y2[0], k[0], v[0]
