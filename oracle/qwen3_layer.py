"""Float64 definition of the Qwen3/Qwen3-VL text decoder layer prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by the tests, the
smoke check and the bench's CPU-baseline leg, never by the product path.

Layer (hf2q 0.1.1 ``qwen3vl_text/forward.rs``, module doc, per-layer graph;
cortiq-engine 0.8.21 ``qwen3te.rs``, ``encode_with_images`` layer loop):

    xn = rmsnorm(x, attn_norm)
    q, k, v = xn Wq^T, xn Wk^T, xn Wv^T                 (no biases)
    q, k = per-head rmsnorm(q_norm / k_norm), then interleaved MRoPE
    o = causal GQA softmax(q k^T / sqrt(hd)) v
    y1 = x + o Wo^T
    yn = rmsnorm(y1, ffn_norm)
    y2 = y1 + (silu(yn Wg^T) * (yn Wu^T)) Wd^T
    y2[r] += D[k] for each DeepStack row r = rows[k]   (optional)

No final norm follows (the encoder's output is the unnormalized residual).
"""

import numpy as np

F64 = np.float64


def _f64(a):
    return np.asarray(a, dtype=F64)


def rms_norm(x, w, eps):
    """RMSNorm over the last axis with a plain weight.

    cortiq-engine ``qwen3te.rs``, ``rms_norm_into``: the mean of the squares of
    the row, eps added to that mean inside the square root, the row divided by
    it and then multiplied elementwise by w (plain w, not 1 + w, per that
    module's doc).
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(w)


def linear(x, w):
    """y = x W^T with W in torch nn.Linear layout [out, in], no bias
    (cortiq-engine ``qwen3te.rs``, the ``q``/``k``/``v``/``o``/``gate``/``up``/
    ``down`` projections; hf2q ``forward.rs`` notes the biases are absent)."""
    return _f64(x) @ _f64(w).T


def silu(z):
    """silu(z) = z / (1 + exp(-z)) (cortiq-engine ``qwen3te.rs``, ``silu``;
    inferencelayer ``vision.rs``, ``act_inplace``)."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def rope_inv_freq(head_dim, theta):
    """Frequency of rotation pair i, i < head_dim/2: theta^(-2i/head_dim)
    (cortiq-engine ``qwen3te.rs``, ``norm_rope``)."""
    i = np.arange(head_dim // 2, dtype=F64)
    return 1.0 / np.power(F64(theta), 2.0 * i / head_dim)


def mrope_axes(head_dim, sections):
    """Position axis (0 = t, 1 = h, 2 = w) that drives each rotation pair.

    Qwen3-VL's interleaved MRoPE (cortiq-engine ``qwen3te.rs``, ``norm_rope``):
    the time axis by default; height takes every third pair starting at 1 and
    width every third pair starting at 2, each only below three times its
    section size. For sections (24, 20, 20) and head_dim 128 this is the page's
    literal rule (pairs below 60 with i % 3 == 1 -> h, == 2 -> w); in general it
    gives each axis exactly its section's number of pairs.
    """
    _s_t, s_h, s_w = sections
    axes = np.zeros(head_dim // 2, dtype=np.int64)
    for i in range(head_dim // 2):
        if i % 3 == 1 and i < 3 * s_h:
            axes[i] = 1
        elif i % 3 == 2 and i < 3 * s_w:
            axes[i] = 2
    return axes


def qk_norm_mrope(x, w, eps, pos, theta, sections):
    """Per-head RMSNorm then split-half interleaved-MRoPE rotation.

    cortiq-engine ``qwen3te.rs``, ``norm_rope``. x: [S, heads, hd]; w: [hd];
    pos: [3, S] (t, h, w) positions. Each (token, head) row is RMS-normalized
    over hd and multiplied by w (before the rotation, per the module doc); then
    for every pair i < hd/2 with angle phi = pos[axis(i), s] * theta^(-2i/hd),
    (a, b) = (x_i, x_{i+hd/2}) becomes (a cos phi - b sin phi, a sin phi + b cos phi).
    """
    x = _f64(x)
    _s, _heads, hd = x.shape
    half = hd // 2
    xn = rms_norm(x, w, eps)
    inv = rope_inv_freq(hd, theta)
    axes = mrope_axes(hd, sections)
    pos = _f64(pos)
    phi = pos[axes, :].T * inv[None, :]          # [S, half]: pos[axis(i), s] * inv_i
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    a = xn[..., :half]
    b = xn[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def causal_gqa_attention(q, k, v, q_rows=None):
    """Causal grouped-query softmax attention with scale 1/sqrt(head_dim).

    cortiq-engine ``qwen3te.rs``, the per-pair causal loop and
    ``attention_gemm``: query head h reads KV head h // (nh / nkv); for query
    token s the scores q_h[s] . k[j] / sqrt(hd) over keys j <= s are
    softmax-normalized (maximum subtracted) and weight the rows v[j].

    q: [R, nh, hd] for query tokens ``q_rows`` (default 0..R-1); k, v:
    [S', nkv, hd] with S' > max(q_rows). Returns [R, nh, hd].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    r, nh, hd = q.shape
    nkv = k.shape[1]
    group = nh // nkv
    rows = np.arange(r) if q_rows is None else np.asarray(q_rows)
    n_keys = int(rows.max()) + 1
    live = np.arange(n_keys)[None, :] <= rows[:, None]      # [R, keys]
    scale = 1.0 / np.sqrt(hd)
    out = np.empty((r, nh, hd), dtype=F64)
    for h in range(nh):
        g = h // group
        z = (q[:, h, :] @ k[:n_keys, g, :].T) * scale
        z = np.where(live, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:n_keys, g, :]
    return out


def swiglu_ffn(yn, w_gate, w_up, w_down):
    """(silu(yn Wg^T) * (yn Wu^T)) Wd^T (cortiq-engine ``qwen3te.rs``, the
    gate/up/act/down steps of the layer loop; hf2q ``forward.rs``, SILU FFN
    with parallel gate and up)."""
    a = silu(linear(yn, w_gate)) * linear(yn, w_up)
    return linear(a, w_down)


def layer_prefill_rows(x, w, cfg, pos, rows, ds_rows=None, ds=None, taps=None):
    """Output rows ``rows`` of one decoder layer (the definition restricted to rows).

    Causality makes output row s depend on input rows 0..s only, so only keys
    and values up to max(rows) are formed. ``w`` maps the names attn_norm, wq,
    wk, wv, q_norm, k_norm, wo, ffn_norm, w_gate, w_up, w_down to arrays;
    ``cfg`` supplies n_heads, n_kv_heads, head_dim, eps, theta and sections.
    DeepStack (hf2q ``forward.rs``, Phase D; cortiq ``encode_with_images``):
    after the FFN residual, ``ds[k]`` is added to output row ``ds_rows[k]``.
    ``taps``, if a dict, receives the intermediates.
    """
    x = _f64(x)
    rows = np.asarray(rows, dtype=np.int64)
    nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    n_keys = int(rows.max()) + 1
    xk = x[:n_keys]
    pos = np.asarray(pos)[:, :n_keys]

    xn = rms_norm(xk, w["attn_norm"], cfg.eps)
    k = linear(xn, w["wk"]).reshape(n_keys, nkv, hd)
    v = linear(xn, w["wv"]).reshape(n_keys, nkv, hd)
    k = qk_norm_mrope(k, w["k_norm"], cfg.eps, pos, cfg.theta, cfg.sections)
    q = linear(xn[rows], w["wq"]).reshape(len(rows), nh, hd)
    q = qk_norm_mrope(q, w["q_norm"], cfg.eps, pos[:, rows], cfg.theta, cfg.sections)
    o = causal_gqa_attention(q, k, v, rows).reshape(len(rows), nh * hd)
    y1 = x[rows] + linear(o, w["wo"])
    yn = rms_norm(y1, w["ffn_norm"], cfg.eps)
    a = silu(linear(yn, w["w_gate"])) * linear(yn, w["w_up"])
    y2 = y1 + linear(a, w["w_down"])
    if ds_rows is not None and ds is not None and len(ds_rows) > 0:
        ds = _f64(ds)
        where = {int(r): i for i, r in enumerate(np.asarray(ds_rows))}
        for j, r in enumerate(rows):
            i = where.get(int(r))
            if i is not None:
                y2[j] += ds[i]
    if taps is not None:
        taps.update(xn=xn[rows], q=q, k=k, v=v, o=o, y1=y1, yn=yn, a=a, y2=y2)
    return y2


def layer_prefill(x, w, cfg, pos, ds_rows=None, ds=None, taps=None):
    """All S output rows of one decoder layer: [S, H] float64."""
    s = np.asarray(x).shape[0]
    return layer_prefill_rows(x, w, cfg, pos, np.arange(s), ds_rows, ds, taps)


def stack_prefill(x, layers, cfg, pos, ds_rows=None, ds_per_layer=None):
    """Decoder layers applied in sequence, each feeding the next (cortiq
    ``encode_with_images``); ``ds_per_layer[l]`` is layer l's DeepStack slab."""
    h = _f64(x)
    for li, w in enumerate(layers):
        ds = None if ds_per_layer is None or li >= len(ds_per_layer) else ds_per_layer[li]
        h = layer_prefill(h, w, cfg, pos, ds_rows, ds)
    return h


def mrope_positions(n, spans):
    """Three-axis positions [3, n] of a prompt with image spans.

    inferencelayer 0.2.3 ``vision.rs``, ``mrope_positions``, and cortiq-engine
    ``qwen3te.rs``, ``mrope_positions``: text tokens advance all three axes
    together; an image span of a merged gh x gw grid keeps one t (the counter at
    the span's start) while h and w walk the grid row-major from that value; the
    counter then advances by max(gh, gw), not by the span's token count.
    ``spans``: (start, gh, gw) tuples in increasing start order.
    """
    pos = np.zeros((3, n), dtype=np.int64)
    cur = 0
    i = 0
    span_at = {s: (gh, gw) for s, gh, gw in spans}
    while i < n:
        if i in span_at:
            gh, gw = span_at[i]
            for r in range(gh):
                for c in range(gw):
                    pos[:, i] = (cur, cur + r, cur + c)
                    i += 1
            cur += max(gh, gw)
        else:
            pos[:, i] = cur
            cur += 1
            i += 1
    return pos
