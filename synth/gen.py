"""Seeded normal draws for weights, hidden states, DeepStack slabs and positions.

Every tensor is drawn from its own numpy ``SFC64`` stream, keyed by the seed,
the tensor's name and a block index, in fixed blocks of ``_BLOCK`` values; so
a tensor's values do not depend on how many threads draw it. Values are
drawn in float64, scaled, rounded to float32, and (for bf16 workloads) rounded
to the nearest bf16 value with ties to even; they are returned as float32
arrays holding those exact values.
"""

import hashlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_BLOCK = 1 << 22

WEIGHT_NAMES = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                "ffn_norm", "w_gate", "w_up", "w_down")


def _key(name):
    return int.from_bytes(hashlib.blake2b(name.encode(), digest_size=8).digest(), "little")


def _normal_block(seed, key, blk, n):
    g = np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, key, blk])))
    return g.standard_normal(n)


def round_to_bf16(a):
    """Round float32 values to the nearest bf16 value (ties to even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def normal(seed, name, shape, mean=0.0, std=1.0, dtype="bf16", threads=8):
    """mean + std * N(0,1) draws for tensor `name`, rounded to the storage dtype."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    key = _key(name)

    def fill(b):
        lo = b * _BLOCK
        hi = min(n, lo + _BLOCK)
        v = _normal_block(seed, key, b, hi - lo) * std + mean
        out[lo:hi] = v.astype(np.float32)

    nblk = (n + _BLOCK - 1) // _BLOCK
    if nblk <= 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nblk)))
    if dtype == "bf16":
        out = round_to_bf16(out)
    return out.reshape(shape)


def make_layer_weights(cfg, layer=0, names=WEIGHT_NAMES):
    """The weight tensors `names` (default all eleven) of decoder layer `layer`, torch
    nn.Linear layout [out, in].

    Projection weights ~ N(0, 0.02), norm weights ~ 1 + N(0, 0.1); no biases.
    """
    h, hd, f = cfg.hidden, cfg.head_dim, cfg.ffn
    shapes = {
        "attn_norm": (h,), "wq": (cfg.q_dim, h), "wk": (cfg.kv_dim, h), "wv": (cfg.kv_dim, h),
        "q_norm": (hd,), "k_norm": (hd,), "wo": (h, cfg.q_dim), "ffn_norm": (h,),
        "w_gate": (f, h), "w_up": (f, h), "w_down": (h, f),
    }
    w = {}
    for name in names:
        is_norm = name.endswith("norm")
        w[name] = normal(cfg.seed, f"L{layer}.{name}", shapes[name],
                         mean=1.0 if is_norm else 0.0, std=0.1 if is_norm else 0.02,
                         dtype=cfg.dtype)
    return w


def make_x(cfg):
    """Input hidden states [S, H] ~ N(0, 1) (bf16-exact values for bf16 workloads)."""
    return normal(cfg.seed, "x", (cfg.seq_len, cfg.hidden), dtype=cfg.dtype)


def make_positions(cfg):
    """The [3, S] int32 (t, h, w) position table the workload prescribes.

    Text-only: t = h = w = token index. Image span: text tokens before the span
    count 0, 1, ...; the span's merged grid tokens come in 2x2 block-major order
    with t pinned at the span's first position and h, w = that position plus the
    grid row and column; text after the span resumes at the span's first
    position plus the grid's longer side and counts up.
    """
    s = cfg.seq_len
    pos = np.empty((3, s), dtype=np.int32)
    idx = np.arange(s, dtype=np.int32)
    pos[:] = idx
    if cfg.positions == "image_span":
        p0, gh, gw = cfg.span_start, cfg.span_h, cfg.span_w
        n = gh * gw
        k = np.arange(n)
        blk, sub = k // 4, k % 4
        blocks_per_row = gw // 2
        row = 2 * (blk // blocks_per_row) + sub // 2
        col = 2 * (blk % blocks_per_row) + sub % 2
        pos[0, p0:p0 + n] = p0
        pos[1, p0:p0 + n] = p0 + row
        pos[2, p0:p0 + n] = p0 + col
        after = np.arange(s - (p0 + n), dtype=np.int32) + p0 + max(gh, gw)
        pos[:, p0 + n:] = after
    return pos


def make_deepstack(cfg):
    """(rows, slab): DeepStack rows (the image span, ascending) and the [n, H] slab
    ~ N(0, deepstack_std) added on them; (None, None) when the workload has none."""
    if cfg.deepstack_std <= 0:
        return None, None
    rows = np.arange(cfg.span_start, cfg.span_start + cfg.span_len, dtype=np.int32)
    slab = normal(cfg.seed, "deepstack", (len(rows), cfg.hidden), std=cfg.deepstack_std,
                  dtype=cfg.dtype)
    return rows, slab


def make_model_weights(cfg, vocab, tied=False):
    """Whole-model tensors besides the layers: token_embd [vocab, H] ~ N(0, 0.02),
    output_norm [H] ~ 1 + N(0, 0.1) and lm_head [vocab, H] ~ N(0, 0.02) (None when the
    embeddings are tied)."""
    h = cfg.hidden
    emb = normal(cfg.seed, "token_embd", (vocab, h), std=0.02, dtype=cfg.dtype)
    norm = normal(cfg.seed, "output_norm", (h,), mean=1.0, std=0.1, dtype=cfg.dtype)
    head = None if tied else normal(cfg.seed, "lm_head", (vocab, h), std=0.02, dtype=cfg.dtype)
    return emb, norm, head


def make_tokens(cfg, vocab, name="tokens"):
    """[S] int32 token ids drawn uniformly from [0, vocab)."""
    g = np.random.Generator(np.random.SFC64(np.random.SeedSequence([cfg.seed, _key(name), 0])))
    return g.integers(0, vocab, size=cfg.seq_len, dtype=np.int64).astype(np.int32)


def make_deepstack_layers(cfg, n_layers):
    """One DeepStack slab per layer for the first `n_layers` layers, on the workload's
    DeepStack rows: (rows, [slab_0, ...]); (None, None) when the workload has none."""
    rows, _ = make_deepstack(cfg)
    if rows is None:
        return None, None
    slabs = [normal(cfg.seed, f"deepstack.L{li}", (len(rows), cfg.hidden), std=cfg.deepstack_std,
                    dtype=cfg.dtype) for li in range(n_layers)]
    return rows, slabs


PROJ_NAMES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
NORM_NAMES = ("attn_norm", "q_norm", "k_norm", "ffn_norm")


def _uniform_block(seed, key, n):
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, key, 1 << 20])))


def make_q4_0_weight(seed, name, rows, cols, std=0.02):
    """Q4_0 blocks of a [rows, cols] matrix as uint8 [rows, cols / 32, 18]: per block a
    binary16 scale drawn as std / 4.6 * U(0.75, 1.25) (4.6 is about the spread of a uniform
    4-bit code around 8), stored little-endian, then 16 bytes of uniform random codes."""
    g = _uniform_block(seed, _key(name), 0)
    nb = cols // 32
    blocks = g.integers(0, 256, size=(rows, nb, 18), dtype=np.uint8)
    d = (std / 4.6 * g.uniform(0.75, 1.25, size=(rows, nb))).astype("<f2")
    blocks[:, :, 0:2] = d[..., None].view(np.uint8)
    return blocks


def make_q8_row_weight(seed, name, rows, cols, std=0.02):
    """(codes int8 [rows, cols] uniform in [-127, 127], row scales float32 [rows] drawn as
    std / 73.6 * U(0.75, 1.25); 73.6 is about the spread of such a code)."""
    g = _uniform_block(seed, _key(name), 0)
    q = g.integers(-127, 128, size=(rows, cols), dtype=np.int16).astype(np.int8)
    rs = (std / 73.6 * g.uniform(0.75, 1.25, size=rows)).astype(np.float32)
    return q, rs


def make_quant_layer_weights(cfg, layer=0, formats=None):
    """(norms, projections) of decoder layer `layer` with quantized projections: norms as in
    make_layer_weights; projections[name] = (format, data, row_scale) with format "q4_0"
    (data = blocks), "q8_row" (data = codes, row_scale) or "dense" (data = the matrix of
    make_layer_weights). `formats` maps projection names to formats (default all "q4_0")."""
    formats = formats or {}
    h, f = cfg.hidden, cfg.ffn
    shapes = {"wq": (cfg.q_dim, h), "wk": (cfg.kv_dim, h), "wv": (cfg.kv_dim, h), "wo": (h, cfg.q_dim),
              "w_gate": (f, h), "w_up": (f, h), "w_down": (h, f)}
    norms = make_layer_weights(cfg, layer, NORM_NAMES)
    proj = {}
    for name in PROJ_NAMES:
        fmt = formats.get(name, "q4_0")
        rows, cols = shapes[name]
        tag = f"L{layer}.{name}.{fmt}"
        if fmt == "q4_0":
            proj[name] = (fmt, make_q4_0_weight(cfg.seed, tag, rows, cols), None)
        elif fmt == "q8_row":
            q, rs = make_q8_row_weight(cfg.seed, tag, rows, cols)
            proj[name] = (fmt, q, rs)
        elif fmt == "dense":
            proj[name] = (fmt, make_layer_weights(cfg, layer, (name,))[name], None)
        else:
            raise ValueError(f"unknown weight format {fmt}")
    return norms, proj
