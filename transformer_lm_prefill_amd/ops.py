"""Python entry points with the C ABI's names: argument marshalling only.

Tensors are torch tensors on the GPU (bf16 or float32, contiguous); work is enqueued on
torch's current stream. Every check of shapes and sizes happens in the library, which
raises Qwen3Error (status and message) on any violation.
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import Qwen3Error  # noqa: F401

WEIGHT_NAMES = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm",
                "w_gate", "w_up", "w_down")


@dataclass(frozen=True)
class LayerSpec:
    """Shape and numerics of one decoder layer (fields of qwen3_layer_cfg)."""
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    eps: float = 1e-6
    theta: float = 5e6
    sections: tuple = (24, 20, 20)
    dtype: str = "bf16"      # weights: "bf16", "f16", "f32", or "f16t": fp16 with the seven
                             # projection matrices in the tiled layout (tile_weights)
    act: str = ""            # matrix-product operands: "f16", "bf16" or "f32"; "" = f16 for
                             # 16-bit weights, f32 for f32 weights

    @classmethod
    def of(cls, c, act=""):
        """From any object with these attribute names."""
        return cls(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, c.eps, c.theta,
                   tuple(c.sections), c.dtype, act)

    @property
    def act_dtype(self):
        if self.act:
            return self.act
        return "f32" if self.dtype == "f32" else "f16"


_CODES = {"f32": _lib.QWEN3_F32, "bf16": _lib.QWEN3_BF16, "f16": _lib.QWEN3_F16,
          "f16t": _lib.QWEN3_F16_TILED}
TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "f16t": torch.float16}
# the seven projection matrices (tiled under "f16t"; the vectors stay plain)
MATRIX_NAMES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def _dt(t):
    if t.dtype == torch.bfloat16:
        return _lib.QWEN3_BF16
    if t.dtype == torch.float16:
        return _lib.QWEN3_F16
    if t.dtype == torch.float32:
        return _lib.QWEN3_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _cfg(spec):
    c = _lib.LayerCfg()
    c.hidden, c.n_heads, c.n_kv_heads = spec.hidden, spec.n_heads, spec.n_kv_heads
    c.head_dim, c.ffn = spec.head_dim, spec.ffn
    c.rms_eps, c.rope_theta = spec.eps, spec.theta
    c.mrope_section = (ctypes.c_int32 * 3)(*spec.sections)
    c.wdtype = _CODES[spec.dtype]
    c.act_dtype = _CODES[spec.act_dtype]
    c.resid_dtype = _lib.QWEN3_F32
    return c


def _host_rows(ds_rows):
    """DeepStack rows as a host int32 array for the C ABI: (ctypes array or None, count).
    Accepts a sequence of ints, a numpy array or a CPU tensor; a GPU tensor is refused (the
    library checks the list on the host before it enqueues anything)."""
    if ds_rows is None:
        return None, 0
    if isinstance(ds_rows, torch.Tensor):
        if ds_rows.device.type != "cpu":
            raise TypeError("ds_rows must be host data (a sequence, numpy array or CPU tensor)")
        ds_rows = ds_rows.tolist()
    vals = [int(r) for r in (ds_rows.tolist() if hasattr(ds_rows, "tolist") else ds_rows)]
    if not vals:
        return None, 0
    return (ctypes.c_int32 * len(vals))(*vals), len(vals)


def layer_workspace_bytes(spec, seq_len):
    return int(_lib.load().qwen3_layer_workspace_bytes(ctypes.byref(_cfg(spec)), int(seq_len)))


def layer_prefill(spec, weights, x, positions, ds_rows=None, ds=None, out=None, workspace=None):
    """qwen3_layer_prefill: one decoder layer over x [S, H] float32; returns out [S, H] float32.

    weights: mapping of the eleven weight names to tensors of spec's dtype; positions [3, S]
    int32; ds_rows: n host row indices (strictly increasing, < S) and ds [n, H] (spec's dtype)
    on the GPU for DeepStack, or None.
    out may be x (in place). workspace: a uint8 tensor of layer_workspace_bytes() or None.
    """
    lib = _lib.load()
    cfg = _cfg(spec)
    s = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    need = int(lib.qwen3_layer_workspace_bytes(ctypes.byref(cfg), int(s)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    w = _lib.LayerWeights(*[_ptr(weights[n]) for n in WEIGHT_NAMES])
    rows, n_ds = _host_rows(ds_rows)
    _lib.check(lib.qwen3_layer_prefill(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(s), _ptr(positions),
        rows, n_ds, _ptr(ds), _ptr(workspace), int(workspace.numel()), _stream()))
    return out


def kv_cache_alloc(spec, capacity, device="cuda"):
    """(k_cache, v_cache): zeroed [n_kv_heads, capacity, head_dim] tensors of spec's act dtype."""
    shape = (spec.n_kv_heads, int(capacity), spec.head_dim)
    dt = TORCH_DTYPES[spec.act_dtype]
    return torch.zeros(shape, dtype=dt, device=device), torch.zeros(shape, dtype=dt, device=device)


def kv_cache_write(k, v, k_cache, v_cache, row0=0):
    """kv_cache_write: rows of k, v [n, n_kv_heads, head_dim] (rows may be strided views of a
    wider row, heads contiguous) into cache rows row0.. of k_cache / v_cache [nkv, cap, hd]."""
    lib = _lib.load()
    n, nkv, hd = k.shape
    for t in (k, v):
        if t.stride(2) != 1 or t.stride(1) != hd:
            raise ValueError("heads of a row must be contiguous")
    if v.dtype != k.dtype:
        raise TypeError("k and v must have one dtype")
    _lib.check(lib.kv_cache_write(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), int(k.stride(0)),
                                  int(v.stride(0)), int(n), int(nkv), int(hd), _dt(k), _ptr(k_cache),
                                  _ptr(v_cache), _dt(k_cache), int(k_cache.shape[1]), int(row0), _stream()))


def layer_prefill_kv(spec, weights, x, positions, k_cache, v_cache, ds_rows=None, ds=None, out=None,
                     workspace=None):
    """qwen3_layer_prefill_kv: layer_prefill that also writes k', v of every position into rows
    0..S-1 of the caches ([n_kv_heads, capacity, head_dim], spec's act dtype)."""
    lib = _lib.load()
    cfg = _cfg(spec)
    s = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    need = int(lib.qwen3_layer_workspace_bytes(ctypes.byref(cfg), int(s)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    w = _lib.LayerWeights(*[_ptr(weights[n]) for n in WEIGHT_NAMES])
    rows, n_ds = _host_rows(ds_rows)
    _lib.check(lib.qwen3_layer_prefill_kv(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(s), _ptr(positions),
        rows, n_ds, _ptr(ds), _ptr(k_cache), _ptr(v_cache), int(k_cache.shape[1]),
        _ptr(workspace), int(workspace.numel()), _stream()))
    return out


def decode_attention_workspace_bytes(n_heads, n_kv_heads, head_dim, length):
    return int(_lib.load().gqa_decode_attention_workspace_bytes(int(n_heads), int(n_kv_heads), int(head_dim),
                                                                int(length)))


def gqa_decode_attention(q, k_cache, v_cache, length, scale=None, out=None, workspace=None):
    """gqa_decode_attention: q [n_heads, head_dim] float32 over cache rows 0..length-1;
    returns out [n_heads, head_dim] float32."""
    lib = _lib.load()
    nh, hd = q.shape
    nkv, cap = k_cache.shape[0], k_cache.shape[1]
    if scale is None:
        scale = hd ** -0.5
    if out is None:
        out = torch.empty_like(q)
    need = decode_attention_workspace_bytes(nh, nkv, hd, length)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.gqa_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(cap), int(length), int(nh),
                                        int(nkv), int(hd), float(scale), _dt(k_cache), _ptr(out), _ptr(workspace),
                                        int(workspace.numel()), _stream()))
    return out


def gqa_decode_attention_noalloc(q, k_cache, v_cache, length, scale=None, out=None):
    """gqa_decode_attention_noalloc: gqa_decode_attention with the library's fixed per-GPU
    scratch array in place of a workspace (nothing is allocated except `out` when None)."""
    lib = _lib.load()
    nh, hd = q.shape
    nkv, cap = k_cache.shape[0], k_cache.shape[1]
    if scale is None:
        scale = hd ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _lib.check(lib.gqa_decode_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(cap), int(length),
                                                int(nh), int(nkv), int(hd), float(scale), _dt(k_cache), _ptr(out),
                                                _stream()))
    return out


def layer_decode_workspace_bytes(spec, capacity):
    return int(_lib.load().qwen3_layer_decode_workspace_bytes(ctypes.byref(_cfg(spec)), int(capacity)))


def layer_decode(spec, weights, x, position, k_cache, v_cache, length, out=None, workspace=None):
    """qwen3_layer_decode: one new token x [H] float32 at `position` (int32 [3] on the GPU) over
    cache rows 0..length-1; appends its k', v at row `length`; returns out [H] float32."""
    lib = _lib.load()
    cfg = _cfg(spec)
    cap = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(x)
    need = int(lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(cfg), int(cap)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    w = _lib.LayerWeights(*[_ptr(weights[n]) for n in WEIGHT_NAMES])
    _lib.check(lib.qwen3_layer_decode(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(position),
                                      _ptr(k_cache), _ptr(v_cache), int(cap), int(length), _ptr(workspace),
                                      int(workspace.numel()), _stream()))
    return out


_WFORMATS = {"dense": _lib.W_DENSE, "q4_0": _lib.W_Q4_0, "q8_row": _lib.W_Q8_ROW}
PROJ_NAMES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
NORM_NAMES = ("attn_norm", "q_norm", "k_norm", "ffn_norm")


def _qmatrix(entry):
    """(format name, data tensor, row_scale tensor or None) -> QMatrix."""
    fmt, data, rs = entry
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("quantized weights must be contiguous GPU tensors")
    return _lib.QMatrix(_WFORMATS[fmt], ctypes.c_void_p(data.data_ptr()), _ptr(rs))


def _qweights(norms, proj):
    args = {n: _ptr(norms[n]) for n in NORM_NAMES}
    args.update({n: _qmatrix(proj[n]) for n in PROJ_NAMES})
    return _lib.LayerQWeights(**args)


def dequantize_matrix(fmt, data, rows, cols, row_scale=None, out_dtype=torch.float16, out=None):
    """dequantize_matrix: [rows, cols] of out_dtype from Q4_0 blocks (uint8) or int8 rows + scales."""
    lib = _lib.load()
    if out is None:
        out = torch.empty(rows, cols, dtype=out_dtype, device=data.device)
    m = _qmatrix((fmt, data, row_scale))
    _lib.check(lib.dequantize_matrix(ctypes.byref(m), int(rows), int(cols), _dt(out), _ptr(out), _stream()))
    return out


def layer_quant_workspace_bytes(spec, seq_len):
    return int(_lib.load().qwen3_layer_quant_workspace_bytes(ctypes.byref(_cfg(spec)), int(seq_len)))


def layer_prefill_quant(spec, norms, proj, x, positions, ds_rows=None, ds=None, k_cache=None, v_cache=None,
                        out=None, workspace=None):
    """qwen3_layer_prefill_quant: norms maps the four norm names to tensors of spec's dtype; proj
    maps the seven projection names to (format, data, row_scale) with format "dense", "q4_0"
    or "q8_row". Optional caches as for layer_prefill_kv."""
    lib = _lib.load()
    cfg = _cfg(spec)
    s = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    need = int(lib.qwen3_layer_quant_workspace_bytes(ctypes.byref(cfg), int(s)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    w = _qweights(norms, proj)
    rows, n_ds = _host_rows(ds_rows)
    cap = 0 if k_cache is None else int(k_cache.shape[1])
    _lib.check(lib.qwen3_layer_prefill_quant(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(s), _ptr(positions), rows, n_ds,
        _ptr(ds), _ptr(k_cache), _ptr(v_cache), cap, _ptr(workspace), int(workspace.numel()), _stream()))
    return out


def layer_decode_quant(spec, norms, proj, x, position, k_cache, v_cache, length, out=None, workspace=None):
    """qwen3_layer_decode_quant: layer_decode with the weights of layer_prefill_quant."""
    lib = _lib.load()
    cfg = _cfg(spec)
    cap = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(x)
    need = int(lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(cfg), int(cap)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    w = _qweights(norms, proj)
    _lib.check(lib.qwen3_layer_decode_quant(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(position),
                                            _ptr(k_cache), _ptr(v_cache), int(cap), int(length), _ptr(workspace),
                                            int(workspace.numel()), _stream()))
    return out


def _model_cfg(spec, n_layers, vocab, n_deepstack_layers):
    m = _lib.ModelCfg()
    m.layer = _cfg(spec)
    m.n_layers, m.vocab, m.n_deepstack_layers = int(n_layers), int(vocab), int(n_deepstack_layers)
    return m


def model_workspace_bytes(spec, n_layers, vocab, seq_len, n_deepstack_layers=0):
    m = _model_cfg(spec, n_layers, vocab, n_deepstack_layers)
    return int(_lib.load().qwen3_model_workspace_bytes(ctypes.byref(m), int(seq_len)))


def _model_weights(layers, token_embd, output_norm, lm_head):
    lw = (_lib.LayerWeights * max(len(layers), 1))()
    for i, w in enumerate(layers):
        lw[i] = _lib.LayerWeights(*[_ptr(w[n]) for n in WEIGHT_NAMES])
    return _lib.ModelWeights(_ptr(token_embd), lw if layers else None, _ptr(output_norm), _ptr(lm_head)), lw


def _cache_arrays(caches):
    """[(k, v) per layer] -> two host arrays of device pointers (or None, None)."""
    if caches is None:
        return None, None
    for k, v in caches:
        _ptr(k), _ptr(v)
    kc = (ctypes.c_void_p * max(len(caches), 1))(*[k.data_ptr() for k, _ in caches])
    vc = (ctypes.c_void_p * max(len(caches), 1))(*[v.data_ptr() for _, v in caches])
    return kc, vc


def model_decode_workspace_bytes(spec, n_layers, vocab, capacity):
    m = _model_cfg(spec, n_layers, vocab, 0)
    return int(_lib.load().qwen3_model_decode_workspace_bytes(ctypes.byref(m), int(capacity)))


def model_decode_logits(spec, layers, token_embd, output_norm, lm_head, token, position, caches, length,
                        out=None, workspace=None):
    """qwen3_model_decode_logits: logits [vocab] float32 of one new token (host int id) at
    `position` (int32 [3] on the GPU) after `length` cached tokens; caches: [(k, v)] per layer
    as from kv_cache_alloc, filled by model_prefill_logits_last(..., caches=...)."""
    lib = _lib.load()
    vocab = int(token_embd.shape[0])
    m = _model_cfg(spec, len(layers), vocab, 0)
    cap = int(caches[0][0].shape[1]) if caches else 1
    if out is None:
        out = torch.empty(vocab, dtype=torch.float32, device=token_embd.device)
    need = int(lib.qwen3_model_decode_workspace_bytes(ctypes.byref(m), cap))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=token_embd.device)
    mw, _keep = _model_weights(layers, token_embd, output_norm, lm_head)
    kc, vc = _cache_arrays(caches)
    _lib.check(lib.qwen3_model_decode_logits(ctypes.byref(m), ctypes.byref(mw), int(token), _ptr(position), kc, vc,
                                             cap, int(length), _ptr(out), _ptr(workspace), int(workspace.numel()),
                                             _stream()))
    return out


def model_prefill_logits_last(spec, layers, token_embd, output_norm, lm_head, tokens, positions,
                              ds_rows=None, ds=None, out=None, workspace=None, caches=None):
    """qwen3_model_prefill_logits_last: logits [vocab] float32 of the last prompt position.

    layers: list of weight mappings (one per decoder layer); token_embd [vocab, H],
    output_norm [H], lm_head [vocab, H] or None (tied) on the GPU in spec's dtype; tokens: a
    host sequence of int token ids; positions [3, S] int32 on the GPU; ds_rows n host row indices
    (strictly increasing, < S) and ds a list of [n, H] slabs (one per DeepStack layer, the first len(ds) layers) or None.
    caches: None, or [(k, v)] per layer (kv_cache_alloc) to be filled with every layer's k', v
    (qwen3_model_prefill_logits_last_kv).
    """
    lib = _lib.load()
    vocab = int(token_embd.shape[0])
    n_dsl = 0 if ds is None else len(ds)
    m = _model_cfg(spec, len(layers), vocab, n_dsl)
    tok = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
    s = len(tokens)
    if out is None:
        out = torch.empty(vocab, dtype=torch.float32, device=token_embd.device)
    need = int(lib.qwen3_model_workspace_bytes(ctypes.byref(m), int(s)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=token_embd.device)
    lw = (_lib.LayerWeights * max(len(layers), 1))()
    for i, w in enumerate(layers):
        lw[i] = _lib.LayerWeights(*[_ptr(w[n]) for n in WEIGHT_NAMES])
    mw = _lib.ModelWeights(_ptr(token_embd), lw if layers else None, _ptr(output_norm), _ptr(lm_head))
    slabs = None
    if ds is not None:
        slabs = (ctypes.c_void_p * len(ds))(*[t.data_ptr() if t is not None else None for t in ds])
        for t in ds:
            _ptr(t)  # device and contiguity checks
    rows, n_ds = _host_rows(ds_rows)
    if caches is None:
        _lib.check(lib.qwen3_model_prefill_logits_last(
            ctypes.byref(m), ctypes.byref(mw), tok, int(s), _ptr(positions), rows, n_ds, slabs,
            _ptr(out), _ptr(workspace), int(workspace.numel()), _stream()))
    else:
        kc, vc = _cache_arrays(caches)
        _lib.check(lib.qwen3_model_prefill_logits_last_kv(
            ctypes.byref(m), ctypes.byref(mw), tok, int(s), _ptr(positions), rows, n_ds, slabs, kc, vc,
            int(caches[0][0].shape[1]) if caches else 0, _ptr(out), _ptr(workspace), int(workspace.numel()),
            _stream()))
    return out


def qk_norm_mrope(q, k, q_norm, k_norm, positions, eps, theta, sections):
    """In place on q [S, nh, hd] and k [S, nkv, hd]; returns (q, k)."""
    lib = _lib.load()
    s, nh, hd = q.shape
    nkv = k.shape[1]
    sec = (ctypes.c_int32 * 3)(*sections)
    _lib.check(lib.qk_norm_mrope(_ptr(q), _ptr(k), int(s), int(nh), int(nkv), int(hd),
                                 _ptr(q_norm), _ptr(k_norm), float(eps), _ptr(positions),
                                 float(theta), sec, _dt(q), _dt(q_norm), _stream()))
    return q, k


def gqa_causal_attention(q, k, v, scale=None, out=None):
    """out [S, nh, hd] = causal GQA softmax(scale q k^T) v."""
    lib = _lib.load()
    s, nh, hd = q.shape
    nkv = k.shape[1]
    if scale is None:
        scale = hd ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _lib.check(lib.gqa_causal_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(s), int(nh),
                                        int(nkv), int(hd), float(scale), _dt(q), _stream()))
    return out


def gqa_bidirectional_attention(q, k, v, scale=None, out=None):
    """out [S, nh, hd] = GQA softmax(scale q k^T) v over every key (no causal mask)."""
    lib = _lib.load()
    s, nh, hd = q.shape
    nkv = k.shape[1]
    if scale is None:
        scale = hd ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _lib.check(lib.gqa_bidirectional_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(s), int(nh),
                                               int(nkv), int(hd), float(scale), _dt(q), _stream()))
    return out


VISION_ROPE_LAYOUTS = {"2d": 0, "3axis": 1}
ROPE_PAIRINGS = {"split": 0, "adjacent": 1}


def vision_rope_tables(grid, head_dim, theta, merge, layout="2d"):
    """(cos, sin) float32 [t*h*w, head_dim] on the GPU for a (t, h, w) patch grid."""
    lib = _lib.load()
    t, h, w = (int(a) for a in grid)
    n = t * h * w
    cos = torch.empty(n, head_dim, dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    _lib.check(lib.vision_rope_tables(t, h, w, int(merge), int(head_dim), float(theta),
                                      VISION_ROPE_LAYOUTS[layout], _ptr(cos), _ptr(sin), _stream()))
    return cos, sin


def apply_rope_tables(x, cos, sin, pairing="split"):
    """In place on x [n, heads, head_dim] (rows may be strided views of a wider row); returns x."""
    lib = _lib.load()
    n, heads, hd = x.shape
    if x.stride(2) != 1 or x.stride(1) != hd:
        raise ValueError("heads of a row must be contiguous")
    _lib.check(lib.apply_rope_tables(ctypes.c_void_p(x.data_ptr()), int(n), int(heads), int(hd),
                                     int(x.stride(0)), _ptr(cos), _ptr(sin), ROPE_PAIRINGS[pairing],
                                     _dt(x), _stream()))
    return x


def swiglu_ffn(x_normed, w_gate, w_up, w_down, residual=None, out_dtype=torch.float32, out=None,
               workspace=None, weights_tiled=False):
    """out [S, H] = [residual +] (silu(x Wg^T) * (x Wu^T)) Wd^T. weights_tiled: the three
    matrices come from tile_weights (wdtype QWEN3_F16_TILED)."""
    lib = _lib.load()
    s, h = x_normed.shape
    f = w_gate.shape[0]
    if out is None:
        out = torch.empty((s, h), dtype=out_dtype, device=x_normed.device)
    need = int(lib.swiglu_ffn_workspace_bytes(int(s), int(f), _dt(x_normed)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x_normed.device)
    _lib.check(lib.swiglu_ffn(_ptr(x_normed), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                              _ptr(residual), _ptr(out), int(s), int(h), int(f),
                              _lib.QWEN3_F16_TILED if weights_tiled else _dt(w_gate),
                              _dt(x_normed), _dt(out), _ptr(workspace), int(workspace.numel()),
                              _stream()))
    return out


def tile_weights(w, out=None):
    """qwen3_tile_weights: a [rows, cols] matrix (f32, bf16 or f16 on the GPU) as fp16 in the
    tiled layout (16-row x 32-column tiles of 1 KiB; element (r, c) at ((r // 16) * (cols // 32)
    + c // 32) * 512 + (r % 16) * 32 + c % 32). The result is a float16 tensor of the same
    shape whose memory holds that order: pass it only where a tiled matrix is expected."""
    if w.dim() != 2:
        raise ValueError("tile_weights takes a 2-D matrix")
    rows, cols = w.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float16, device=w.device)
    _lib.check(_lib.load().qwen3_tile_weights(_ptr(w), _dt(w), int(rows), int(cols), _ptr(out), _stream()))
    return out


def tile_layer_weights(weights):
    """The eleven weights of a layer prepared for dtype "f16t": projection matrices tiled,
    vectors converted to plain fp16."""
    return {n: tile_weights(t) if n in MATRIX_NAMES else t.to(torch.float16).contiguous()
            for n, t in weights.items()}


def rms_norm_rows(x, w, eps, out_dtype=torch.bfloat16, out=None):
    """y [rows, H] = x / sqrt(mean(x^2) + eps) * w, x float32."""
    lib = _lib.load()
    rows, h = x.shape
    if out is None:
        out = torch.empty((rows, h), dtype=out_dtype, device=x.device)
    _lib.check(lib.rms_norm_rows(_ptr(x), _ptr(w), _ptr(out), int(rows), int(h), float(eps),
                                 _dt(w), _dt(out), _stream()))
    return out


def timing_enable(on=True):
    _lib.check(_lib.load().qwen3_timing_enable(1 if on else 0))


def timing_collect(max_entries=64, medians=None):
    """{kernel name: (launches, total ms)} for launches since the last collect; with a dict as
    `medians`, also fills {kernel name: median ms of one launch}."""
    lib = _lib.load()
    arr = (_lib.KernelTime * max_entries)()
    n = ctypes.c_int32(0)
    _lib.check(lib.qwen3_timing_collect(arr, max_entries, ctypes.byref(n)))
    if medians is not None:
        medians.update({arr[i].name.decode(): arr[i].median_ms for i in range(n.value)})
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def mfma_probe(workgroups, iters):
    """qwen3_mfma_probe on the current stream: returns (milliseconds, FLOP, shader clock in GHz)
    of one launch, timed with events around it."""
    lib = _lib.load()
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    _lib.check(lib.qwen3_mfma_probe(int(workgroups), int(iters), _ptr(sink), _ptr(clocks), _stream()))
    e1.record(s)
    torch.cuda.synchronize()
    cyc, ticks = (int(v) for v in clocks.cpu().tolist())
    ghz = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else float("nan")
    flop = float(workgroups) * 4 * iters * 8 * 32768.0
    return e0.elapsed_time(e1), flop, ghz
