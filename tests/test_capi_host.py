"""Host-side checks of the C ABI library: it loads, exports every symbol the header declares,
and rejects invalid arguments with the documented status before touching the GPU."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwen3_prefill.h")

L = pytest.importorskip("transformer_lm_prefill_amd._lib")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    return L.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\*?\s*(\w+)\s*\(", src, flags=re.M))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("qwen3_layer_prefill", "qk_norm_mrope", "gqa_causal_attention", "swiglu_ffn",
              "qwen3_layer_workspace_bytes", "qwen3_last_error", "rms_norm_rows"):
        assert n in names
    assert names == set(L.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def _cfg(**kw):
    c = L.LayerCfg()
    d = dict(hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128, ffn=6144, rms_eps=1e-6,
             rope_theta=5e6, wdtype=L.QWEN3_BF16, act_dtype=L.QWEN3_F16, resid_dtype=L.QWEN3_F32)
    d.update(kw)
    sec = d.pop("sections", (24, 20, 20))
    for k, v in d.items():
        setattr(c, k, v)
    c.mrope_section = (ctypes.c_int32 * 3)(*sec)
    return c


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its checks first


def _weights():
    return L.LayerWeights(*([FAKE] * 11))


def _call_layer(lib, cfg, s=16, ws_bytes=None, n_ds=0, ds=None, ds_rows=None, weights=None,
                x_out=FAKE, workspace=ctypes.c_void_p(0x100000)):
    if ws_bytes is None:
        ws_bytes = lib.qwen3_layer_workspace_bytes(ctypes.byref(cfg), max(s, 1))
    w = weights or _weights()
    return lib.qwen3_layer_prefill(ctypes.byref(cfg), ctypes.byref(w), FAKE, x_out, s, FAKE,
                                   ds_rows, n_ds, ds, workspace, ws_bytes, None)


def test_workspace_size_formula(lib):
    c = _cfg(hidden=4096, n_heads=32, n_kv_heads=8, ffn=12288)
    s = 4096
    # 16-bit xn | qkv | o | act, then the DeepStack row list (S int32)
    expect = 2 * s * (4096 + (4096 + 2048) + 4096 + 12288)
    assert lib.qwen3_layer_workspace_bytes(ctypes.byref(c), s) == expect + 4 * s
    c32 = _cfg(hidden=4096, n_heads=32, n_kv_heads=8, ffn=12288, wdtype=0, act_dtype=0)
    assert lib.qwen3_layer_workspace_bytes(ctypes.byref(c32), s) == 2 * expect + 4 * s
    assert lib.qwen3_layer_workspace_bytes(ctypes.byref(c), 0) == 0
    assert lib.qwen3_layer_workspace_bytes(None, 16) == 0
    # a ragged length: xn, o and act (the product A operands, tiled for 16-bit operands) take
    # whole 16-row groups; qkv and the row list take S rows
    a256 = lambda b: (b + 255) // 256 * 256
    s, s16 = 77, 80
    expect = (a256(2 * s16 * 4096) + a256(2 * s * 6144) + a256(2 * s16 * 4096) + a256(2 * s16 * 12288)
              + a256(4 * s))
    assert lib.qwen3_layer_workspace_bytes(ctypes.byref(c), s) == expect


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n_heads=12, n_kv_heads=8), 1, "multiple of n_kv_heads"),
    (dict(n_heads=32, n_kv_heads=2), 2, "1, 2, 4 or 8"),
    (dict(head_dim=96, sections=(16, 16, 16)), 2, "head_dim must be 64 or 128"),
    (dict(wdtype=0, act_dtype=2), 2, "supported pairs"),
    (dict(wdtype=2, act_dtype=1), 2, "supported pairs"),
    (dict(act_dtype=9), 1, "qwen3_dtype"),
    (dict(sections=(24, 20, 21)), 1, "sum to head_dim/2"),
    (dict(sections=(4, 30, 30)), 1, "interleaved"),
    (dict(hidden=1000), 2, "multiple of 256"),
    (dict(ffn=100), 2, "multiple of 128"),
    (dict(resid_dtype=1), 2, "resid_dtype"),
    (dict(wdtype=7), 1, "qwen3_dtype"),
    (dict(rope_theta=0.5), 1, "rope_theta"),
    (dict(rms_eps=-1.0), 1, "rms_eps"),
])
def test_bad_config_rejected(lib, kw, status, needle):
    rc = _call_layer(lib, _cfg(**kw))
    assert rc == status
    assert needle in lib.qwen3_last_error().decode()


def test_empty_sequence_rejected(lib):
    rc = _call_layer(lib, _cfg(), s=0, ws_bytes=1 << 30)
    assert rc == 1 and "empty" in lib.qwen3_last_error().decode()


def _rows(*r):
    return (ctypes.c_int32 * len(r))(*r)


def test_deepstack_argument_rules(lib):
    """The DeepStack row list is a host array checked before anything is enqueued (hf2q
    forward.rs, `forward_text_prefill_logits_last`: an image-token position outside the
    sequence is an error, and a slab needs its rows)."""
    c = _cfg()
    assert _call_layer(lib, c, n_ds=0, ds=FAKE) == 1
    assert "n_ds == 0" in lib.qwen3_last_error().decode()
    assert _call_layer(lib, c, n_ds=4, ds=FAKE, ds_rows=None) == 1
    assert "ds_rows" in lib.qwen3_last_error().decode()
    assert _call_layer(lib, c, n_ds=17, ds=FAKE, ds_rows=_rows(*range(17))) == 1
    assert _call_layer(lib, c, n_ds=-1) == 1
    # S = 16: a row at or past S, a negative row, a repeat and a decrease are each rejected
    for bad, needle in (((3, 16), "outside"), ((-1, 4), "outside"), ((3, 3), "strictly increasing"),
                        ((5, 9, 7), "strictly increasing")):
        assert _call_layer(lib, c, n_ds=len(bad), ds=FAKE, ds_rows=_rows(*bad)) == 1, bad
        assert needle in lib.qwen3_last_error().decode(), bad
    # rows given but no slab
    assert _call_layer(lib, c, n_ds=2, ds=None, ds_rows=_rows(1, 2)) == 1
    # a valid list passes these checks: the call then stops at the (too small) workspace
    need = lib.qwen3_layer_workspace_bytes(ctypes.byref(c), 16)
    assert _call_layer(lib, c, n_ds=3, ds=FAKE, ds_rows=_rows(0, 7, 15), ws_bytes=need - 1) == 3


def test_qk_norm_mrope_rejects_empty_head_counts(lib):
    """Both head counts must be >= 1: the kernel reads both norm weight vectors."""
    sec = (ctypes.c_int32 * 3)(24, 20, 20)
    for nh, nkv in ((0, 8), (32, 0), (0, 0)):
        rc = lib.qk_norm_mrope(FAKE, FAKE, 4, nh, nkv, 128, FAKE, FAKE, 1e-6, FAKE, 5e6, sec,
                               L.QWEN3_F16, L.QWEN3_BF16, None)
        assert rc == 1 and "must be >= 1" in lib.qwen3_last_error().decode(), (nh, nkv)
    # a NULL q or k is rejected as well
    rc = lib.qk_norm_mrope(None, FAKE, 4, 32, 8, 128, FAKE, FAKE, 1e-6, FAKE, 5e6, sec,
                           L.QWEN3_F16, L.QWEN3_BF16, None)
    assert rc == 1 and "NULL" in lib.qwen3_last_error().decode()


def test_null_weight_and_workspace_rejected(lib):
    c = _cfg()
    w = _weights()
    w.k_norm = None
    assert _call_layer(lib, c, weights=w) == 1
    assert "k_norm" in lib.qwen3_last_error().decode()
    need = lib.qwen3_layer_workspace_bytes(ctypes.byref(c), 16)
    assert _call_layer(lib, c, ws_bytes=need - 1) == 3
    assert _call_layer(lib, c, workspace=None) == 3
    assert _call_layer(lib, c, workspace=ctypes.c_void_p(0x100010)) == 3


def test_partial_overlap_rejected(lib):
    assert _call_layer(lib, _cfg(), x_out=ctypes.c_void_p(0x1000 + 64)) == 1
    assert "overlap" in lib.qwen3_last_error().decode()


def test_misaligned_pointers_rejected(lib):
    odd = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    c = _cfg()
    rc = lib.qwen3_layer_prefill(ctypes.byref(c), ctypes.byref(_weights()), odd, odd, 16, FAKE,
                                 None, 0, None, ctypes.c_void_p(0x100000),
                                 lib.qwen3_layer_workspace_bytes(ctypes.byref(c), 16), None)
    assert rc == 1 and "16-byte" in lib.qwen3_last_error().decode()
    w = _weights()
    w.w_down = odd
    assert _call_layer(lib, c, weights=w) == 1
    assert lib.gqa_causal_attention(FAKE, odd, FAKE, FAKE, 8, 4, 2, 128, 0.1, 1, None) == 1
    assert "16-byte" in lib.qwen3_last_error().decode()
    assert lib.swiglu_ffn(FAKE, FAKE, odd, FAKE, None, FAKE, 8, 2048, 6144, 1, 2, 0, FAKE, 1 << 30, None) == 1
    assert lib.rms_norm_rows(FAKE, FAKE, odd, 4, 256, 1e-6, 1, 1, None) == 1
    sec = (ctypes.c_int32 * 3)(24, 20, 20)
    assert lib.qk_norm_mrope(odd, FAKE, 4, 4, 2, 128, FAKE, FAKE, 1e-6, FAKE, 5e6, sec, 1, 1, None) == 1


def test_sub_op_argument_checks(lib):
    sec = (ctypes.c_int32 * 3)(24, 20, 20)
    assert lib.qk_norm_mrope(FAKE, FAKE, 0, 4, 2, 128, FAKE, FAKE, 1e-6, FAKE, 5e6, sec, 1, 1, None) == 1
    assert lib.qk_norm_mrope(FAKE, FAKE, 4, 4, 2, 96, FAKE, FAKE, 1e-6, FAKE, 5e6, sec, 1, 1, None) == 2
    assert lib.qk_norm_mrope(FAKE, FAKE, 4, 4, 2, 128, FAKE, FAKE, 1e-6, FAKE, 5e6, sec, 1, 5, None) == 1
    assert lib.gqa_causal_attention(FAKE, FAKE, FAKE, FAKE, 8, 6, 4, 128, 0.1, 1, None) == 1
    assert lib.gqa_causal_attention(FAKE, FAKE, FAKE, FAKE, 8, 4, 2, 128, 0.0, 1, None) == 1
    assert lib.gqa_causal_attention(FAKE, FAKE, FAKE, FAKE, 8, 4, 2, 96, 0.1, 1, None) == 2
    assert lib.gqa_bidirectional_attention(FAKE, FAKE, FAKE, FAKE, 8, 6, 4, 128, 0.1, 1, None) == 1
    assert lib.gqa_bidirectional_attention(FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 128, 0.1, 1, None) == 1
    assert lib.vision_rope_tables(1, 4, 6, 4, 64, 1e4, 0, FAKE, FAKE, None) == 1      # 6 % merge
    assert lib.vision_rope_tables(1, 4, 4, 2, 48, 1e4, 1, FAKE, FAKE, None) == 1      # 3-axis needs hd % 32
    assert lib.vision_rope_tables(1, 4, 4, 2, 64, 1e4, 2, FAKE, FAKE, None) == 1      # layout
    assert lib.apply_rope_tables(FAKE, 4, 2, 64, 100, FAKE, FAKE, 0, 1, None) == 1    # stride < heads*hd
    assert lib.apply_rope_tables(FAKE, 4, 2, 64, 128, FAKE, FAKE, 3, 1, None) == 1    # pairing
    assert lib.swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 2048, 6144, 1, 2, 0, FAKE, 10, None) == 3
    assert lib.swiglu_ffn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 2048, 6144, 1, 2, 2, FAKE, 1 << 30, None) == 2
    assert lib.swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 2048, 6144, 1, 2, 1, FAKE, 1 << 30, None) == 2
    assert lib.swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 2048, 6144, 0, 1, 0, FAKE, 1 << 30, None) == 2
    assert lib.rms_norm_rows(FAKE, FAKE, FAKE, 4, 300, 1e-6, 1, 1, None) == 2
    assert lib.rms_norm_rows(FAKE, FAKE, FAKE, 0, 256, 1e-6, 1, 1, None) == 1


def _model_cfg(n_layers=2, vocab=100, n_ds_layers=0, **kw):
    m = L.ModelCfg()
    m.layer = _cfg(**kw)
    m.n_layers, m.vocab, m.n_deepstack_layers = n_layers, vocab, n_ds_layers
    return m


def _call_model(lib, m, tokens, ws_bytes=None, n_ds=0, ds_rows=None, slabs=None):
    s = len(tokens)
    if ws_bytes is None:
        ws_bytes = lib.qwen3_model_workspace_bytes(ctypes.byref(m), max(s, 1))
    lw = (L.LayerWeights * max(m.n_layers, 1))(*([_weights()] * max(m.n_layers, 1)))
    mw = L.ModelWeights(FAKE, lw, FAKE, None)
    tok = (ctypes.c_int32 * max(s, 1))(*tokens)
    return lib.qwen3_model_prefill_logits_last(ctypes.byref(m), ctypes.byref(mw), tok, s, FAKE, ds_rows,
                                               n_ds, slabs, FAKE, ctypes.c_void_p(0x100000), ws_bytes, None)


def test_model_workspace_formula(lib):
    m = _model_cfg(n_layers=4, vocab=1000, hidden=4096, n_heads=32, n_kv_heads=8, ffn=12288)
    s = 300
    layer = lib.qwen3_layer_workspace_bytes(ctypes.byref(m.layer), s)
    def a256(b):
        return (b + 255) // 256 * 256
    assert lib.qwen3_model_workspace_bytes(ctypes.byref(m), s) == a256(4 * s) + a256(4 * s * 4096) + a256(4 * 4096) + layer
    assert lib.qwen3_model_workspace_bytes(ctypes.byref(m), 0) == 0
    assert lib.qwen3_model_workspace_bytes(None, 16) == 0


def test_model_argument_checks(lib):
    m = _model_cfg()
    assert _call_model(lib, m, [1, 100, 3]) == 1
    assert "outside [0, vocab = 100)" in lib.qwen3_last_error().decode()
    assert _call_model(lib, m, [-1]) == 1
    assert _call_model(lib, m, []) == 1 and "empty" in lib.qwen3_last_error().decode()
    assert _call_model(lib, _model_cfg(n_layers=2, n_ds_layers=3), [1, 2]) == 1
    assert "n_deepstack_layers" in lib.qwen3_last_error().decode()
    assert _call_model(lib, _model_cfg(vocab=0), [0]) == 1
    assert _call_model(lib, _model_cfg(n_layers=-1), [0]) == 1
    assert _call_model(lib, _model_cfg(n_ds_layers=1), [1, 2], n_ds=1, ds_rows=None) == 1
    slab = (ctypes.c_void_p * 1)(0x2000)
    assert _call_model(lib, _model_cfg(n_ds_layers=1), [1, 2], n_ds=1, ds_rows=_rows(2), slabs=slab) == 1
    assert "outside" in lib.qwen3_last_error().decode()
    assert _call_model(lib, _model_cfg(n_ds_layers=1), [1, 2, 3], n_ds=2, ds_rows=_rows(1, 1), slabs=slab) == 1
    assert "strictly increasing" in lib.qwen3_last_error().decode()
    m2 = _model_cfg()
    need = lib.qwen3_model_workspace_bytes(ctypes.byref(m2), 3)
    assert _call_model(lib, m2, [1, 2, 3], ws_bytes=need - 1) == 3


def test_timing_collect_empty(lib):
    n = ctypes.c_int32(-1)
    assert lib.qwen3_timing_collect(None, 0, ctypes.byref(n)) == 0 and n.value == 0


# ---- KV cache and decode step: every call below fails a host check before any launch

def test_kv_cache_write_argument_checks(lib):
    # rows [50, 90) do not fit a capacity of 80
    assert lib.kv_cache_write(FAKE, FAKE, 512, 512, 40, 4, 128, 2, FAKE, FAKE, 2, 80, 50, None) == 1
    assert "capacity" in lib.qwen3_last_error().decode()
    assert lib.kv_cache_write(FAKE, FAKE, 512, 512, 4, 4, 100, 2, FAKE, FAKE, 2, 80, 0, None) == 2   # hd % 8
    assert lib.kv_cache_write(FAKE, FAKE, 256, 512, 4, 4, 128, 2, FAKE, FAKE, 2, 80, 0, None) == 1   # stride
    assert lib.kv_cache_write(FAKE, FAKE, 512, 512, 4, 4, 128, 2, FAKE, FAKE, 5, 80, 0, None) == 1   # dtype
    assert lib.kv_cache_write(FAKE, FAKE, 512, 512, 0, 4, 128, 2, FAKE, FAKE, 2, 80, 0, None) == 1   # n
    assert lib.kv_cache_write(FAKE, None, 512, 512, 4, 4, 128, 2, FAKE, FAKE, 2, 80, 0, None) == 1
    odd = ctypes.c_void_p(0x1002)
    assert lib.kv_cache_write(FAKE, FAKE, 512, 512, 4, 4, 128, 2, odd, FAKE, 2, 80, 0, None) == 1


def test_decode_attention_argument_checks(lib):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 30
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 17, 8, 2, 128, 0.1, 2, FAKE, ws, big, None) == 1   # len > cap
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 0, 8, 2, 128, 0.1, 2, FAKE, ws, big, None) == 1    # len 0
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 8, 34, 2, 128, 0.1, 2, FAKE, ws, big, None) == 2   # group 17
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 8, 8, 2, 96, 0.1, 2, FAKE, ws, big, None) == 2     # hd 96
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 8, 8, 3, 128, 0.1, 2, FAKE, ws, big, None) == 1    # 8 % 3
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 8, 8, 2, 128, 0.0, 2, FAKE, ws, big, None) == 1    # scale
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 8, 8, 2, 128, 0.1, 2, FAKE, ws, 16, None) == 3     # workspace
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 16, 8, 8, 2, 128, 0.1, 2, FAKE, ctypes.c_void_p(0x100010),
                                    big, None) == 3                                                           # alignment


def test_decode_workspace_formula(lib):
    def a256(b):
        return (b + 255) // 256 * 256
    # 8 KV heads: about 512 workgroups, so at most 64 key splits; 4096 keys = 64 tiles of 64
    assert lib.gqa_decode_attention_workspace_bytes(32, 8, 128, 4096) == a256(32 * 64 * 128 * 4) + a256(32 * 64 * 8)
    assert lib.gqa_decode_attention_workspace_bytes(32, 8, 128, 100) == a256(32 * 2 * 128 * 4) + a256(32 * 2 * 8)
    assert lib.gqa_decode_attention_workspace_bytes(32, 8, 128, 10 ** 6) == lib.gqa_decode_attention_workspace_bytes(
        32, 8, 128, 4096)
    assert lib.gqa_decode_attention_workspace_bytes(32, 8, 128, 0) == 0
    c = _cfg(hidden=4096, n_heads=32, n_kv_heads=8, ffn=12288)
    attn = lib.gqa_decode_attention_workspace_bytes(32, 8, 128, 8192)
    want = a256(4096 * 4) + a256((4096 + 2048) * 4) + a256(4096 * 4) + a256(12288 * 4) + attn
    assert lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(c), 8192) == want
    assert lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(c), 0) == 0


def test_layer_decode_and_prefill_kv_argument_checks(lib):
    c = _cfg()
    w = _weights()
    ws = ctypes.c_void_p(0x100000)
    need = lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(c), 64)
    # len must leave the new token's row inside the cache
    assert lib.qwen3_layer_decode(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x2000),
                                  64, 64, ws, need, None) == 1
    assert "capacity" in lib.qwen3_last_error().decode()
    assert lib.qwen3_layer_decode(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, 64, 3, ws, need,
                                  None) == 1                                                 # same k and v cache
    assert lib.qwen3_layer_decode(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x2000),
                                  64, 3, ws, need - 256, None) == 3
    assert lib.qwen3_layer_decode(ctypes.byref(_cfg(n_heads=32, n_kv_heads=1)), ctypes.byref(w), FAKE, FAKE, FAKE,
                                  FAKE, ctypes.c_void_p(0x2000), 64, 3, ws, 1 << 30, None) == 2
    ws_p = lib.qwen3_layer_workspace_bytes(ctypes.byref(c), 16)
    assert lib.qwen3_layer_prefill_kv(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 16, FAKE, None, 0, None, FAKE,
                                      ctypes.c_void_p(0x2000), 15, ws, ws_p, None) == 1     # capacity < S
    assert lib.qwen3_layer_prefill_kv(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 16, FAKE, None, 0, None, None,
                                      ctypes.c_void_p(0x2000), 16, ws, ws_p, None) == 1


# ---- quantized weights: every call below fails a host check before any launch

def _qweights(fmt=1, data=FAKE, rs=None, **over):
    m = {n: L.QMatrix(fmt, data, rs) for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")}
    for k, v in over.items():
        m[k] = v
    return L.LayerQWeights(attn_norm=FAKE, q_norm=FAKE, k_norm=FAKE, ffn_norm=FAKE, **m)


def test_quant_weight_rules(lib):
    c = _cfg(act_dtype=2)
    ws = ctypes.c_void_p(0x100000)
    need = lib.qwen3_layer_quant_workspace_bytes(ctypes.byref(c), 16)
    assert need > lib.qwen3_layer_workspace_bytes(ctypes.byref(c), 16)

    def call(w, ws_bytes=need, cfg=c):
        return lib.qwen3_layer_prefill_quant(ctypes.byref(cfg), ctypes.byref(w), FAKE, FAKE, 16, FAKE, None, 0, None,
                                             None, None, 0, ws, ws_bytes, None)
    assert call(_qweights(fmt=7)) == 1 and "qwen3_wformat" in lib.qwen3_last_error().decode()
    assert call(_qweights(wk=L.QMatrix(0, FAKE, None))) == 2                  # dense wk with quantized wq
    assert "all dense or all quantized" in lib.qwen3_last_error().decode()
    assert call(_qweights(w_up=L.QMatrix(2, FAKE, FAKE))) == 2                # gate Q4_0, up q8
    assert call(_qweights(fmt=2, rs=None)) == 1 and "row_scale" in lib.qwen3_last_error().decode()
    assert call(_qweights(data=ctypes.c_void_p(0x1002))) == 1                 # Q4_0 needs 4-byte alignment
    assert call(_qweights(fmt=2, data=ctypes.c_void_p(0x1004), rs=FAKE)) == 1  # int8 rows need 16 bytes
    assert call(_qweights(), need - 256) == 3
    assert call(_qweights(), cfg=_cfg(wdtype=0, act_dtype=0, head_dim=64, sections=(12, 10, 10))) == 2
    assert "16-bit operands" in lib.qwen3_last_error().decode()
    # caches must come in pairs
    assert lib.qwen3_layer_prefill_quant(ctypes.byref(c), ctypes.byref(_qweights()), FAKE, FAKE, 16, FAKE, None, 0,
                                         None, FAKE, None, 16, ws, need, None) == 1
    dws = lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(c), 64)
    assert lib.qwen3_layer_decode_quant(ctypes.byref(c), ctypes.byref(_qweights(fmt=9)), FAKE, FAKE, FAKE, FAKE,
                                        ctypes.c_void_p(0x2000), 64, 3, ws, dws, None) == 1


def test_dequantize_matrix_checks(lib):
    m = L.QMatrix(1, FAKE, None)
    assert lib.dequantize_matrix(ctypes.byref(m), 4, 96, 2, FAKE, None) == 2      # cols % 64
    assert lib.dequantize_matrix(ctypes.byref(m), 4, 128, 0, FAKE, None) == 2     # f32 output
    assert lib.dequantize_matrix(ctypes.byref(L.QMatrix(0, FAKE, None)), 4, 128, 2, FAKE, None) == 1
    assert lib.dequantize_matrix(ctypes.byref(m), 0, 128, 2, FAKE, None) == 1
    assert lib.dequantize_matrix(ctypes.byref(L.QMatrix(2, FAKE, None)), 4, 128, 2, FAKE, None) == 1


def test_model_decode_argument_checks(lib):
    m = _model_cfg(n_layers=2, vocab=100)
    lw = (L.LayerWeights * 2)(_weights(), _weights())
    mw = L.ModelWeights(FAKE, lw, FAKE, None)
    ws = ctypes.c_void_p(0x100000)
    need = lib.qwen3_model_decode_workspace_bytes(ctypes.byref(m), 64)
    assert need > lib.qwen3_layer_decode_workspace_bytes(ctypes.byref(m.layer), 64)
    kc = (ctypes.c_void_p * 2)(0x2000, 0x3000)
    vc = (ctypes.c_void_p * 2)(0x4000, 0x5000)

    def call(token=5, length=3, caches=(kc, vc), ws_bytes=need, cap=64):
        return lib.qwen3_model_decode_logits(ctypes.byref(m), ctypes.byref(mw), token, FAKE, caches[0], caches[1],
                                             cap, length, FAKE, ws, ws_bytes, None)
    assert call(token=100) == 1 and "vocab" in lib.qwen3_last_error().decode()
    assert call(token=-1) == 1
    assert call(length=64) == 1 and "capacity" in lib.qwen3_last_error().decode()
    assert call(caches=(kc, None)) == 1
    assert call(caches=(kc, (ctypes.c_void_p * 2)(0x2000, 0x5000))) == 1      # layer 0: same k and v
    assert call(ws_bytes=need - 256) == 3
    # the model prefill that leaves the caches checks them the same way
    tok = (ctypes.c_int32 * 16)(*range(16))
    mws = lib.qwen3_model_workspace_bytes(ctypes.byref(m), 16)
    assert lib.qwen3_model_prefill_logits_last_kv(ctypes.byref(m), ctypes.byref(mw), tok, 16, FAKE, None, 0, None,
                                                  kc, vc, 15, FAKE, ws, mws, None) == 1
    assert lib.qwen3_model_prefill_logits_last_kv(ctypes.byref(m), ctypes.byref(mw), tok, 16, FAKE, None, 0, None,
                                                  None, None, 16, FAKE, ws, mws, None) == 1


def test_tiled_weight_format_rules(lib):
    """QWEN3_F16_TILED (3) is a weight format for fp16 operands only, never an operand type."""
    assert _call_layer(lib, _cfg(wdtype=3, act_dtype=1)) == 2     # with bf16 operands
    assert _call_layer(lib, _cfg(wdtype=3, act_dtype=0)) == 2     # with f32 operands
    assert _call_layer(lib, _cfg(wdtype=2, act_dtype=3)) == 1     # as an operand type
    assert _call_layer(lib, _cfg(wdtype=3, act_dtype=2), ws_bytes=16) == 3   # accepted: stops at the workspace


def test_tile_weights_checks(lib):
    """Every rejection happens before anything is enqueued (fake pointers, never dereferenced)."""
    src = ctypes.c_void_p(0x200000)
    dst = ctypes.c_void_p(0x800000)
    t = lib.qwen3_tile_weights
    assert t(None, 1, 64, 128, dst, None) == 1                      # NULL source
    assert t(src, 1, 64, 128, None, None) == 1                      # NULL destination
    assert t(src, 3, 64, 128, dst, None) == 1                       # the tiled format is no source type
    assert t(src, 7, 64, 128, dst, None) == 1                       # not a dtype
    assert t(ctypes.c_void_p(0x200008), 1, 64, 128, dst, None) == 1  # misaligned
    assert t(src, 1, 60, 128, dst, None) == 2                       # rows not a multiple of 16
    assert t(src, 1, 64, 112, dst, None) == 2                       # cols not a multiple of 32
    assert t(src, 1, 0, 128, dst, None) == 2
    # bf16 [64, 128] spans 16 KiB from src: a destination starting inside it overlaps
    assert t(src, 1, 64, 128, ctypes.c_void_p(0x200000 + 0x3000), None) == 1
    assert t(src, 0, 64, 128, ctypes.c_void_p(0x200000 - 0x3000), None) == 1   # dst (16 KiB) runs into src
    assert b"overlap" in lib.qwen3_last_error()
