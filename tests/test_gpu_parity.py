"""GPU parity: every entry point of the C ABI against the float64 oracle on seeded inputs.

Small cases span several tiles and a ragged tail; the full-size workloads are checked on
sampled rows (and on a prefix of the 4-layer stack, exact by causality).
"""

import numpy as np
import pytest

import oracle
import synth
from util import ALLOW16, ALLOW_ATTN16, TOL, TOL16, dev, dev_i32, dev_weights, err16, host, log_err, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402


def _rng(seed):
    return np.random.default_rng(seed)


def _normal(seed, shape, std=1.0, mean=0.0, dtype="bf16"):
    a = (mean + std * _rng(seed).standard_normal(shape)).astype(np.float32)
    return synth.round_to_bf16(a) if dtype == "bf16" else a


# ------------------------------------------------------------------ RMSNorm (a1, a7)

@pytest.mark.parametrize("wdt,ydt,rows,hidden", [("bf16", "bf16", 37, 2048), ("bf16", "f16", 5, 5120),
                                                 ("f32", "f32", 33, 256), ("f32", "f32", 3, 4096),
                                                 ("bf16", "f32", 7, 16384),
                                                 # more rows than the RMSNorm grid: each
                                                 # workgroup walks two or three rows
                                                 ("bf16", "f16", 3001, 1024)])
def test_rms_norm_rows(wdt, ydt, rows, hidden):
    from transformer_lm_prefill_amd.ops import TORCH_DTYPES
    x = _normal(1, (rows, hidden), dtype="f32") * 3
    w = _normal(2, (hidden,), std=0.1, mean=1.0, dtype=wdt)
    y = q3.rms_norm_rows(dev(x), dev(w, wdt), 1e-6, out_dtype=TORCH_DTYPES[ydt])
    torch.cuda.synchronize()
    ref = oracle.rms_norm(x, w, 1e-6)
    log_err(f"rms_norm_rows[{wdt},{ydt},{rows}x{hidden}]", rel_err(host(y), ref))
    assert err16(host(y), ref, ydt) <= ALLOW16[ydt]


# ------------------------------------------------------------------ q/k norm + MRoPE (a3, a4)

@pytest.mark.parametrize("dtype,ndt,hd,sec,theta,s,nh,nkv,image", [
    ("bf16", "bf16", 128, (24, 20, 20), 5e6, 300, 16, 8, False),
    ("f16", "bf16", 128, (24, 20, 20), 5e6, 1200, 4, 2, True),
    ("f16", "bf16", 128, (24, 20, 20), 5e6, 77, 64, 8, False),
    ("f32", "f32", 64, (12, 10, 10), 1e6, 45, 4, 2, False),
    ("f32", "f32", 128, (24, 20, 20), 5e6, 70, 3, 1, True),
    # one token at the 8B head layout (two passes of rows, one workgroup each) and a few
    # tokens with three passes per token
    ("f16", "bf16", 128, (24, 20, 20), 5e6, 1, 32, 8, False),
    ("bf16", "bf16", 128, (24, 20, 20), 5e6, 3, 64, 8, False),
])
def test_qk_norm_mrope(dtype, ndt, hd, sec, theta, s, nh, nkv, image):
    q = _normal(3, (s, nh, hd), dtype=dtype if dtype != "f16" else "f32") * 2
    k = _normal(4, (s, nkv, hd), dtype=dtype if dtype != "f16" else "f32")
    if dtype == "f16":
        q, k = q.astype(np.float16).astype(np.float32), k.astype(np.float16).astype(np.float32)
    qn = _normal(5, (hd,), std=0.1, mean=1.0, dtype=ndt)
    kn = _normal(6, (hd,), std=0.1, mean=1.0, dtype=ndt)
    if image:
        pos = oracle.mrope_positions(s, [(10, 4, 6)] if s < 1000 else [(100, 32, 32)])
    else:
        pos = np.tile(np.arange(s), (3, 1))
    qd, kd = dev(q, dtype), dev(k, dtype)
    q3.qk_norm_mrope(qd, kd, dev(qn, ndt), dev(kn, ndt), dev_i32(pos), 1e-6, theta, sec)
    torch.cuda.synchronize()
    rq = oracle.qk_norm_mrope(q, qn, 1e-6, pos, theta, sec)
    rk = oracle.qk_norm_mrope(k, kn, 1e-6, pos, theta, sec)
    log_err(f"qk_norm_mrope[{dtype},hd{hd},S{s}]", max(rel_err(host(qd), rq), rel_err(host(kd), rk)))
    assert err16(host(qd), rq, dtype) <= ALLOW16[dtype] and err16(host(kd), rk, dtype) <= ALLOW16[dtype]


def test_qk_norm_mrope_large_positions_bf16():
    s, hd = 64, 128
    q = _normal(7, (s, 2, hd))
    k = _normal(8, (s, 1, hd))
    one = np.ones(hd, np.float32)
    pos = np.tile(8191 - np.arange(s)[::-1] * 3, (3, 1))
    qd, kd = dev(q, "bf16"), dev(k, "bf16")
    q3.qk_norm_mrope(qd, kd, dev(one, "bf16"), dev(one, "bf16"), dev_i32(pos), 1e-6, 5e6, (24, 20, 20))
    torch.cuda.synchronize()
    assert rel_err(host(qd), oracle.qk_norm_mrope(q, one, 1e-6, pos, 5e6, (24, 20, 20))) <= TOL16["bf16"]
    # fp32 data at the same positions: the angle error must stay far below the bf16 level
    qf, kf = dev(q), dev(k)
    q3.qk_norm_mrope(qf, kf, dev(one), dev(one), dev_i32(pos), 1e-6, 5e6, (24, 20, 20))
    torch.cuda.synchronize()
    assert rel_err(host(qf), oracle.qk_norm_mrope(q, one, 1e-6, pos, 5e6, (24, 20, 20))) <= 2e-6


# ------------------------------------------------------------------ attention (a5)

@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("s,nh,nkv", [(1, 4, 1), (77, 8, 2), (300, 16, 8), (333, 8, 1), (250, 8, 8),
                                      (129, 16, 2), (640, 64, 8)])
def test_attention_16bit(fmt, s, nh, nkv):
    hd = 128

    def inp(seed, heads, scale):
        a = _normal(seed, (s, heads, hd), dtype="f32") * scale
        return synth.round_to_bf16(a) if fmt == "bf16" else a.astype(np.float16).astype(np.float32)

    q, k, v = inp(10 + s, nh, 2.0), inp(11 + s, nkv, 2.0), inp(12 + s, nkv, 1.0)
    o = q3.gqa_causal_attention(dev(q, fmt), dev(k, fmt), dev(v, fmt))
    torch.cuda.synchronize()
    ref = oracle.causal_gqa_attention(q, k, v)
    log_err(f"attention[{fmt},S{s},{nh}/{nkv}]", rel_err(host(o), ref))
    assert err16(host(o), ref, fmt) <= ALLOW_ATTN16[fmt]


@pytest.mark.parametrize("s,nh,nkv,hd", [(33, 4, 2, 64), (100, 6, 3, 128), (1, 2, 2, 64)])
def test_attention_f32(s, nh, nkv, hd):
    q = _normal(20, (s, nh, hd), dtype="f32")
    k = _normal(21, (s, nkv, hd), dtype="f32")
    v = _normal(22, (s, nkv, hd), dtype="f32")
    o = q3.gqa_causal_attention(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    assert rel_err(host(o), oracle.causal_gqa_attention(q, k, v)) <= 1e-5


@pytest.mark.parametrize("fmt,s,nh,nkv", [("f16", 333, 16, 4), ("bf16", 97, 8, 8)])
def test_attention_64bit_address_path(monkeypatch, fmt, s, nh, nkv):
    """K/V fetched through 64-bit addresses (the path taken when an operand's byte extent
    exceeds the 32-bit range of buffer loads) give the same bits as the buffer-load path."""
    hd = 128
    q, k, v = (dev(_normal(70 + i, (s, n, hd)) * 2.0, fmt) for i, n in enumerate((nh, nkv, nkv)))
    o_buf = q3.gqa_causal_attention(q, k, v)
    torch.cuda.synchronize()
    monkeypatch.setenv("Q3_ATTN_ADDR64", "1")
    o_64 = q3.gqa_causal_attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o_buf, o_64)
    ref = oracle.causal_gqa_attention(host(q), host(k), host(v))
    assert err16(host(o_64), ref, fmt) <= ALLOW_ATTN16[fmt]


def test_attention_gqa_equals_mha_with_repeated_kv():
    s, nh, nkv, hd = 200, 8, 2, 128
    q, k, v = (dev(_normal(30 + i, (s, n, hd)), "bf16") for i, n in enumerate((nh, nkv, nkv)))
    o1 = q3.gqa_causal_attention(q, k, v)
    o2 = q3.gqa_causal_attention(q, k.repeat_interleave(4, dim=1).contiguous(),
                                 v.repeat_interleave(4, dim=1).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_attention_causality_bitwise():
    s, nh, nkv, hd = 260, 8, 2, 128
    q, k, v = (dev(_normal(40 + i, (s, n, hd)), "bf16") for i, n in enumerate((nh, nkv, nkv)))
    o1 = q3.gqa_causal_attention(q, k, v)
    k2, v2, q2 = k.clone(), v.clone(), q.clone()
    k2[150:] *= -3
    v2[150:] += 1
    q2[150:] *= 0.5
    o2 = q3.gqa_causal_attention(q2, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(o1[:150], o2[:150])
    assert not torch.equal(o1[150:], o2[150:])


# ------------------------------------------------------------------ SwiGLU FFN (a8, a9)

@pytest.mark.parametrize("wdt,xdt,s,h,f,resid", [("bf16", "f16", 300, 2048, 1536, True),
                                                 ("bf16", "bf16", 300, 2048, 1536, True),
                                                 ("bf16", "f16", 64, 256, 640, False),
                                                 ("f16", "f16", 100, 512, 256, True),
                                                 ("f32", "f32", 40, 256, 512, True),
                                                 # 6 x 48 = 288 gate/up tiles with a ragged last
                                                 # tile row: persistent workgroups walk 1-2 tiles
                                                 ("bf16", "f16", 1500, 2048, 6144, True)])
def test_swiglu_ffn(wdt, xdt, s, h, f, resid):
    x = _normal(50, (s, h), dtype="f32")
    x = synth.round_to_bf16(x) if xdt == "bf16" else (x.astype(np.float16).astype(np.float32) if xdt == "f16" else x)
    wd_ = "bf16" if wdt == "bf16" else "f32"
    wg = _normal(51, (f, h), std=0.02, dtype=wd_)
    wu = _normal(52, (f, h), std=0.02, dtype=wd_)
    wd = _normal(53, (h, f), std=0.02, dtype=wd_)
    if wdt == "f16":
        wg, wu, wd = (a.astype(np.float16).astype(np.float32) for a in (wg, wu, wd))
    r = _normal(54, (s, h), dtype="f32") if resid else None
    out = q3.swiglu_ffn(dev(x, xdt), dev(wg, wdt), dev(wu, wdt), dev(wd, wdt),
                        residual=None if r is None else dev(r))
    torch.cuda.synchronize()
    ref = oracle.swiglu_ffn(x, wg, wu, wd) + (0 if r is None else r)
    err = rel_err(host(out), ref)
    log_err(f"swiglu_ffn[{wdt},{xdt},S{s},H{h},F{f}]", err)
    assert err <= (TOL["f32"] if wdt == "f32" else TOL["bf16"])


@pytest.mark.parametrize("wdt,out_dtype,s,h,f", [("bf16", None, 300, 512, 640), ("f16", torch.float16, 300, 512, 640),
                                                 # 288 gate/up tiles: the persistent form walks
                                                 # tiles on the 64-bit path too
                                                 ("bf16", None, 1500, 2048, 6144)])
def test_swiglu_ffn_64bit_address_path(monkeypatch, wdt, out_dtype, s, h, f):
    """GEMM operands fetched through 64-bit addresses (taken when an operand's byte extent
    exceeds the 32-bit range of buffer loads) give the same bits as the buffer-load path."""
    x = dev(_normal(80, (s, h)), "f16")
    wg, wu, wd = (dev(_normal(81 + i, sh, std=0.02), wdt) for i, sh in enumerate(((f, h), (f, h), (h, f))))
    r = None if out_dtype is not None else dev(_normal(84, (s, h), dtype="f32"))
    kw = dict(residual=r) if out_dtype is None else dict(out_dtype=out_dtype)
    o_buf = q3.swiglu_ffn(x, wg, wu, wd, **kw)
    torch.cuda.synchronize()
    monkeypatch.setenv("Q3_GEMM_ADDR64", "1")
    o_64 = q3.swiglu_ffn(x, wg, wu, wd, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_buf, o_64)


def test_swiglu_ffn_bf16_out():
    s, h, f = 100, 512, 384
    x = _normal(60, (s, h))
    wg = _normal(61, (f, h), std=0.02)
    wu = _normal(62, (f, h), std=0.02)
    wd = _normal(63, (h, f), std=0.02)
    for xdt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        xx = x if xdt == "bf16" else x.astype(np.float16).astype(np.float32)
        out = q3.swiglu_ffn(dev(xx, xdt), dev(wg, "bf16"), dev(wu, "bf16"), dev(wd, "bf16"),
                            out_dtype=tdt)
        torch.cuda.synchronize()
        assert rel_err(host(out), oracle.swiglu_ffn(xx, wg, wu, wd)) <= TOL16[xdt]


# ------------------------------------------------------------------ whole layer

def _run_layer(cfg, w, x, pos, ds_rows=None, ds=None, act=""):
    spec = q3.LayerSpec.of(cfg, act)
    out = q3.layer_prefill(spec, dev_weights(w, cfg.dtype), dev(x), dev_i32(pos),
                           None if ds_rows is None else dev_i32(ds_rows),
                           None if ds is None else dev(ds, cfg.dtype))
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3vl_2b_text", "qwen3vl_2b_image"])
def test_layer_matches_oracle(name):
    cfg = synth.get_config(name)
    w = synth.make_layer_weights(cfg)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    ds_rows, ds = synth.make_deepstack(cfg)
    ref = oracle.layer_prefill(x, w, cfg, pos, ds_rows, ds)
    acts = ["f32"] if cfg.dtype == "f32" else ["f16", "bf16"]
    for act in acts:
        err = rel_err(_run_layer(cfg, w, x, pos, ds_rows, ds, act), ref)
        log_err(f"layer[{name},act={act}]", err)
        print(f"{name} act={act}: max|err|/rms = {err:.3e}")
        assert err <= TOL[cfg.dtype], act


@pytest.mark.parametrize("name,s", [("qwen3vl_2b_text", 1), ("qwen3vl_2b_text", 257),
                                    ("qwen3vl_8b_stack4", 300), ("qwen3_32b_encoder", 130),
                                    ("tiny_f32", 1), ("tiny_f32", 97)])
def test_layer_ragged_lengths(name, s):
    cfg = synth.get_config(name).with_seq(s, n_layers=1)
    w = synth.make_layer_weights(cfg)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    err = rel_err(_run_layer(cfg, w, x, pos), oracle.layer_prefill(x, w, cfg, pos))
    log_err(f"layer_ragged[{name},S{s}]", err)
    assert err <= TOL[cfg.dtype]


def test_layer_in_place_and_deterministic():
    cfg = synth.get_config("qwen3vl_2b_image")
    w = dev_weights(synth.make_layer_weights(cfg), "bf16")
    x = dev(synth.make_x(cfg))
    pos = dev_i32(synth.make_positions(cfg))
    rows, ds = synth.make_deepstack(cfg)
    rows, ds = dev_i32(rows), dev(ds, "bf16")
    spec = q3.LayerSpec.of(cfg)
    y1 = q3.layer_prefill(spec, w, x, pos, rows, ds)
    y2 = q3.layer_prefill(spec, w, x, pos, rows, ds)
    xi = x.clone()
    q3.layer_prefill(spec, w, xi, pos, rows, ds, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, xi)


def test_layer_causality_bitwise():
    cfg = synth.get_config("qwen3vl_2b_text")
    w = dev_weights(synth.make_layer_weights(cfg), "bf16")
    x = dev(synth.make_x(cfg))
    pos = dev_i32(synth.make_positions(cfg))
    spec = q3.LayerSpec.of(cfg)
    y1 = q3.layer_prefill(spec, w, x, pos)
    x2 = x.clone()
    x2[700:] = -x2[700:]
    y2 = q3.layer_prefill(spec, w, x2, pos)
    torch.cuda.synchronize()
    assert torch.equal(y1[:700], y2[:700])
    assert not torch.equal(y1[700:], y2[700:])


def test_layer_zero_output_projections_identity_plus_deepstack():
    cfg = synth.get_config("qwen3vl_2b_image")
    w = synth.make_layer_weights(cfg)
    w["wo"] = np.zeros_like(w["wo"])
    w["w_down"] = np.zeros_like(w["w_down"])
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    rows, ds = synth.make_deepstack(cfg)
    y = _run_layer(cfg, w, x, pos, rows, ds)
    ref = x.astype(np.float64).copy()
    ref[rows] += ds
    assert np.array_equal(y, ref.astype(np.float32))


def test_deepstack_invalid_rows_are_skipped():
    cfg = synth.get_config("qwen3vl_2b_text").with_seq(64)
    w = synth.make_layer_weights(cfg)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    rows = np.array([3, 3, 10, 9, 70, 20], dtype=np.int32)   # dup, decreasing, out of range
    ds = _normal(70, (6, cfg.hidden), dtype="bf16")
    base = _run_layer(cfg, w, x, pos)
    y = _run_layer(cfg, w, x, pos, rows, ds)
    # kept: rows 3 (first), 10 (above 3); skipped: the repeated 3, 9 (below 10), 70 (>= S),
    # 20 (below its predecessor 70)
    ref = base.astype(np.float64).copy()
    ref[3] += ds[0]
    ref[10] += ds[2]
    assert np.allclose(y, ref, rtol=0, atol=1e-6)


# ------------------------------------------------------------------ full-size workloads

def test_8b_stack_prefix_and_layer1_sampled_rows():
    """The 4-layer 8B-shaped stack at S=4096: (a) the first 256 output rows of the whole stack
    (exact by causality: the oracle runs the stack on the first 256 tokens); (b) layer 1 on
    sampled rows across the full sequence, including the last positions."""
    cfg = synth.get_config("qwen3vl_8b_stack4")
    layers = [synth.make_layer_weights(cfg, li) for li in range(cfg.n_layers)]
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    spec = q3.LayerSpec.of(cfg)
    dw = [dev_weights(w, "bf16") for w in layers]
    h = dev(x)
    ws = torch.empty(q3.layer_workspace_bytes(spec, cfg.seq_len), dtype=torch.uint8, device="cuda")
    dpos = dev_i32(pos)
    y_first = None
    for li in range(cfg.n_layers):
        h = q3.layer_prefill(spec, dw[li], h, dpos, workspace=ws, out=None)
        if li == 0:
            y_first = h.clone()
    torch.cuda.synchronize()
    out = host(h)
    p = 256
    ref_prefix = oracle.stack_prefill(x[:p], layers, cfg, pos[:, :p])
    err_a = rel_err(out[:p], ref_prefix)
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 3071, 4031, 4094, 4095])
    ref_rows = oracle.layer_prefill_rows(x, layers[0], cfg, pos, rows)
    err_b = rel_err(host(y_first)[rows], ref_rows)
    print(f"8B stack prefix err {err_a:.3e}, layer-1 sampled rows err {err_b:.3e}")
    log_err("8b_stack4[prefix 256 rows, 4 layers]", err_a)
    log_err("8b_stack4[layer 1, sampled rows]", err_b)
    assert err_a <= TOL["bf16"] and err_b <= TOL["bf16"]


def test_32b_encoder_sampled_rows():
    cfg = synth.get_config("qwen3_32b_encoder")
    w = synth.make_layer_weights(cfg)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    y = _run_layer(cfg, w, x, pos)
    rows = np.array([0, 5, 511, 4096, 8000, 8190, 8191])
    err = rel_err(y[rows], oracle.layer_prefill_rows(x, w, cfg, pos, rows))
    print(f"32B encoder sampled rows err {err:.3e}")
    log_err("32b_encoder[sampled rows]", err)
    assert err <= TOL["bf16"]


# ------------------------------------------------------------------ other head layouts

_SHAPES = {
    # name: hidden, n_heads, n_kv_heads, head_dim, ffn, seq_len, sections
    "hd64_mha": (1024, 16, 16, 64, 2048, 300, (12, 10, 10)),
    "hd64_gqa4": (1024, 16, 4, 64, 2048, 333, (12, 10, 10)),
    "hd128_gqa8": (2048, 16, 2, 128, 2048, 200, (24, 20, 20)),
    # 3 heads of 64: the o-projection has K = 192, 6 K steps per tile, not a multiple of the
    # 4-stage ring (the GEMM's tail steps)
    "hd64_mha3_k192": (256, 3, 3, 64, 256, 150, (12, 10, 10)),
}


@pytest.mark.parametrize("shape", sorted(_SHAPES))
def test_layer_and_decode_other_head_layouts(shape):
    """The layer (16-bit path) and a decode step after it on head layouts the named workloads do
    not use: head_dim 64 with and without grouping, 8 query heads per KV head."""
    h, nh, nkv, hd, f, s, sec = _SHAPES[shape]
    cfg = synth.LayerConfig(name=shape, hidden=h, n_heads=nh, n_kv_heads=nkv, head_dim=hd, ffn=f,
                            seq_len=s + 1, sections=sec, theta=1e6)
    w = synth.make_layer_weights(cfg)
    x, pos = synth.make_x(cfg), synth.make_positions(cfg)
    ref = oracle.layer_prefill(x, w, cfg, pos)
    spec = q3.LayerSpec.of(cfg)
    dw = dev_weights(w, cfg.dtype)
    kc, vc = q3.kv_cache_alloc(spec, s + 1)
    y = host(q3.layer_prefill_kv(spec, dw, dev(x[:s]), dev_i32(pos[:, :s]), kc, vc))
    err = rel_err(y, ref[:s])
    yd = host(q3.layer_decode(spec, dw, dev(x[s]), dev_i32(pos[:, s]), kc, vc, s))
    err_d = rel_err(yd, ref[s])
    log_err(f"layer[{shape}]", err)
    log_err(f"layer_decode[{shape}]", err_d)
    assert err <= TOL[cfg.dtype] and err_d <= TOL[cfg.dtype], (err, err_d)
