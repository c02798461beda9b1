"""GPU parity: every entry point of the C ABI against the float64 oracle on seeded inputs.

Small cases span several tiles and a ragged tail; the full-size workloads (the 8B-shaped
4-layer stack at 4096 tokens and the 32B-shaped layer at 8192 tokens) are compared on every
output row.
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


def test_rms_norm_degenerate_rows():
    """Rows of zeros give exact zeros (the mean of squares is 0, the scale 1/sqrt(eps) multiplies
    zeros); rows far below eps in magnitude are scaled by about 1/sqrt(eps); one nonzero element
    in a row gives +-sqrt(H)-scaled weight there (closed form of the definition)."""
    rows, hidden = 40, 2048
    x = _normal(3, (rows, hidden), dtype="f32")
    x[0:5] = 0.0
    x[5:10] *= 1e-12
    x[10:15] = 0.0
    x[10:15, 7] = 5.0
    w = _normal(4, (hidden,), std=0.1, mean=1.0, dtype="bf16")
    y = host(q3.rms_norm_rows(dev(x), dev(w, "bf16"), 1e-6, out_dtype=torch.float32))
    assert np.all(y[0:5] == 0.0)
    ref = oracle.rms_norm(x, w, 1e-6)
    # elementwise: an fp32 reciprocal square root and two products (a few ulps of each element;
    # the single-element rows hold values ~30x the RMS, beyond what the generic allowance
    # assumes) plus the mean's summation error
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    assert np.all(np.abs(y - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 2e-6 * rms)
    # one element 5 in a row of H: mean of squares 25/H, so y = 5 / sqrt(25/H + eps) * w
    expect = 5.0 / np.sqrt(25.0 / hidden + 1e-6) * w[7]
    assert np.allclose(y[10:15, 7], expect, rtol=2e-6) and np.all(np.delete(y[10:15], 7, axis=1) == 0.0)


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


def test_qk_norm_mrope_zero_heads_and_position_zero():
    """Head vectors of zeros stay exact zeros (normalized by 1/sqrt(eps), then rotated); at
    position 0 on every axis the rotation is the identity, so the output is the plain per-head
    RMSNorm of the row."""
    s, nh, nkv, hd = 20, 4, 2, 128
    q = _normal(9, (s, nh, hd), dtype="f32")
    k = _normal(10, (s, nkv, hd), dtype="f32")
    q[3, 1] = 0.0
    k[7, 0] = 0.0
    pos = np.tile(np.arange(s), (3, 1))
    pos[:, 0] = 0
    nq = _normal(11, (hd,), std=0.1, mean=1.0, dtype="f32")
    nk = _normal(12, (hd,), std=0.1, mean=1.0, dtype="f32")
    qd, kd = dev(q), dev(k)
    q3.qk_norm_mrope(qd, kd, dev(nq), dev(nk), dev_i32(pos), 1e-6, 5e6, (24, 20, 20))
    torch.cuda.synchronize()
    hq, hk = host(qd), host(kd)
    assert np.all(hq[3, 1] == 0.0) and np.all(hk[7, 0] == 0.0)
    # token 0 sits at position 0: only the normalization applies
    assert rel_err(hq[0], oracle.rms_norm(q[0], nq, 1e-6)) <= 2e-6
    assert rel_err(hk[0], oracle.rms_norm(k[0], nk, 1e-6)) <= 2e-6
    assert rel_err(hq, oracle.qk_norm_mrope(q, nq, 1e-6, pos, 5e6, (24, 20, 20))) <= 2e-6


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


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("pattern", ["rising", "spikes"])
def test_attention_running_max_stress(fmt, pattern):
    """Scores that keep raising the running maximum, tile after tile, by far more than the lazy
    rescaling's slack (rising: key j scaled by 1 + j/32, so a row's largest score grows ~30x
    along the sequence; spikes: every 50th key is a scaled copy of a query row, a score far
    above all others that must dominate its rows' softmax)."""
    s, nh, nkv, hd = 700, 8, 2, 128

    def rnd(a):
        return synth.round_to_bf16(a) if fmt == "bf16" else a.astype(np.float16).astype(np.float32)

    q = _normal(80, (s, nh, hd), dtype="f32")
    k = _normal(81, (s, nkv, hd), dtype="f32")
    v = _normal(82, (s, nkv, hd), dtype="f32")
    if pattern == "rising":
        k = k * (1.0 + np.arange(s, dtype=np.float32) / 32.0)[:, None, None]
    else:
        for j in range(0, s, 50):
            k[j] = 3.0 * q[min(j + 5, s - 1), ::nh // nkv]
    q, k, v = rnd(q), rnd(k), rnd(v)
    o = q3.gqa_causal_attention(dev(q, fmt), dev(k, fmt), dev(v, fmt))
    torch.cuda.synchronize()
    ref = oracle.causal_gqa_attention(q, k, v)
    log_err(f"attention[{fmt},{pattern}]", rel_err(host(o), ref))
    assert np.all(np.isfinite(host(o)))
    # bf16 operands carry the probabilities with an 8-bit significand: where one key dominates a
    # row, rounding its neighbours' probabilities moves o by up to 2^-9 |v_j - o| per key, more
    # than in the spread-out rows the generic allowance was set for (on this data, rounding P
    # to bf16 alone, emulated in float64, already gives 6.1e-3); fp16 keeps the generic one
    allow = 8e-3 if (fmt == "bf16" and pattern == "spikes") else ALLOW_ATTN16[fmt]
    assert err16(host(o), ref, fmt) <= allow


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


@pytest.mark.parametrize("fmt,causal", [("f16", True), ("bf16", True), ("f16", False)])
@pytest.mark.parametrize("s", [77, 333])
def test_attention_ignores_rows_past_the_sequence(fmt, causal, s):
    """K and V are views of the first S rows of buffers whose next 64 rows hold NaN: a last,
    partial key tile must not let them reach the output (masked keys get probability 0, and
    0 * NaN would still poison it)."""
    nh, nkv, hd = 8, 2, 128
    q = dev(_normal(90 + s, (s, nh, hd)) * 2.0, fmt)
    kf = torch.full((s + 64, nkv, hd), float("nan"), device="cuda").to(q.dtype)
    vf = torch.full((s + 64, nkv, hd), float("nan"), device="cuda").to(q.dtype)
    kf[:s] = dev(_normal(91 + s, (s, nkv, hd)) * 2.0, fmt)
    vf[:s] = dev(_normal(92 + s, (s, nkv, hd)), fmt)
    k, v = kf[:s], vf[:s]
    fn = q3.gqa_causal_attention if causal else q3.gqa_bidirectional_attention
    o = fn(q, k, v)
    torch.cuda.synchronize()
    got = host(o)
    assert np.all(np.isfinite(got))
    ref = (oracle.causal_gqa_attention if causal else oracle.bidirectional_attention)(host(q), host(k), host(v))
    assert err16(got, ref, fmt) <= ALLOW_ATTN16[fmt]


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


def test_swiglu_ffn_activations_beyond_fp16_range():
    """SwiGLU activations above fp16's largest value (65504) stay finite with fp16 operands: the
    activation is stored as 2^-4 * a and the down product scales back by 2^4, both exact. The
    normalized input is scaled by 200 (gate and up outputs with standard deviation ~130), so the
    largest activation of this data is over twice 65504; the oracle confirms that."""
    s, h, f = 300, 1024, 768
    x = (_normal(90, (s, h), dtype="f32") * 200).astype(np.float16).astype(np.float32)
    wg = _normal(91, (f, h), std=0.02)
    wu = _normal(92, (f, h), std=0.02)
    wd = _normal(93, (h, f), std=0.02)
    r = _normal(94, (s, h), dtype="f32")
    a = oracle.silu(oracle.linear(x, wg)) * oracle.linear(x, wu)
    assert 65504 * 2 < np.abs(a).max() < 65504 * 16, np.abs(a).max()
    ref = oracle.swiglu_ffn(x, wg, wu, wd) + r
    for xdt in ("f16", "bf16"):
        xx = x if xdt == "f16" else synth.round_to_bf16(x)
        refx = ref if xdt == "f16" else oracle.swiglu_ffn(xx, wg, wu, wd) + r
        out = host(q3.swiglu_ffn(dev(xx, xdt), dev(wg, "bf16"), dev(wu, "bf16"), dev(wd, "bf16"),
                                 residual=dev(r)))
        assert np.isfinite(out).all(), xdt
        err = rel_err(out, refx)
        log_err(f"swiglu_ffn_large_act[{xdt}]", err)
        assert err <= TOL["bf16"], (xdt, err)


def test_layer_activations_beyond_fp16_range():
    """The layer's own gate/up and down products with SwiGLU activations above 65504: the FFN
    norm weights are scaled by 150 (bf16 values), so the normalized rows reach a few hundred and
    the activation several times 65504 (checked on the oracle's intermediate)."""
    cfg = synth.get_config("qwen3vl_2b_text").with_seq(257, n_layers=1)
    w = synth.make_layer_weights(cfg)
    w["ffn_norm"] = synth.round_to_bf16(np.asarray(w["ffn_norm"], dtype=np.float32) * 150)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    taps = {}
    ref = oracle.layer_prefill(x, w, cfg, pos, taps=taps)
    assert 65504 * 2 < np.abs(taps["a"]).max() < 65504 * 16, np.abs(taps["a"]).max()
    for act in ("f16", "bf16"):
        out = _run_layer(cfg, w, x, pos, act=act)
        assert np.isfinite(out).all(), act
        err = rel_err(out, ref)
        log_err(f"layer_large_act[act={act}]", err)
        assert err <= TOL["bf16"], (act, err)


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
                           ds_rows,
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
    ds = dev(ds, "bf16")
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


def test_deepstack_rows_checked_before_launch():
    """The DeepStack row list is host data checked before anything is enqueued: a row at or
    past S or a non-increasing list raises and leaves the output untouched; a valid sparse
    list adds exactly its slab rows (hf2q forward.rs, forward_text_prefill_logits_last)."""
    cfg = synth.get_config("qwen3vl_2b_text").with_seq(64)
    w = synth.make_layer_weights(cfg)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    spec = q3.LayerSpec.of(cfg)
    dw = dev_weights(w, "bf16")
    ds = _normal(70, (3, cfg.hidden), dtype="bf16")
    dds = dev(ds, "bf16")
    for bad in ([3, 70, 20], [3, 3, 10], [10, 9, 12], [-1, 5, 6]):
        out = torch.full((cfg.seq_len, cfg.hidden), 7.0, device="cuda")
        with pytest.raises(RuntimeError):
            q3.layer_prefill(spec, dw, dev(x), dev_i32(pos), bad, dds, out=out)
        torch.cuda.synchronize()
        assert bool(torch.all(out == 7.0)), bad
    with pytest.raises(TypeError):
        q3.layer_prefill(spec, dw, dev(x), dev_i32(pos), dev_i32([3, 10, 63]), dds)
    base = _run_layer(cfg, w, x, pos)
    y = _run_layer(cfg, w, x, pos, np.array([3, 10, 63], np.int32), ds)
    ref = base.astype(np.float64).copy()
    ref[[3, 10, 63]] += ds
    assert np.allclose(y, ref, rtol=0, atol=1e-6)


# ------------------------------------------------------------------ full-size workloads

def _as_f16(w):
    """The layer's bf16 weight values stored as fp16 (round to nearest even; exact for every
    magnitude in [2^-17, 65504]), as float32 arrays holding those values."""
    return {n: a.astype(np.float16).astype(np.float32) for n, a in w.items()}


def _spec16(cfg):
    spec = q3.LayerSpec.of(cfg)
    return q3.LayerSpec(**{**spec.__dict__, "dtype": "f16"})


def test_8b_stack_every_row_every_layer():
    """The 4-layer 8B-shaped stack at S=4096, run as the bench runs it (weights stored as fp16,
    one workspace, layer outputs chained in place on the GPU): every output row of every layer
    against the oracle's stack run from the same input on the same weight values, the error
    logged per layer."""
    cfg = synth.get_config("qwen3vl_8b_stack4")
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    spec = _spec16(cfg)
    ws = torch.empty(q3.layer_workspace_bytes(spec, cfg.seq_len), dtype=torch.uint8, device="cuda")
    dpos = dev_i32(pos)
    h = dev(x)
    ref = x.astype(np.float64)
    errs = []
    for li in range(cfg.n_layers):
        w = _as_f16(synth.make_layer_weights(cfg, li))
        h = q3.layer_prefill(spec, dev_weights(w, "f16"), h, dpos, workspace=ws, out=h)
        torch.cuda.synchronize()
        ref = oracle.layer_prefill(ref, w, cfg, pos)
        err = rel_err(host(h), ref)
        errs.append(err)
        print(f"8B stack layer {li + 1}: max|err|/rms over all {cfg.seq_len} rows = {err:.3e}", flush=True)
        log_err(f"8b_stack4[layer {li + 1}, all rows, fp16-stored weights]", err)
    assert max(errs) <= TOL["bf16"], errs


def test_8b_layer_every_row_bf16_weights():
    """Layer 1 of the 8B-shaped stack at S=4096 with the bf16 weights as given (each weight tile
    converted to fp16 inside the GEMM loop): every output row against the oracle."""
    cfg = synth.get_config("qwen3vl_8b_stack4").with_seq(4096, n_layers=1)
    w = synth.make_layer_weights(cfg, 0)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    err = rel_err(_run_layer(cfg, w, x, pos), oracle.layer_prefill(x, w, cfg, pos))
    print(f"8B layer, bf16 weights, all rows: max|err|/rms = {err:.3e}")
    log_err("8b_layer1[all rows, bf16 weights]", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", ["qwen3vl_2b_text", "qwen3vl_2b_image"])
def test_layer_fp16_stored_weights(name):
    """The 2B workloads with their weights stored as fp16 (the products then read operand-format
    weights, no conversion in the loop) against the oracle on the same values."""
    cfg = synth.get_config(name)
    w = _as_f16(synth.make_layer_weights(cfg))
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    rows, ds = synth.make_deepstack(cfg)
    if ds is not None:
        ds = ds.astype(np.float16).astype(np.float32)
    out = q3.layer_prefill(_spec16(cfg), dev_weights(w, "f16"), dev(x), dev_i32(pos), rows,
                           None if ds is None else dev(ds, "f16"))
    torch.cuda.synchronize()
    err = rel_err(host(out), oracle.layer_prefill(x, w, cfg, pos, rows, ds))
    log_err(f"layer[{name}, fp16-stored weights]", err)
    assert err <= TOL["bf16"]


def test_32b_encoder_every_row():
    """The 32B-encoder-shaped layer at S=8192 (64/8 heads, q_dim 8192 != hidden 5120): every
    output row against the oracle."""
    cfg = synth.get_config("qwen3_32b_encoder")
    w = synth.make_layer_weights(cfg)
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    y = _run_layer(cfg, w, x, pos)
    ref = oracle.layer_prefill(x, w, cfg, pos)
    err = rel_err(y, ref)
    # also per 1024-row band, so a failure names where it is
    bands = [rel_err(y[i:i + 1024], ref[i:i + 1024]) for i in range(0, cfg.seq_len, 1024)]
    print(f"32B encoder, all {cfg.seq_len} rows: max|err|/rms = {err:.3e}; per 1024-row band "
          + " ".join(f"{b:.2e}" for b in bands))
    log_err("32b_encoder[all rows]", err)
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
