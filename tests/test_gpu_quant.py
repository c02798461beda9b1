"""GPU parity of the weight-only quantized projections (Q4_0 blocks, int8 rows with a row scale)
against the float64 oracle: the expansion to 16 bits, the layer prefill with quantized weights
(with and without the KV cache), and decode steps that read the quantized bytes directly."""

import numpy as np
import pytest

import oracle
import synth
from util import TOL, dev, dev_i32, host, log_err, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _dev_raw(a):
    """Host array of any integer/byte dtype -> GPU tensor with the same bytes."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def _dev_layer(cfg, norms, proj):
    dn = {n: dev(a, cfg.dtype) for n, a in norms.items()}
    dp = {}
    for n, (f, d, rs) in proj.items():
        data = dev(d, cfg.dtype) if f == "dense" else _dev_raw(d)
        dp[n] = (f, data, None if rs is None else dev(rs))
    return dn, dp


def _oracle_weights(cfg, norms, proj):
    w = dict(norms)
    for n, (f, d, rs) in proj.items():
        rows = d.shape[0]
        cols = d.shape[1] * 32 if f == "q4_0" else d.shape[1]
        w[n] = oracle.dequant(f, d, rows, cols, rs)
    return w


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_dequantize_q4_0_is_the_rounded_oracle(out):
    rows, cols = 96, 512
    blocks = synth.gen.make_q4_0_weight(0, "t.q4", rows, cols)
    got = q3.dequantize_matrix("q4_0", _dev_raw(blocks), rows, cols, out_dtype=TDT[out])
    torch.cuda.synchronize()
    # d * (code - 8) is exact in fp32, so one rounding of the exact value
    want = torch.from_numpy(oracle.dequant_q4_0(blocks, rows, cols).astype(np.float32)).to(TDT[out])
    assert torch.equal(got.cpu(), want)


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_dequantize_q8_row_is_the_rounded_oracle(out):
    rows, cols = 80, 256
    q, rs = synth.gen.make_q8_row_weight(0, "t.q8", rows, cols)
    got = q3.dequantize_matrix("q8_row", _dev_raw(q), rows, cols, row_scale=dev(rs), out_dtype=TDT[out])
    torch.cuda.synchronize()
    # the product row_scale * q is formed in fp32, then rounded to the 16-bit format
    prod32 = (rs[:, None].astype(np.float32) * q.astype(np.float32)).astype(np.float32)
    assert np.array_equal(prod32.astype(np.float64), oracle.dequant_q8_row(q, rs).astype(np.float32))
    want = torch.from_numpy(prod32).to(TDT[out])
    assert torch.equal(got.cpu(), want)


MIXED = {"wq": "q4_0", "wk": "q8_row", "wv": "q4_0", "wo": "dense", "w_gate": "q8_row", "w_up": "q8_row",
         "w_down": "q4_0"}


@pytest.mark.parametrize("name,s,formats,act", [
    ("qwen3vl_2b_text", 300, None, ""),
    ("qwen3vl_2b_text", 257, MIXED, ""),
    ("qwen3vl_2b_image", 2048, None, ""),
    ("qwen3vl_2b_text", 130, {n: "q8_row" for n in synth.PROJ_NAMES}, "bf16"),
])
def test_layer_prefill_quant_matches_oracle(name, s, formats, act):
    cfg = synth.get_config(name)
    norms, proj = synth.make_quant_layer_weights(cfg, 0, formats)
    x, pos = synth.make_x(cfg)[:s], synth.make_positions(cfg)[:, :s]
    rows, slab = synth.make_deepstack(cfg)
    if rows is not None:
        keep = rows < s
        rows, slab = rows[keep], slab[keep]
    spec = q3.LayerSpec.of(cfg, act)
    dn, dp = _dev_layer(cfg, norms, proj)
    args = (rows, dev(slab, cfg.dtype)) if rows is not None else (None, None)
    got = host(q3.layer_prefill_quant(spec, dn, dp, dev(x), dev_i32(pos), *args))
    ref = oracle.layer_prefill(x, _oracle_weights(cfg, norms, proj), cfg, pos, rows, slab)
    err = rel_err(got, ref)
    log_err(f"layer_prefill_quant[{name},S{s},{'mixed' if formats else 'q4_0'},{act or 'f16'}]", err)
    print(f"{name} S{s}: max|err|/rms = {err:.3e}")
    assert err <= TOL[cfg.dtype]


def test_quant_prefill_with_cache_then_quant_decode():
    cfg = synth.get_config("qwen3vl_2b_text")
    s0, steps = 200, 3
    full = s0 + steps
    norms, proj = synth.make_quant_layer_weights(cfg, 0, MIXED)
    x, pos = synth.make_x(cfg)[:full], synth.make_positions(cfg)[:, :full]
    spec = q3.LayerSpec.of(cfg)
    dn, dp = _dev_layer(cfg, norms, proj)
    kc, vc = q3.kv_cache_alloc(spec, full + 1)
    y0 = q3.layer_prefill_quant(spec, dn, dp, dev(x[:s0]), dev_i32(pos[:, :s0]), k_cache=kc, v_cache=vc)
    y1 = q3.layer_prefill_quant(spec, dn, dp, dev(x[:s0]), dev_i32(pos[:, :s0]))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    outs = []
    for t in range(s0, full):
        outs.append(host(q3.layer_decode_quant(spec, dn, dp, dev(x[t]), dev_i32(pos[:, t]), kc, vc, t)))
    w = _oracle_weights(cfg, norms, proj)
    ref = oracle.layer_prefill_rows(x, w, cfg, pos, np.arange(s0, full))
    err = rel_err(np.stack(outs), ref)
    log_err("layer_decode_quant[2b_text,mixed,S0=200,+3]", err)
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_row"])
def test_quant_decode_from_empty_cache_is_the_one_token_prefill(fmt):
    cfg = synth.get_config("qwen3vl_2b_text")
    norms, proj = synth.make_quant_layer_weights(cfg, 0, {n: fmt for n in synth.PROJ_NAMES})
    x, pos = synth.make_x(cfg)[:1], synth.make_positions(cfg)[:, :1]
    spec = q3.LayerSpec.of(cfg)
    dn, dp = _dev_layer(cfg, norms, proj)
    kc, vc = q3.kv_cache_alloc(spec, 4)
    got = host(q3.layer_decode_quant(spec, dn, dp, dev(x[0]), dev_i32(pos[:, 0]), kc, vc, 0))
    ref = oracle.layer_prefill(x, _oracle_weights(cfg, norms, proj), cfg, pos)[0]
    # the decode step keeps its vectors in fp32: only the cache row is 16-bit
    assert rel_err(got, ref) <= 1e-3


def test_quant_8b_prefill_4096_then_decode():
    """The 8B layer shape at full size with Q4_0 projections: prefill 4096 tokens with the cache
    (sampled output rows) and decode token 4096."""
    cfg = synth.get_config("qwen3vl_8b_stack4").with_seq(4097)
    norms, proj = synth.make_quant_layer_weights(cfg, 0)
    x, pos = synth.make_x(cfg), synth.make_positions(cfg)
    s0 = 4096
    spec = q3.LayerSpec.of(cfg)
    dn, dp = _dev_layer(cfg, norms, proj)
    kc, vc = q3.kv_cache_alloc(spec, 4100)
    y = host(q3.layer_prefill_quant(spec, dn, dp, dev(x[:s0]), dev_i32(pos[:, :s0]), k_cache=kc, v_cache=vc))
    yd = host(q3.layer_decode_quant(spec, dn, dp, dev(x[s0]), dev_i32(pos[:, s0]), kc, vc, s0))
    w = _oracle_weights(cfg, norms, proj)
    rows = np.array([0, 1, 777, 2048, 4095])
    ref = oracle.layer_prefill_rows(x[:s0], w, cfg, pos[:, :s0], rows)
    err = rel_err(y[rows], ref)
    ref_d = oracle.layer_prefill_rows(x, w, cfg, pos, np.array([s0]))[0]
    err_d = rel_err(yd, ref_d)
    log_err("layer_prefill_quant[8b,S4096,q4_0] sampled rows", err)
    log_err("layer_decode_quant[8b,S0=4096,q4_0]", err_d)
    print(f"8B Q4_0: prefill rows {err:.3e}, decode {err_d:.3e}")
    assert err <= TOL[cfg.dtype] and err_d <= TOL[cfg.dtype]


@pytest.mark.parametrize("act,s", [("f16", 300), ("bf16", 300), ("f16", 1030)])
def test_q4_0_decoded_in_product_equals_expanded_product(act, s):
    """A layer whose projections are all Q4_0 decodes the blocks inside the matrix products'
    weight-tile path. Each weight is the same one rounding of d * (code - 8) that the expansion
    kernel stores, placed in the same tile layout, so the layer's output equals, bit for bit,
    the dense layer run on the expanded matrices."""
    cfg = synth.get_config("qwen3vl_2b_text").with_seq(s)
    formats = {n: "q4_0" for n in synth.PROJ_NAMES}
    norms, proj = synth.make_quant_layer_weights(cfg, 0, formats)
    x, pos = synth.make_x(cfg), synth.make_positions(cfg)
    spec = q3.LayerSpec.of(cfg, act)
    dn, dp = _dev_layer(cfg, norms, proj)
    yq = q3.layer_prefill_quant(spec, dn, dp, dev(x), dev_i32(pos))
    dense = {n: q3.dequantize_matrix("q4_0", dp[n][1], d.shape[0], d.shape[1] * 32, out_dtype=TDT[act])
             for n, (_, d, _) in proj.items()}
    dense.update({n: t.to(TDT[act]) for n, t in dn.items()})
    spec_d = q3.LayerSpec(**{**spec.__dict__, "dtype": act})
    yd = q3.layer_prefill(spec_d, dense, dev(x), dev_i32(pos))
    torch.cuda.synchronize()
    assert torch.equal(yq, yd)
    # against the oracle on the weights the products multiply (each rounded once to `act`)
    w_used = dict(norms)
    w_used.update({n: host(t) for n, t in dense.items() if n in proj})
    err = rel_err(host(yq), oracle.layer_prefill(x, w_used, cfg, pos))
    log_err(f"layer_q4_0_in_product[{act},S{s}]", err)
    # fp16 operands: the layer bound. bf16 operands carry 8-bit significands through every
    # product and sit at that bound on these weights (2.0e-2 measured); their pin here is the
    # equality with the expanded product above, whose own numerics the other tests bound.
    if act == "f16":
        assert err <= TOL["bf16"]
