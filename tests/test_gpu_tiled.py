"""Tiled fp16 weights (wdtype QWEN3_F16_TILED): the layout qwen3_tile_weights writes, checked
element by element against its index formula, and every entry point that takes tiled weights
computing the same bits as with the same fp16 values stored row-major (the products read the
same operand values in the same order; only their addresses differ). The row-major fp16 path
itself is checked against the oracle in the other GPU tests; the 8B-shaped stack with tiled
weights is also compared with the oracle here on every row."""

import numpy as np
import pytest

import oracle
import synth
from util import TOL, dev, dev_i32, dev_weights, host, log_err, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402


def _tiled_positions(rows, cols):
    """Flat index of every element (r, c) of a [rows, cols] matrix in the tiled layout:
    ((r // 16) * (cols // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32."""
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    return ((r // 16) * (cols // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32


@pytest.mark.parametrize("src,rows,cols", [("bf16", 16, 32), ("bf16", 48, 96), ("f16", 64, 2048),
                                           ("f32", 112, 160), ("bf16", 1024, 4096)])
def test_tile_weights_layout(src, rows, cols):
    a = np.random.default_rng(rows + cols).standard_normal((rows, cols)).astype(np.float32) * 0.05
    if src == "bf16":
        a = synth.round_to_bf16(a)
    elif src == "f16":
        a = a.astype(np.float16).astype(np.float32)
    t = q3.tile_weights(dev(a, src))
    torch.cuda.synchronize()
    got = t.cpu().numpy().reshape(-1)
    want = np.empty(rows * cols, np.float16)
    want[_tiled_positions(rows, cols).reshape(-1)] = a.astype(np.float16).reshape(-1)  # RNE
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def _spec(cfg, dtype):
    spec = q3.LayerSpec.of(cfg)
    return q3.LayerSpec(**{**spec.__dict__, "dtype": dtype})


def _f16(w):
    return {n: a.astype(np.float16).astype(np.float32) for n, a in w.items()}


def _both(w):
    """(plain fp16 device weights, the same values prepared for "f16t")."""
    plain = dev_weights(_f16(w), "f16")
    return plain, q3.tile_layer_weights(plain)


@pytest.mark.parametrize("name,s", [("qwen3vl_2b_text", 333), ("qwen3vl_2b_image", None),
                                    ("qwen3vl_8b_stack4", 130), ("qwen3_32b_encoder", 65)])
def test_layer_tiled_weights_equal_plain(name, s):
    cfg = synth.get_config(name)
    if s is not None:
        cfg = cfg.with_seq(s, n_layers=1)
    plain, tiled = _both(synth.make_layer_weights(cfg))
    x, pos = dev(synth.make_x(cfg)), dev_i32(synth.make_positions(cfg))
    rows, ds = synth.make_deepstack(cfg)
    dsd = None if ds is None else dev(ds.astype(np.float16).astype(np.float32), "f16")
    a = q3.layer_prefill(_spec(cfg, "f16"), plain, x, pos, rows, dsd)
    b = q3.layer_prefill(_spec(cfg, "f16t"), tiled, x, pos, rows, dsd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_layer_kv_and_decode_tiled_weights_equal_plain():
    cfg = synth.get_config("qwen3vl_2b_text").with_seq(200, n_layers=1)
    plain, tiled = _both(synth.make_layer_weights(cfg))
    x, pos = synth.make_x(cfg), synth.make_positions(cfg)
    s0 = 150
    outs = []
    for spec, w in ((_spec(cfg, "f16"), plain), (_spec(cfg, "f16t"), tiled)):
        kc, vc = q3.kv_cache_alloc(spec, 200)
        y = q3.layer_prefill_kv(spec, w, dev(x[:s0]), dev_i32(pos[:, :s0]), kc, vc)
        steps = [q3.layer_decode(spec, w, dev(x[t]), dev_i32(pos[:, t]), kc, vc, t) for t in range(s0, s0 + 3)]
        torch.cuda.synchronize()
        outs.append((y, steps, kc, vc))
    (ya, da, ka, va), (yb, db, kb, vb) = outs
    assert torch.equal(ya, yb) and torch.equal(ka, kb) and torch.equal(va, vb)
    for p, q in zip(da, db):
        assert torch.equal(p, q)


@pytest.mark.parametrize("s,h,f,resid", [(300, 1024, 2048, True), (77, 2048, 6144, False)])
def test_swiglu_ffn_tiled_weights_equal_plain(s, h, f, resid):
    g = np.random.default_rng(s)
    x = dev(g.standard_normal((s, h)).astype(np.float32), "f16")
    ws = [dev(g.standard_normal(shape).astype(np.float32) * 0.02, "f16") for shape in ((f, h), (f, h), (h, f))]
    r = dev(g.standard_normal((s, h)).astype(np.float32)) if resid else None
    a = q3.swiglu_ffn(x, *ws, residual=r)
    b = q3.swiglu_ffn(x, *[q3.tile_weights(w) for w in ws], residual=r, weights_tiled=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_model_tiled_layers_equal_plain():
    cfg = synth.get_config("qwen3vl_2b_image")
    vocab = 4096
    layers = [_f16(synth.make_layer_weights(cfg, li)) for li in range(2)]
    emb, norm, head = (a.astype(np.float16).astype(np.float32) for a in synth.make_model_weights(cfg, vocab))
    tokens = synth.make_tokens(cfg, vocab).tolist()
    pos = dev_i32(synth.make_positions(cfg))
    rows, slabs = synth.make_deepstack_layers(cfg, 2)
    slabs = [dev(sl.astype(np.float16).astype(np.float32), "f16") for sl in slabs]
    de, dn, dh = dev(emb, "f16"), dev(norm, "f16"), dev(head, "f16")
    plain = [dev_weights(w, "f16") for w in layers]
    tiled = [q3.tile_layer_weights(w) for w in plain]
    a = q3.model_prefill_logits_last(_spec(cfg, "f16"), plain, de, dn, dh, tokens, pos, rows, slabs)
    b = q3.model_prefill_logits_last(_spec(cfg, "f16t"), tiled, de, dn, dh, tokens, pos, rows, slabs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_quant_layer_with_tiled_dense_groups_equals_plain():
    """Quantized layer whose dense groups (wo; gate/up) take tiled fp16 matrices."""
    cfg = synth.get_config("qwen3vl_2b_text").with_seq(257, n_layers=1)
    formats = {"wq": "q4_0", "wk": "q4_0", "wv": "q4_0", "wo": "dense", "w_gate": "dense", "w_up": "dense",
               "w_down": "q8_row"}
    norms, proj = synth.make_quant_layer_weights(cfg, 0, formats)
    dn = {n: dev(a.astype(np.float16).astype(np.float32), "f16") for n, a in norms.items()}

    def dev_proj(tiled):
        out = {}
        for n, (fmt, d, rs) in proj.items():
            if fmt == "dense":
                t = dev(d.astype(np.float16).astype(np.float32), "f16")
                out[n] = (fmt, q3.tile_weights(t) if tiled else t, None)
            else:
                out[n] = (fmt, torch.from_numpy(np.ascontiguousarray(d)).cuda(),
                          None if rs is None else dev(rs))
        return out

    x, pos = dev(synth.make_x(cfg)), dev_i32(synth.make_positions(cfg))
    a = q3.layer_prefill_quant(_spec(cfg, "f16"), dn, dev_proj(False), x, pos)
    b = q3.layer_prefill_quant(_spec(cfg, "f16t"), dn, dev_proj(True), x, pos)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_8b_stack_tiled_weights_every_row():
    """The 4-layer 8B-shaped stack at S=4096 as the benchmark runs it (weights tiled once, one
    workspace, layers chained in place): every output row of every layer against the oracle."""
    cfg = synth.get_config("qwen3vl_8b_stack4")
    x = synth.make_x(cfg)
    pos = synth.make_positions(cfg)
    spec = _spec(cfg, "f16t")
    ws = torch.empty(q3.layer_workspace_bytes(spec, cfg.seq_len), dtype=torch.uint8, device="cuda")
    dpos = dev_i32(pos)
    h = dev(x)
    ref = x.astype(np.float64)
    errs = []
    for li in range(cfg.n_layers):
        w = _f16(synth.make_layer_weights(cfg, li))
        h = q3.layer_prefill(spec, q3.tile_layer_weights(dev_weights(w, "f16")), h, dpos, workspace=ws, out=h)
        torch.cuda.synchronize()
        ref = oracle.layer_prefill(ref, w, cfg, pos)
        err = rel_err(host(h), ref)
        errs.append(err)
        print(f"8B stack (tiled weights) layer {li + 1}: max|err|/rms over all rows = {err:.3e}", flush=True)
        log_err(f"8b_stack4[layer {li + 1}, all rows, tiled fp16 weights]", err)
    assert max(errs) <= TOL["bf16"], errs
