"""GPU parity of the whole-model text prefill (qwen3_model_prefill_logits_last) against the
float64 oracle: embedding lookup, the layer chain with per-layer DeepStack, final RMSNorm and
the tied or untied LM head on the last position."""

import numpy as np
import pytest

import oracle
import synth
from util import TOL, dev, dev_i32, dev_weights, host, log_err, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402


def _model(cfg, n_layers, vocab, n_ds_layers=0, tied=False, seq_len=None):
    if seq_len is not None:
        cfg = cfg.with_seq(seq_len)
    layers = [synth.make_layer_weights(cfg, li) for li in range(n_layers)]
    emb, norm, head = synth.make_model_weights(cfg, vocab, tied)
    tokens = synth.make_tokens(cfg, vocab)
    pos = synth.make_positions(cfg)
    ds_rows, slabs = synth.make_deepstack_layers(cfg, n_ds_layers) if n_ds_layers else (None, None)
    return cfg, layers, emb, norm, head, tokens, pos, ds_rows, slabs


def _run(cfg, layers, emb, norm, head, tokens, pos, ds_rows, slabs, act=""):
    d = cfg.dtype
    spec = q3.LayerSpec.of(cfg, act)
    out = q3.model_prefill_logits_last(
        spec, [dev_weights(w, d) for w in layers], dev(emb, d), dev(norm, d),
        None if head is None else dev(head, d), tokens.tolist(), dev_i32(pos),
        ds_rows,
        None if slabs is None else [dev(s, d) for s in slabs])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,n_layers,vocab,n_ds,tied", [
    ("tiny_f32", 2, 1000, 0, False),
    ("tiny_f32", 3, 257, 0, True),
    ("qwen3vl_2b_image", 2, 32768, 2, False),
])
def test_model_logits_match_oracle(name, n_layers, vocab, n_ds, tied):
    cfg, layers, emb, norm, head, tokens, pos, ds_rows, slabs = _model(synth.get_config(name), n_layers,
                                                                       vocab, n_ds, tied)
    ref = oracle.model_prefill_logits_last(tokens, emb, layers, norm, head, cfg, pos, ds_rows, slabs)
    got = host(_run(cfg, layers, emb, norm, head, tokens, pos, ds_rows, slabs))
    err = rel_err(got, ref)
    log_err(f"model[{name},L{n_layers},V{vocab},ds{n_ds},tied={tied}]", err)
    print(f"{name} L{n_layers} V{vocab}: max|err|/rms = {err:.3e}")
    assert err <= TOL[cfg.dtype]


def test_model_tied_head_equals_passing_the_table_and_no_layers():
    cfg, layers, emb, norm, _, tokens, pos, _, _ = _model(synth.get_config("qwen3vl_2b_text"), 1, 4096,
                                                          seq_len=97)
    a = _run(cfg, layers, emb, norm, None, tokens, pos, None, None)
    b = _run(cfg, layers, emb, norm, emb, tokens, pos, None, None)
    assert torch.equal(a, b)
    # no layers, one token: the head applied to the normalized embedding row
    one = tokens[:1]
    got = host(_run(cfg.with_seq(1), [], emb, norm, None, one, pos[:, :1], None, None))
    ref = oracle.model_prefill_logits_last(one, emb, [], norm, None, cfg, pos[:, :1])
    assert rel_err(got, ref) <= 1e-5


@pytest.mark.parametrize("name,n_layers,vocab,s0,steps,tied", [
    ("tiny_f32", 2, 300, 20, 5, False),
    ("qwen3vl_2b_text", 2, 4096, 64, 2, True),
    ("qwen3vl_2b_image", 2, 2048, 1200, 2, False),   # the prompt holds the image span
])
def test_model_decode_continues_the_prefill(name, n_layers, vocab, s0, steps, tied):
    """Whole-model prefill with every layer's cache, then decode steps: the logits of each new
    token equal the oracle's last-position logits of the prefill over the longer sequence."""
    cfg, layers, emb, norm, head, tokens, pos, _, _ = _model(synth.get_config(name), n_layers, vocab, tied=tied)
    d = cfg.dtype
    spec = q3.LayerSpec.of(cfg)
    dl = [dev_weights(w, d) for w in layers]
    de, dn, dh = dev(emb, d), dev(norm, d), None if head is None else dev(head, d)
    caches = [q3.kv_cache_alloc(spec, s0 + steps) for _ in range(n_layers)]
    first = q3.model_prefill_logits_last(spec, dl, de, dn, dh, tokens[:s0].tolist(), dev_i32(pos[:, :s0]),
                                         caches=caches)
    plain = q3.model_prefill_logits_last(spec, dl, de, dn, dh, tokens[:s0].tolist(), dev_i32(pos[:, :s0]))
    torch.cuda.synchronize()
    assert torch.equal(first, plain)
    for t in range(s0, s0 + steps):
        got = host(q3.model_decode_logits(spec, dl, de, dn, dh, int(tokens[t]), dev_i32(pos[:, t]), caches, t))
        ref = oracle.model_prefill_logits_last(tokens[:t + 1], emb, layers, norm, head, cfg, pos[:, :t + 1])
        err = rel_err(got, ref)
        log_err(f"model_decode[{name},L{n_layers},V{vocab},t={t}]", err)
        assert err <= TOL[cfg.dtype], (t, err)
