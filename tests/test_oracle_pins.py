"""Pins of the float64 oracle against what the pages and mathematics fix.

Each check is chosen so a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand, the norm after instead of before
the rotation, a wrong axis rule or position rule) fails at least one of them.
"""

import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.special

import brute
import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    vals = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                vals.extend(int(t) for t in line.split())
    return np.array(vals)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    for c in (0.5, 3.0, -2.0):
        x = np.full(8, c)
        y = oracle.rms_norm(x, np.ones(8), 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=0, atol=1e-15)


def test_rmsnorm_three_four():
    y = oracle.rms_norm(np.array([3.0, 4.0]), np.ones(2), 1e-6)
    ref = np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-6)
    assert np.allclose(y, ref, rtol=1e-15, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    x = _rng().standard_normal((5, 16))
    y1 = oracle.rms_norm(x, np.ones(16), 0.0)
    y2 = oracle.rms_norm(7.5 * x, np.ones(16), 0.0)
    assert np.allclose(y1, y2, rtol=1e-13, atol=0)
    assert np.allclose(np.mean(y1 * y1, axis=1), 1.0, rtol=1e-13)


def test_rmsnorm_weight_is_plain_and_applied_after():
    x = _rng(1).standard_normal((3, 16))
    g = 1.0 + 0.1 * _rng(2).standard_normal(16)
    y = oracle.rms_norm(x, g, 1e-6)
    for s in range(3):
        assert np.allclose(y[s], brute.rmsnorm_row(list(x[s]), list(g), 1e-6), rtol=1e-13)
    # plain w: a zero weight gives zero, not the normalized row (which 1+w would)
    assert np.all(oracle.rms_norm(x, np.zeros(16), 1e-6) == 0)


# ---------------------------------------------------------------- linear, silu

def test_linear_matches_loops_and_layout():
    x = _rng(3).standard_normal((3, 5))
    w = _rng(4).standard_normal((7, 5))            # [out, in]
    y = oracle.linear(x, w)
    assert y.shape == (3, 7)
    assert np.allclose(y, brute.matvec_rows(x.tolist(), w.tolist()), rtol=1e-13, atol=1e-14)


def test_silu_closed_forms_and_library():
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(float(oracle.silu(1.0)), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    z = np.linspace(-30, 30, 121)
    assert np.allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- MRoPE

def test_inv_freq_closed_form():
    assert np.allclose(oracle.rope_inv_freq(4, 100.0), [1.0, 0.1], rtol=1e-15)
    f = oracle.rope_inv_freq(128, 5e6)
    assert f[0] == 1.0 and math.isclose(f[-1], 5e6 ** (-126 / 128), rel_tol=1e-14)


def test_mrope_axes_match_page_literal_rule():
    want = _golden_ints("mrope_axes_hd128_sections_24_20_20.txt")
    assert want.shape == (64,)
    assert np.array_equal(oracle.mrope_axes(128, (24, 20, 20)), want)


@pytest.mark.parametrize("hd,sec", [(128, (24, 20, 20)), (64, (12, 10, 10)), (128, (32, 16, 16))])
def test_mrope_axis_counts_equal_sections(hd, sec):
    ax = oracle.mrope_axes(hd, sec)
    assert [int(np.sum(ax == a)) for a in range(3)] == list(sec)


def _textbook_rope(x, positions, theta):
    """1-D RoPE in the rotate_half form: x*cos(emb) + rotate_half(x)*sin(emb), with
    emb = cat(freqs, freqs) and rotate_half(x) = cat(-x2, x1)."""
    hd = x.shape[-1]
    inv = 1.0 / theta ** (np.arange(0, hd, 2) / hd)
    freqs = np.outer(positions, inv)
    emb = np.concatenate([freqs, freqs], axis=-1)[:, None, :]
    x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
    rot = np.concatenate([-x2, x1], axis=-1)
    return x * np.cos(emb) + rot * np.sin(emb)


@pytest.mark.parametrize("hd,sec,theta", [(128, (24, 20, 20), 5e6), (64, (12, 10, 10), 1e6)])
def test_text_only_mrope_is_textbook_rope(hd, sec, theta):
    s, heads = 40, 3
    x = _rng(5).standard_normal((s, heads, hd))
    g = 1.0 + 0.1 * _rng(6).standard_normal(hd)
    pos = np.tile(np.arange(s) * 37 % 4096, (3, 1))
    y = oracle.qk_norm_mrope(x, g, 1e-6, pos, theta, sec)
    # norm (with its weight) first, then the rotation
    ref = _textbook_rope(oracle.rms_norm(x, g, 1e-6), pos[0], theta)
    assert np.allclose(y, ref, rtol=0, atol=1e-12)
    # complex-number form of the same rotation on pair (i, i + hd/2)
    z = (ref[..., : hd // 2] + 1j * ref[..., hd // 2:])
    zn = oracle.rms_norm(x, g, 1e-6)
    z0 = zn[..., : hd // 2] + 1j * zn[..., hd // 2:]
    ang = np.outer(pos[0], oracle.rope_inv_freq(hd, theta))[:, None, :]
    assert np.allclose(z, z0 * np.exp(1j * ang), atol=1e-12)


def test_mrope_position_zero_is_identity_and_pairs_keep_norm():
    hd = 128
    x = _rng(7).standard_normal((6, 2, hd))
    g = 1.0 + 0.1 * _rng(8).standard_normal(hd)
    y0 = oracle.qk_norm_mrope(x, g, 1e-6, np.zeros((3, 6), dtype=np.int64), 5e6, (24, 20, 20))
    assert np.array_equal(y0, oracle.rms_norm(x, g, 1e-6))
    pos = _rng(9).integers(0, 8192, (3, 6))
    y = oracle.qk_norm_mrope(x, g, 1e-6, pos, 5e6, (24, 20, 20))
    n = oracle.rms_norm(x, g, 1e-6)
    h = hd // 2
    assert np.allclose(y[..., :h] ** 2 + y[..., h:] ** 2, n[..., :h] ** 2 + n[..., h:] ** 2, rtol=1e-12)


def test_rope_scores_depend_on_offset_only():
    hd = 64
    q = _rng(10).standard_normal((1, 1, hd))
    k = _rng(11).standard_normal((1, 1, hd))
    one = np.ones(hd)

    def rot(x, p):
        return oracle.qk_norm_mrope(x, one, 0.0, np.full((3, 1), p), 1e4, (12, 10, 10))[0, 0]

    d1 = rot(q, 10) @ rot(k, 3)
    d2 = rot(q, 107) @ rot(k, 100)
    d3 = rot(q, 10) @ rot(k, 4)
    assert math.isclose(d1, d2, rel_tol=1e-10)
    assert not math.isclose(d1, d3, rel_tol=1e-6)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_perturbing_one_axis_changes_exactly_its_pairs(axis):
    hd, sec = 128, (24, 20, 20)
    x = _rng(12).standard_normal((4, 2, hd))
    g = np.ones(hd)
    pos = np.tile(np.arange(4) + 50, (3, 1))
    pos2 = pos.copy()
    pos2[axis] += 17
    y1 = oracle.qk_norm_mrope(x, g, 1e-6, pos, 5e6, sec)
    y2 = oracle.qk_norm_mrope(x, g, 1e-6, pos2, 5e6, sec)
    ax = oracle.mrope_axes(hd, sec)
    lanes = np.concatenate([ax, ax]) == axis
    assert np.all(np.abs(y1 - y2)[..., lanes].max(axis=(0, 1)) > 1e-9)
    assert np.array_equal(y1[..., ~lanes], y2[..., ~lanes])


def test_norm_rope_matches_brute_force():
    hd, sec = 64, (12, 10, 10)
    x = _rng(13).standard_normal((5, 2, hd))
    g = 1.0 + 0.1 * _rng(14).standard_normal(hd)
    pos = _rng(15).integers(0, 300, (3, 5))
    y = oracle.qk_norm_mrope(x, g, 1e-6, pos, 1e6, sec)
    axes = list(oracle.mrope_axes(hd, sec))
    for s in range(5):
        for h in range(2):
            n = brute.rmsnorm_row(list(x[s, h]), list(g), 1e-6)
            r = brute.rope_row(n, pos[0, s], pos[1, s], pos[2, s], 1e6, axes)
            assert np.allclose(y[s, h], r, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- positions

def test_positions_text_only_reduce_to_arange():
    p = oracle.mrope_positions(9, [])
    assert np.array_equal(p, np.tile(np.arange(9), (3, 1)))


def test_positions_small_worked_example():
    want = _golden_ints("mrope_positions_small.txt").reshape(-1, 3).T
    assert np.array_equal(oracle.mrope_positions(10, [(3, 2, 3)]), want)


def test_image_workload_positions_follow_the_rules():
    cfg = synth.get_config("qwen3vl_2b_image")
    gen = synth.make_positions(cfg)
    ref = oracle.mrope_positions(cfg.seq_len, [(cfg.span_start, cfg.span_h, cfg.span_w)])
    a, b = cfg.span_start, cfg.span_start + cfg.span_len
    # text before and after the span: identical, 3 equal axes; the text after resumes at 132
    assert np.array_equal(gen[:, :a], ref[:, :a]) and np.array_equal(gen[:, b:], ref[:, b:])
    assert gen[0, b] == 132 and np.all(gen[:, b:] == gen[0, b:])
    # the span: t pinned at 100; the same (t, h, w) set as the row-major rule, in
    # the workload's 2x2 block-major order
    assert np.all(gen[0, a:b] == 100)
    assert gen[1, a:b].min() == 100 and gen[1, a:b].max() == 131
    assert sorted(map(tuple, gen[:, a:b].T)) == sorted(map(tuple, ref[:, a:b].T))
    assert tuple(gen[:, a:a + 4].T.ravel()) == (100, 100, 100, 100, 100, 101,
                                                100, 101, 100, 100, 101, 101)
    # generation would resume one past the largest position on any axis
    assert ref[:, :b].max() + 1 == 132


# ---------------------------------------------------------------- attention

def _attn_inputs(s, nh, nkv, hd, seed=20):
    r = _rng(seed)
    return (r.standard_normal((s, nh, hd)), r.standard_normal((s, nkv, hd)),
            r.standard_normal((s, nkv, hd)))


def test_attention_matches_brute_force():
    s, nh, nkv, hd = 6, 4, 2, 8
    q, k, v = _attn_inputs(s, nh, nkv, hd)
    o = oracle.causal_gqa_attention(q, k, v)
    ref = brute.attention(q.reshape(s, -1).tolist(), k.reshape(s, -1).tolist(),
                          v.reshape(s, -1).tolist(), nh, nkv, hd)
    assert np.allclose(o.reshape(s, -1), ref, rtol=1e-12, atol=1e-13)


def test_attention_single_token_returns_v():
    q, k, v = _attn_inputs(1, 4, 2, 8)
    o = oracle.causal_gqa_attention(q, k, v)
    assert np.allclose(o[0], np.repeat(v[0], 2, axis=0), rtol=1e-15)


def test_attention_zero_query_is_running_mean():
    s = 9
    q, k, v = _attn_inputs(s, 4, 2, 8)
    o = oracle.causal_gqa_attention(np.zeros_like(q), k, v)
    mean = np.cumsum(v, axis=0) / np.arange(1, s + 1)[:, None, None]
    assert np.allclose(o, np.repeat(mean, 2, axis=1), rtol=1e-13)


def test_attention_two_keys_scale():
    hd = 16
    q = np.zeros((2, 1, hd)); q[1, 0, 0] = 3.0
    k = np.zeros((2, 1, hd)); k[0, 0, 0] = 1.0; k[1, 0, 0] = -1.0
    v = np.zeros((2, 1, hd)); v[0, 0, 1] = 1.0; v[1, 0, 1] = 2.0
    o = oracle.causal_gqa_attention(q, k, v)
    z = np.array([3.0, -3.0]) / 4.0                     # 1/sqrt(16)
    p = np.exp(z) / np.exp(z).sum()
    assert math.isclose(o[1, 0, 1], p[0] * 1 + p[1] * 2, rel_tol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _attn_inputs(11, 8, 2, 16)
    o = oracle.causal_gqa_attention(q, k, v)
    o2 = oracle.causal_gqa_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    assert np.allclose(o, o2, rtol=1e-14, atol=0)


def test_attention_causality_bitwise():
    q, k, v = _attn_inputs(12, 4, 2, 8)
    o = oracle.causal_gqa_attention(q, k, v)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[7:] += 5.0; v2[7:] -= 3.0; q2[7:] *= 2
    o2 = oracle.causal_gqa_attention(q2, k2, v2)
    assert np.array_equal(o[:7], o2[:7])
    assert not np.allclose(o[7:], o2[7:])


def test_attention_row_subset():
    q, k, v = _attn_inputs(10, 4, 2, 8)
    rows = np.array([0, 3, 9])
    o = oracle.causal_gqa_attention(q, k, v)
    o_sub = oracle.causal_gqa_attention(q[rows], k, v, rows)
    assert np.allclose(o[rows], o_sub, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- FFN and layer

def test_swiglu_matches_loops():
    r = _rng(30)
    yn, wg, wu, wd = r.standard_normal((3, 6)), r.standard_normal((5, 6)), r.standard_normal((5, 6)), r.standard_normal((6, 5))
    y = oracle.swiglu_ffn(yn, wg, wu, wd)
    g = brute.matvec_rows(yn.tolist(), wg.tolist())
    u = brute.matvec_rows(yn.tolist(), wu.tolist())
    a = [[gv / (1 + math.exp(-gv)) * uv for gv, uv in zip(gr, ur)] for gr, ur in zip(g, u)]
    assert np.allclose(y, brute.matvec_rows(a, wd.tolist()), rtol=1e-12, atol=1e-13)


def _tiny_cfg():
    return SimpleNamespace(n_heads=4, n_kv_heads=2, head_dim=8, eps=1e-6, theta=1e4,
                           sections=(2, 1, 1), hidden=12, ffn=10)


def _tiny_weights(cfg, seed=40):
    r = _rng(seed)
    h, hd, f = cfg.hidden, cfg.head_dim, cfg.ffn
    qd, kd = cfg.n_heads * hd, cfg.n_kv_heads * hd
    sh = {"attn_norm": (h,), "wq": (qd, h), "wk": (kd, h), "wv": (kd, h), "q_norm": (hd,),
          "k_norm": (hd,), "wo": (h, qd), "ffn_norm": (h,), "w_gate": (f, h), "w_up": (f, h),
          "w_down": (h, f)}
    return {n: (1 + 0.1 * r.standard_normal(s)) if n.endswith("norm") else 0.3 * r.standard_normal(s)
            for n, s in sh.items()}


def test_layer_matches_brute_force_with_image_positions_and_deepstack():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    s = 7
    x = _rng(41).standard_normal((s, cfg.hidden))
    pos = oracle.mrope_positions(s, [(2, 2, 2)])
    ds_rows = np.array([2, 3, 4, 5])
    ds = _rng(42).standard_normal((4, cfg.hidden))
    y = oracle.layer_prefill(x, w, cfg, pos, ds_rows, ds)
    wl = {n: a.tolist() for n, a in w.items()}
    axes = list(oracle.mrope_axes(cfg.head_dim, cfg.sections))
    ref = brute.layer(x.tolist(), wl, 4, 2, 8, 1e-6, 1e4, axes, pos.tolist(),
                      ds_rows.tolist(), ds.tolist())
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_zero_output_projections_give_identity_plus_deepstack():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    w["wo"] = np.zeros_like(w["wo"])
    w["w_down"] = np.zeros_like(w["w_down"])
    x = _rng(43).standard_normal((5, cfg.hidden))
    pos = oracle.mrope_positions(5, [])
    assert np.array_equal(oracle.layer_prefill(x, w, cfg, pos), x)
    ds = _rng(44).standard_normal((2, cfg.hidden))
    y = oracle.layer_prefill(x, w, cfg, pos, np.array([1, 3]), ds)
    ref = x.copy(); ref[1] += ds[0]; ref[3] += ds[1]
    assert np.array_equal(y, ref)


def test_zero_down_projection_gives_attention_residual():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    w["w_down"] = np.zeros_like(w["w_down"])
    x = _rng(45).standard_normal((6, cfg.hidden))
    taps = {}
    y = oracle.layer_prefill(x, w, cfg, oracle.mrope_positions(6, []), taps=taps)
    assert np.array_equal(y, taps["y1"])
    assert not np.allclose(y, x)


def test_layer_causality_and_row_sampling():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    x = _rng(46).standard_normal((9, cfg.hidden))
    pos = oracle.mrope_positions(9, [])
    y = oracle.layer_prefill(x, w, cfg, pos)
    x2 = x.copy(); x2[5:] += 1.0
    y2 = oracle.layer_prefill(x2, w, cfg, pos)
    assert np.array_equal(y[:5], y2[:5]) and not np.allclose(y[5:], y2[5:])
    rows = np.array([0, 4, 8])
    assert np.allclose(oracle.layer_prefill_rows(x, w, cfg, pos, rows), y[rows], rtol=1e-13, atol=1e-14)
    # prefix: the layer on x[:5] gives the first 5 rows of the layer on x
    assert np.allclose(oracle.layer_prefill(x[:5], w, cfg, pos[:, :5]), y[:5], rtol=1e-13, atol=1e-14)


def test_stack_feeds_each_layer_the_previous_output():
    cfg = _tiny_cfg()
    w1, w2 = _tiny_weights(cfg, 50), _tiny_weights(cfg, 51)
    x = _rng(47).standard_normal((4, cfg.hidden))
    pos = oracle.mrope_positions(4, [])
    y = oracle.stack_prefill(x, [w1, w2], cfg, pos)
    ref = oracle.layer_prefill(oracle.layer_prefill(x, w1, cfg, pos), w2, cfg, pos)
    assert np.array_equal(y, ref)


# ---------------------------------------------------------------- whole-model prefill (f1)

def _tiny_model(vocab=11, seed=60):
    cfg = _tiny_cfg()
    r = _rng(seed)
    emb = 0.5 * r.standard_normal((vocab, cfg.hidden))
    norm = 1 + 0.1 * r.standard_normal(cfg.hidden)
    head = 0.5 * r.standard_normal((vocab, cfg.hidden))
    return cfg, emb, norm, head


def _brute_logits(h_last, norm, head, eps):
    """RMSNorm and the LM head product written as loops."""
    n = len(h_last)
    ms = sum(v * v for v in h_last) / n
    inv = 1.0 / math.sqrt(ms + eps)
    y = [h_last[k] * inv * norm[k] for k in range(n)]
    return [sum(y[k] * head[v][k] for k in range(n)) for v in range(len(head))]


def test_embedding_lookup_is_one_hot_product_and_checks_ids():
    _, emb, _, _ = _tiny_model()
    tokens = np.array([3, 0, 10, 3, 7])
    one_hot = np.eye(emb.shape[0])[tokens]
    assert np.array_equal(oracle.embed_tokens(tokens, emb), one_hot @ emb)
    with pytest.raises(ValueError):
        oracle.embed_tokens(np.array([1, 11]), emb)
    with pytest.raises(ValueError):
        oracle.embed_tokens(np.array([-1]), emb)
    with pytest.raises(ValueError):
        oracle.embed_tokens(np.array([], dtype=np.int64), emb)


def test_model_without_layers_is_norm_and_head_of_last_embedding():
    cfg, emb, norm, head = _tiny_model()
    tokens = np.array([4, 9, 2])
    pos = oracle.mrope_positions(3, [])
    got = oracle.model_prefill_logits_last(tokens, emb, [], norm, head, cfg, pos)
    ref = _brute_logits(emb[2].tolist(), norm.tolist(), head.tolist(), cfg.eps)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_model_zero_projection_layers_carry_embedding_plus_deepstack_per_layer():
    """With Wo = Wd = 0 every layer passes the residual through, so the last row is the
    embedding plus the DeepStack slabs of the layers il < len(slabs) that reach it."""
    cfg, emb, norm, head = _tiny_model()
    layers = []
    for li in range(3):
        w = _tiny_weights(cfg, 61 + li)
        w["wo"] = np.zeros_like(w["wo"]); w["w_down"] = np.zeros_like(w["w_down"])
        layers.append(w)
    tokens = np.array([1, 5, 8, 6])
    pos = oracle.mrope_positions(4, [])
    ds_rows = np.array([1, 3])
    slabs = [_rng(70 + i).standard_normal((2, cfg.hidden)) for i in range(2)]
    got = oracle.model_prefill_logits_last(tokens, emb, layers, norm, head, cfg, pos, ds_rows, slabs)
    last = emb[6] + slabs[0][1] + slabs[1][1]    # row 3 = DeepStack row 1, layers 0 and 1 only
    ref = _brute_logits(last.tolist(), norm.tolist(), head.tolist(), cfg.eps)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)
    got1 = oracle.model_prefill_logits_last(tokens, emb, layers, norm, head, cfg, pos, ds_rows, slabs[:1])
    ref1 = _brute_logits((emb[6] + slabs[0][1]).tolist(), norm.tolist(), head.tolist(), cfg.eps)
    assert np.allclose(got1, ref1, rtol=1e-12, atol=1e-13)


def test_model_tied_head_scale_and_vocab_permutation():
    cfg, emb, norm, head = _tiny_model()
    layers = [_tiny_weights(cfg, 80), _tiny_weights(cfg, 81)]
    tokens = np.array([2, 7, 7, 0, 10])
    pos = oracle.mrope_positions(5, [(1, 2, 2)])
    base = oracle.model_prefill_logits_last(tokens, emb, layers, norm, head, cfg, pos)
    # tied embeddings: the head is the embedding table itself
    assert np.array_equal(oracle.model_prefill_logits_last(tokens, emb, layers, norm, None, cfg, pos),
                          oracle.model_prefill_logits_last(tokens, emb, layers, norm, emb, cfg, pos))
    # the final norm weight scales the logits linearly
    scaled = oracle.model_prefill_logits_last(tokens, emb, layers, 3.0 * norm, head, cfg, pos)
    assert np.allclose(scaled, 3.0 * base, rtol=1e-12, atol=1e-13)
    # renumbering the vocabulary renumbers the logits
    perm = _rng(82).permutation(emb.shape[0])
    inv = np.argsort(perm)
    got = oracle.model_prefill_logits_last(inv[tokens], emb[perm], layers, norm, head[perm], cfg, pos)
    assert np.allclose(got, base[perm], rtol=1e-12, atol=1e-13)
    # the last-row restriction of the final layer equals the full stack's last row
    full = oracle.stack_prefill(oracle.embed_tokens(tokens, emb), layers, cfg, pos)
    assert np.allclose(oracle.lm_head_last(full[-1], norm, head, cfg.eps), base, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- vision rope + bidirectional attention (f2)

def test_merge_block_order_matches_hand_example():
    got = oracle.merge_block_positions(1, 4, 4, 2)
    assert np.array_equal(got.reshape(-1), _golden_ints("vision_merge_blocks_1x4x4_m2.txt"))
    two = oracle.merge_block_positions(2, 2, 4, 2)
    assert np.array_equal(two[:8, 1:], got[:8, 1:]) and np.array_equal(two[8:, 1:], got[:8, 1:])
    assert np.array_equal(two[:, 0], [0] * 8 + [1] * 8)


def test_rope_tables_2d_structure():
    hd, theta = 32, 10000.0
    half, nf = hd // 2, hd // 4
    c0, s0 = oracle.rope_tables_2d((1, 1, 1), hd, theta, 1)
    assert np.array_equal(c0, np.ones((1, hd))) and np.array_equal(s0, np.zeros((1, hd)))
    cos, sin = oracle.rope_tables_2d((1, 4, 6), hd, theta, 2)
    pos = oracle.merge_block_positions(1, 4, 6, 2)
    assert np.array_equal(cos[:, :half], cos[:, half:]) and np.array_equal(sin[:, :half], sin[:, half:])
    # frequency 0 is 1: slot 0 rotates by the row, slot nf by the column
    assert np.allclose(np.arctan2(sin[:, 0], cos[:, 0]), pos[:, 1], atol=1e-14)
    assert np.allclose(cos[:, nf], np.cos(pos[:, 2]), atol=1e-15) and np.allclose(sin[:, nf], np.sin(pos[:, 2]), atol=1e-15)
    # slot i of a patch in row 1 turns by theta^(-2i/half)
    k = int(np.nonzero((pos[:, 1] == 1) & (pos[:, 2] == 0))[0][0])
    for i in range(nf):
        assert abs(np.arctan2(sin[k, i], cos[k, i]) - theta ** (-2.0 * i / half)) < 1e-14
        assert abs(sin[k, nf + i]) == 0.0


def test_rope_tables_3axis_structure():
    hd, theta = 64, 10000.0
    half = hd // 2
    nt, nh, nw = 8, 12, 12        # 4:6:6 of the 32 angles
    cos, sin = oracle.rope_tables_3axis((2, 4, 4), hd, theta, 2)
    pos = oracle.merge_block_positions(2, 4, 4, 2)
    assert np.array_equal(cos[:, :half], cos[:, half:])
    for slot, axis in ((0, 0), (nt, 1), (nt + nh, 2)):
        assert np.allclose(np.arctan2(sin[:, slot], cos[:, slot]), pos[:, axis], atol=1e-14)
    k = int(np.nonzero((pos[:, 0] == 1) & (pos[:, 1] == 1) & (pos[:, 2] == 1))[0][0])
    ang = np.arctan2(sin[k, :half], cos[k, :half])
    for n, lo in ((nt, 0), (nh, nt), (nw, nt + nh)):
        assert np.allclose(ang[lo:lo + n], theta ** (-np.arange(n) / n), atol=1e-14)
    assert nt + nh + nw == half


def test_rope_split_half_is_textbook_rotation():
    r = _rng(90)
    n, heads, hd = 5, 3, 16
    x = r.standard_normal((n, heads, hd))
    phi = r.uniform(-3, 3, (n, hd // 2))
    cos = np.cos(np.concatenate([phi, phi], axis=1)); sin = np.sin(np.concatenate([phi, phi], axis=1))
    y = oracle.rope_split_half(x, cos, sin)
    z = (x[..., :hd // 2] + 1j * x[..., hd // 2:]) * np.exp(1j * phi)[:, None, :]
    assert np.allclose(y[..., :hd // 2], z.real, atol=1e-14) and np.allclose(y[..., hd // 2:], z.imag, atol=1e-14)


def test_rope_adjacent_lanes():
    r = _rng(91)
    n, heads, hd = 4, 2, 8
    x = r.standard_normal((n, heads, hd))
    # equal angles on each pair: a rotation of (x_2i, x_2i+1)
    phi = r.uniform(-3, 3, (n, hd // 2))
    ang = np.repeat(phi, 2, axis=1)
    y = oracle.rope_adjacent(x, np.cos(ang), np.sin(ang))
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * phi)[:, None, :]
    assert np.allclose(y[..., 0::2], z.real, atol=1e-14) and np.allclose(y[..., 1::2], z.imag, atol=1e-14)
    # different angles on the two lanes of a pair: lane 1 of e_0 takes the sine of its own angle
    e0 = np.zeros((1, 1, 4)); e0[0, 0, 0] = 1.0
    a = np.array([[0.3, 1.1, 0.0, 0.0]])
    y0 = oracle.rope_adjacent(e0, np.cos(a), np.sin(a))[0, 0]
    assert np.allclose(y0, [math.cos(0.3), math.sin(1.1), 0.0, 0.0], atol=1e-15)


def _brute_attention_full(q, k, v):
    s, nh, hd = q.shape
    group = nh // k.shape[1]
    out = np.zeros_like(q)
    for h in range(nh):
        g = h // group
        for i in range(s):
            z = [sum(q[i, h, e] * k[j, g, e] for e in range(hd)) / math.sqrt(hd) for j in range(s)]
            m = max(z)
            p = [math.exp(t - m) for t in z]
            tot = sum(p)
            for e in range(hd):
                out[i, h, e] = sum(p[j] * v[j, g, e] for j in range(s)) / tot
    return out


def test_bidirectional_attention_pins():
    r = _rng(92)
    s, nh, nkv, hd = 6, 4, 2, 4
    q, k, v = r.standard_normal((s, nh, hd)), r.standard_normal((s, nkv, hd)), r.standard_normal((s, nkv, hd))
    o = oracle.bidirectional_attention(q, k, v)
    assert np.allclose(o, _brute_attention_full(q, k, v), rtol=1e-12, atol=1e-13)
    perm = r.permutation(s)
    assert np.allclose(oracle.bidirectional_attention(q[perm], k[perm], v[perm]), o[perm], rtol=1e-12, atol=1e-13)
    # the last query sees every key, as in causal attention
    assert np.allclose(o[-1], oracle.causal_gqa_attention(q, k, v)[-1], rtol=1e-12, atol=1e-13)
    assert np.allclose(o, oracle.bidirectional_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)),
                       rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- KV cache + decode step (f3)

def test_decode_attention_brute_force_and_last_causal_row():
    r = _rng(93)
    L, nh, nkv, hd = 7, 4, 2, 4
    q, k, v = r.standard_normal((nh, hd)), r.standard_normal((L, nkv, hd)), r.standard_normal((L, nkv, hd))
    o = oracle.decode_attention(q, k, v)
    for h in range(nh):
        g = h // 2
        z = [sum(q[h, e] * k[j, g, e] for e in range(hd)) / math.sqrt(hd) for j in range(L)]
        p = [math.exp(t - max(z)) for t in z]
        want = [sum(p[j] * v[j, g, e] for j in range(L)) / sum(p) for e in range(hd)]
        assert np.allclose(o[h], want, rtol=1e-12, atol=1e-13)
    # the query of the last position of a causal prefill sees exactly the cache
    qs = np.concatenate([r.standard_normal((L - 1, nh, hd)), q[None]], axis=0)
    assert np.allclose(o, oracle.causal_gqa_attention(qs, k, v)[-1], rtol=1e-12, atol=1e-13)
    # a single cached key returns its value; the order of the cache rows does not matter
    assert np.allclose(oracle.decode_attention(q, k[:1], v[:1]), np.repeat(v[0], 2, axis=0), rtol=0, atol=1e-15)
    perm = r.permutation(L)
    assert np.allclose(oracle.decode_attention(q, k[perm], v[perm]), o, rtol=1e-12, atol=1e-13)


def test_prefill_kv_entries_are_the_normed_rotated_keys():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    s = 5
    x = _rng(94).standard_normal((s, cfg.hidden))
    pos = oracle.mrope_positions(s, [(1, 2, 2)])
    y, kc, vc = oracle.prefill_kv(x, w, cfg, pos)
    assert np.allclose(y, oracle.layer_prefill(x, w, cfg, pos), rtol=0, atol=0)
    xn = oracle.rms_norm(x, w["attn_norm"], cfg.eps)
    v = brute.matvec_rows(xn.tolist(), w["wv"].tolist())
    assert np.allclose(vc.reshape(s, -1), v, rtol=1e-12, atol=1e-13)
    # the rotation keeps each (i, i + hd/2) pair's norm: the norm of the per-head RMSNorm
    k = np.asarray(brute.matvec_rows(xn.tolist(), w["wk"].tolist())).reshape(s, cfg.n_kv_heads, cfg.head_dim)
    kn = k / np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + cfg.eps) * w["k_norm"]
    half = cfg.head_dim // 2
    assert np.allclose(kc[..., :half] ** 2 + kc[..., half:] ** 2, kn[..., :half] ** 2 + kn[..., half:] ** 2,
                       rtol=1e-12, atol=1e-13)
    # position 0 is not rotated
    assert np.allclose(kc[0], kn[0], rtol=1e-12, atol=1e-13)


def test_decode_steps_reproduce_the_prefill_rows():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg, seed=95)
    n, s0 = 9, 4
    x = _rng(96).standard_normal((n, cfg.hidden))
    pos = oracle.mrope_positions(n, [(1, 2, 2)])
    full = oracle.layer_prefill(x, w, cfg, pos)
    _, kc, vc = oracle.prefill_kv(x[:s0], w, cfg, pos[:, :s0])
    for t in range(s0, n):
        y, kn, vn = oracle.layer_decode(x[t], w, cfg, pos[:, t], kc, vc)
        assert np.allclose(y, full[t], rtol=1e-11, atol=1e-12)
        kc = np.concatenate([kc, kn[None]], axis=0)
        vc = np.concatenate([vc, vn[None]], axis=0)
    # the appended entries equal the ones a prefill over the whole sequence forms
    _, k_all, v_all = oracle.prefill_kv(x, w, cfg, pos)
    assert np.allclose(kc, k_all, rtol=1e-12, atol=1e-13) and np.allclose(vc, v_all, rtol=1e-12, atol=1e-13)
    # a decode step on an empty cache is the one-token prefill
    y0, _, _ = oracle.layer_decode(x[0], w, cfg, pos[:, 0], kc[:0], vc[:0])
    assert np.allclose(y0, full[0], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- quantized weights (f4)

def _golden_q4_0(name):
    blocks, weights = [], []
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            if line.startswith("bytes"):
                blocks.append([int(t, 16) for t in line.split()[1:]])
            elif line.startswith("weights"):
                weights.append([float(t) for t in line.split()[1:]])
    return np.array(blocks, dtype=np.uint8), np.array(weights)


def test_q4_0_matches_hand_worked_blocks():
    blocks, want = _golden_q4_0("q4_0_two_blocks.txt")
    assert blocks.shape == (2, 18)
    got = oracle.dequant_q4_0(blocks.reshape(-1), 1, 64)
    assert np.array_equal(got.reshape(2, 32), want)


def _q4_0_brute(blocks, rows, cols):
    import struct
    raw = bytes(np.asarray(blocks, dtype=np.uint8).reshape(-1))
    out = [[0.0] * cols for _ in range(rows)]
    for o in range(rows):
        for b in range(cols // 32):
            off = (o * (cols // 32) + b) * 18
            d = struct.unpack("<e", raw[off:off + 2])[0]
            for j in range(16):
                byte = raw[off + 2 + j]
                out[o][32 * b + j] = d * ((byte & 15) - 8)
                out[o][32 * b + j + 16] = d * ((byte >> 4) - 8)
    return np.array(out)


def test_q4_0_against_byte_loops_and_invariants():
    r = _rng(110)
    rows, cols = 3, 96
    blocks = r.integers(0, 256, size=(rows, cols // 32, 18), dtype=np.uint8)
    blocks[:, :, 0:2] = np.array(r.uniform(-2, 2, (rows, cols // 32)), dtype="<f2")[..., None].view(np.uint8)
    w = oracle.dequant_q4_0(blocks, rows, cols)
    assert np.array_equal(w, _q4_0_brute(blocks, rows, cols))
    # every code 8 is the zero matrix; the scale is linear
    z = blocks.copy()
    z[:, :, 2:] = 0x88
    assert np.array_equal(oracle.dequant_q4_0(z, rows, cols), np.zeros((rows, cols)))
    half = blocks.copy()
    half[:, :, 0:2] = (blocks[:, :, 0:2].copy().view("<f2") / 2).astype("<f2").view(np.uint8)
    assert np.array_equal(oracle.dequant_q4_0(half, rows, cols), w / 2)
    with pytest.raises(ValueError):
        oracle.dequant_q4_0(blocks, rows, 100)


def test_q4_0_round_trip_of_a_simple_quantizer():
    # quantize with d = max|w| / 7 and codes round(w / d) + 8 (clipped), then dequantize:
    # every weight comes back within half a step (plus the scale's binary16 rounding)
    r = _rng(111)
    rows, cols = 4, 64
    w = 0.02 * r.standard_normal((rows, cols))
    blocks = np.zeros((rows, cols // 32, 18), dtype=np.uint8)
    for o in range(rows):
        for b in range(cols // 32):
            seg = w[o, 32 * b:32 * b + 32]
            d = np.float16(np.abs(seg).max() / 7)
            codes = np.clip(np.rint(seg / np.float64(d)) + 8, 0, 15).astype(np.uint8)
            blocks[o, b, 0:2] = np.array([d], dtype="<f2").view(np.uint8)
            blocks[o, b, 2:] = codes[:16] | (codes[16:] << 4)
    back = oracle.dequant_q4_0(blocks, rows, cols)
    d_all = np.repeat(blocks[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64), 32, axis=1)
    assert np.all(np.abs(back - w) <= 0.5 * d_all + 1e-3 * np.abs(w) + 1e-12)


def test_q8_row_against_loops_and_invariants():
    r = _rng(112)
    rows, cols = 5, 48
    q = r.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    rs = r.uniform(0.001, 0.01, rows).astype(np.float32)
    w = oracle.dequant_q8_row(q, rs)
    want = [[float(rs[o]) * int(q[o, j]) for j in range(cols)] for o in range(rows)]
    assert np.array_equal(w, np.array(want))
    assert np.array_equal(oracle.dequant_q8_row(q, np.ones(rows)), q.astype(np.float64))
    # the product with the dequantized rows equals the row scale times the integer dot product
    x = r.standard_normal((3, cols))
    assert np.allclose(oracle.linear(x, w), (x @ q.T.astype(np.float64)) * rs[None, :], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- generator

def test_generator_deterministic_and_distributions():
    cfg = synth.get_config("qwen3vl_2b_text")
    w1 = synth.make_layer_weights(cfg)
    w2 = synth.make_layer_weights(cfg)
    for n in synth.WEIGHT_NAMES:
        assert np.array_equal(w1[n], w2[n])
    assert abs(w1["wq"].std() - 0.02) < 2e-4 and abs(w1["wq"].mean()) < 1e-4
    assert abs(w1["attn_norm"].mean() - 1.0) < 0.02 and abs(w1["attn_norm"].std() - 0.1) < 0.01
    # bf16-exact: the low 16 bits of every float32 are zero
    assert np.all((w1["wq"].view(np.uint32) & 0xFFFF) == 0)
    x = synth.make_x(cfg)
    assert abs(x.std() - 1.0) < 0.01
    assert not np.array_equal(synth.make_layer_weights(cfg, 1)["wq"], w1["wq"])


def test_model_generators_deterministic():
    cfg = synth.get_config("tiny_f32")
    t1, t2 = synth.make_tokens(cfg, 1000), synth.make_tokens(cfg, 1000)
    assert np.array_equal(t1, t2) and t1.dtype == np.int32 and t1.min() >= 0 and t1.max() < 1000
    e1, n1, h1 = synth.make_model_weights(cfg, 50)
    e2, _, h2 = synth.make_model_weights(cfg, 50, tied=True)
    assert np.array_equal(e1, e2) and h2 is None and h1.shape == e1.shape == (50, cfg.hidden)
    assert not np.array_equal(e1, h1)


def test_quant_generators_deterministic_and_scaled():
    cfg = synth.get_config("tiny_f32")
    n1, p1 = synth.make_quant_layer_weights(cfg, 0, {"wo": "q8_row", "wk": "dense"})
    n2, p2 = synth.make_quant_layer_weights(cfg, 0, {"wo": "q8_row", "wk": "dense"})
    assert set(p1) == set(synth.PROJ_NAMES) and set(n1) == set(synth.NORM_NAMES)
    for k in p1:
        assert p1[k][0] == p2[k][0] and np.array_equal(p1[k][1], p2[k][1])
    fmt, blocks, _ = p1["w_gate"]
    assert fmt == "q4_0" and blocks.shape == (cfg.ffn, cfg.hidden // 32, 18) and blocks.dtype == np.uint8
    w = oracle.dequant_q4_0(blocks, cfg.ffn, cfg.hidden)
    assert abs(w.std() - 0.02) < 0.002
    q, rs = p1["wo"][1], p1["wo"][2]
    assert q.dtype == np.int8 and q.min() >= -127 and rs.dtype == np.float32
    assert np.array_equal(p1["wk"][1], synth.make_layer_weights(cfg, 0, ("wk",))["wk"])


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.0 - 2 ** -8], np.float32)
    r = synth.round_to_bf16(vals)
    assert list(r) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -1.0]
