"""GPU parity of the vision-tower pieces against the float64 oracle: rotary
tables of a patch grid (2-D and 3-axis), their split-half and adjacent-lane application, and
bidirectional attention (head_dim 64 and 128), plus a composed attention block."""

import numpy as np
import pytest

import oracle
from util import ALLOW16, ALLOW_ATTN16, dev, err16, host, log_err, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402


def _rng(seed):
    return np.random.default_rng(seed)


def _round(a, fmt):
    """Host values exactly representable in fmt."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    conv = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[fmt]
    return t.to(conv).to(torch.float32).numpy()


@pytest.mark.parametrize("layout,grid,merge,hd", [("2d", (1, 16, 24), 2, 64), ("2d", (2, 8, 8), 2, 128),
                                                  ("3axis", (2, 8, 12), 2, 64), ("3axis", (1, 16, 16), 2, 128),
                                                  ("2d", (1, 5, 7), 1, 32)])
def test_vision_rope_tables_match_oracle(layout, grid, merge, hd):
    cos, sin = q3.vision_rope_tables(grid, hd, 10000.0, merge, layout)
    torch.cuda.synchronize()
    fn = oracle.rope_tables_2d if layout == "2d" else oracle.rope_tables_3axis
    rc, rs = fn(grid, hd, 10000.0, merge)
    assert np.max(np.abs(host(cos) - rc)) <= 1e-6 and np.max(np.abs(host(sin) - rs)) <= 1e-6


@pytest.mark.parametrize("pairing,fmt,pad", [("split", "f32", 0), ("split", "bf16", 0), ("adjacent", "f16", 0),
                                             ("adjacent", "f32", 0), ("split", "f16", 0),
                                             # a row stride off the 8-element grid: the scalar form
                                             ("split", "f16", 4), ("adjacent", "bf16", 4)])
def test_apply_rope_tables_matches_oracle(pairing, fmt, pad):
    n, heads, hd = 200, 6, 64
    r = _rng(100)
    # q lives in the first third of a [n, 3 * heads * hd (+ pad)] row (a strided view, as in a
    # qkv buffer)
    rows = _round(r.standard_normal((n, 3 * heads * hd + pad)), fmt)
    phi = r.uniform(-6, 6, (n, hd))
    cos_t, sin_t = np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)
    x = dev(rows, fmt)
    q = x[:, :heads * hd].view(n, heads, hd)
    q3.apply_rope_tables(q, dev(cos_t), dev(sin_t), pairing)
    torch.cuda.synchronize()
    fn = oracle.rope_split_half if pairing == "split" else oracle.rope_adjacent
    ref = fn(rows[:, :heads * hd].reshape(n, heads, hd), cos_t.astype(np.float64), sin_t.astype(np.float64))
    got = host(x)
    assert np.array_equal(got[:, heads * hd:], rows[:, heads * hd:])  # k, v untouched
    if fmt == "f32":
        assert rel_err(got[:, :heads * hd].reshape(n, heads, hd), ref) <= 1e-6
    else:
        assert err16(got[:, :heads * hd].reshape(n, heads, hd), ref, fmt) <= 1e-6


@pytest.mark.parametrize("fmt,s,nh,nkv,hd", [("f16", 333, 16, 16, 64), ("bf16", 640, 32, 8, 128),
                                             ("f16", 100, 8, 2, 64), ("bf16", 1, 4, 4, 128),
                                             ("f16", 1030, 16, 16, 64)])
def test_bidirectional_attention_matches_oracle(fmt, s, nh, nkv, hd):
    r = _rng(110 + s)
    q = _round(2.0 * r.standard_normal((s, nh, hd)), fmt)
    k = _round(2.0 * r.standard_normal((s, nkv, hd)), fmt)
    v = _round(r.standard_normal((s, nkv, hd)), fmt)
    o = q3.gqa_bidirectional_attention(dev(q, fmt), dev(k, fmt), dev(v, fmt))
    torch.cuda.synchronize()
    ref = oracle.bidirectional_attention(q, k, v)
    err = err16(host(o), ref, fmt)
    log_err(f"bidirectional_attention[{fmt},S{s},{nh}/{nkv},hd{hd}]", err)
    assert err <= ALLOW_ATTN16[fmt]


def test_bidirectional_attention_f32_and_causal_head_dim_64():
    r = _rng(120)
    q, k, v = r.standard_normal((50, 4, 64)), r.standard_normal((50, 2, 64)), r.standard_normal((50, 2, 64))
    o = q3.gqa_bidirectional_attention(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    assert rel_err(host(o), oracle.bidirectional_attention(q, k, v)) <= 1e-5
    # the causal kernel at head_dim 64 (16-bit)
    s, nh, nkv, hd = 300, 8, 2, 64
    q = _round(2.0 * r.standard_normal((s, nh, hd)), "f16")
    k = _round(2.0 * r.standard_normal((s, nkv, hd)), "f16")
    v = _round(r.standard_normal((s, nkv, hd)), "f16")
    o = q3.gqa_causal_attention(dev(q, "f16"), dev(k, "f16"), dev(v, "f16"))
    torch.cuda.synchronize()
    assert err16(host(o), oracle.causal_gqa_attention(q, k, v), "f16") <= ALLOW_ATTN16["f16"]


@pytest.mark.parametrize("layout,pairing", [("3axis", "adjacent"), ("2d", "split")])
def test_vision_attention_block(layout, pairing):
    """tables -> rotate q and k inside a fused qkv buffer -> bidirectional attention."""
    grid, merge, heads, hd, fmt = (2, 16, 16), 2, 16, 64, "f16"
    n = grid[0] * grid[1] * grid[2]
    r = _rng(130)
    qkv = _round(r.standard_normal((n, 3 * heads * hd)), fmt)
    x = dev(qkv, fmt)
    cos, sin = q3.vision_rope_tables(grid, hd, 10000.0, merge, layout)
    d = heads * hd
    q3.apply_rope_tables(x[:, :d].view(n, heads, hd), cos, sin, pairing)
    q3.apply_rope_tables(x[:, d:2 * d].view(n, heads, hd), cos, sin, pairing)
    q = x[:, :d].contiguous().view(n, heads, hd)
    k = x[:, d:2 * d].contiguous().view(n, heads, hd)
    v = x[:, 2 * d:].contiguous().view(n, heads, hd)
    o = q3.gqa_bidirectional_attention(q, k, v)
    torch.cuda.synchronize()
    tabs = (oracle.rope_tables_2d if layout == "2d" else oracle.rope_tables_3axis)(grid, hd, 10000.0, merge)
    rope = oracle.rope_split_half if pairing == "split" else oracle.rope_adjacent
    qr = rope(qkv[:, :d].reshape(n, heads, hd), *tabs)
    kr = rope(qkv[:, d:2 * d].reshape(n, heads, hd), *tabs)
    vv = qkv[:, 2 * d:].reshape(n, heads, hd)
    got = host(o)
    # The rotated q and k are stored in fp16 before the products (2^-11 relative per element).
    # Against the oracle fed those same rounded values, the bound of a single 16-bit step holds;
    # against the exact rotation, the storage rounding adds ~4e-3 of the output RMS at this shape.
    ref_rounded = oracle.bidirectional_attention(_round(qr, fmt), _round(kr, fmt), vv)
    err_r = err16(got, ref_rounded, fmt)
    err = err16(got, oracle.bidirectional_attention(qr, kr, vv), fmt)
    log_err(f"vision_block[{layout},{pairing}]", err)
    assert err_r <= ALLOW_ATTN16[fmt] and err <= 1e-2, (err_r, err)
