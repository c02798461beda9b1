"""GPU parity of the KV cache a prefill leaves and of the decode step against the float64 oracle:
cache writes, decode attention over the cache, the prefill that emits the cache, and decode
steps that continue a prefill (whose outputs must equal the longer prefill's rows)."""

import numpy as np
import pytest

import oracle
import synth
from util import TOL, TOL16, dev, dev_i32, dev_weights, host, log_err, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


# the cache rows pass several steps (norm, products, per-head norm, rotation) before their one
# rounding to the cache format: the 16-bit single-step bounds, and 1e-5 for an fp32 cache
CACHE_TOL = {"f32": 1e-5, "f16": TOL16["f16"], "bf16": TOL16["bf16"]}


def _rng(seed):
    return np.random.Generator(np.random.SFC64(seed))


def _round(a, fmt):
    """Host rounding (torch on the CPU, nearest even) of float values to fmt, back as float64."""
    return torch.from_numpy(np.asarray(a, np.float32)).to(TDT[fmt]).to(torch.float64).numpy()


@pytest.mark.parametrize("src,cdt", [("f16", "f16"), ("bf16", "bf16"), ("f32", "f16"), ("f32", "bf16"),
                                     ("f32", "f32"), ("f16", "f32")])
def test_kv_cache_write_places_and_converts_rows(src, cdt):
    n, nkv, hd, cap, row0 = 37, 4, 128, 100, 50
    g = torch.Generator().manual_seed(7)
    wide = torch.randn(n, 3 * nkv * hd, generator=g).to(TDT[src])
    wide_d = wide.cuda()
    k = wide_d[:, nkv * hd:2 * nkv * hd].view(n, nkv, hd)
    v = wide_d[:, 2 * nkv * hd:].view(n, nkv, hd)
    kc = torch.full((nkv, cap, hd), 7.0, dtype=TDT[cdt], device="cuda")
    vc = torch.full_like(kc, -3.0)
    q3.kv_cache_write(k, v, kc, vc, row0)
    torch.cuda.synchronize()
    want_k = torch.full((nkv, cap, hd), 7.0, dtype=TDT[cdt])
    want_v = torch.full((nkv, cap, hd), -3.0, dtype=TDT[cdt])
    want_k[:, row0:row0 + n] = wide[:, nkv * hd:2 * nkv * hd].view(n, nkv, hd).to(TDT[cdt]).permute(1, 0, 2)
    want_v[:, row0:row0 + n] = wide[:, 2 * nkv * hd:].view(n, nkv, hd).to(TDT[cdt]).permute(1, 0, 2)
    assert torch.equal(kc.cpu(), want_k) and torch.equal(vc.cpu(), want_v)


@pytest.mark.parametrize("cdt,hd,nh,nkv,length,cap", [
    ("f16", 128, 32, 8, 1, 16),
    ("f16", 128, 32, 8, 65, 80),
    ("bf16", 128, 32, 8, 1000, 1000),
    ("f16", 128, 32, 8, 4097, 5000),       # two tiles per split, ragged last tile
    ("f16", 64, 16, 16, 777, 800),
    ("bf16", 64, 10, 2, 130, 130),         # 5 query heads per KV head: waves with 2 and 1 heads
    ("f16", 128, 16, 1, 300, 310),         # 16 query heads per KV head: 4 per wave
    ("f32", 64, 4, 2, 300, 301),
    ("f32", 128, 8, 4, 129, 200),
    ("f16", 128, 64, 8, 33000, 33000),     # 32B head layout, long context
])
def test_decode_attention_matches_oracle(cdt, hd, nh, nkv, length, cap):
    r = _rng(100 + length)
    q = 2.0 * r.standard_normal((nh, hd))
    k = _round(r.standard_normal((nkv, cap, hd)), cdt)
    v = _round(r.standard_normal((nkv, cap, hd)), cdt)
    kd, vd = dev(k, cdt), dev(v, cdt)
    if length < cap:   # rows past the live length are never read
        kd[:, length:] = float("nan")
        vd[:, length:] = float("nan")
    got = host(q3.gqa_decode_attention(dev(q, "f32"), kd, vd, length))
    kc, vc = k[:, :length].transpose(1, 0, 2), v[:, :length].transpose(1, 0, 2)
    # the query is rounded to the cache format before the products (the kernel's stated precision)
    ref = oracle.decode_attention(_round(q, cdt), kc, vc)
    err = rel_err(got, ref)
    log_err(f"decode_attention[{cdt},hd{hd},{nh}/{nkv},L{length}]", err)
    assert err <= 2e-5, err
    # against the unrounded query the rounding of q shows (bounded like one 16-bit step)
    assert rel_err(got, oracle.decode_attention(q, kc, vc)) <= 4 * TOL16[cdt]


def test_decode_attention_rejects_bad_arguments():
    q = torch.zeros(8, 128, device="cuda")
    kc = torch.zeros(2, 16, 128, dtype=torch.float16, device="cuda")
    with pytest.raises(q3.Qwen3Error, match="len"):
        q3.gqa_decode_attention(q, kc, kc.clone(), 17)
    with pytest.raises(q3.Qwen3Error, match="len"):
        q3.gqa_decode_attention(q, kc, kc.clone(), 0)
    with pytest.raises(q3.Qwen3Error, match="workspace"):
        q3.gqa_decode_attention(q, kc, kc.clone(), 16, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))


def _layer_case(name, seq=None):
    cfg = synth.get_config(name)
    if seq is not None:
        cfg = cfg.with_seq(seq)
    w = synth.make_layer_weights(cfg)
    return cfg, w, synth.make_x(cfg), synth.make_positions(cfg)


@pytest.mark.parametrize("name,s0", [("tiny_f32", 32), ("qwen3vl_2b_text", 300), ("qwen3vl_2b_image", 1500)])
def test_prefill_kv_writes_the_oracle_cache(name, s0):
    cfg, w, x, pos = _layer_case(name)
    x, pos = x[:s0], pos[:, :s0]
    rows, slab = synth.make_deepstack(cfg)
    if rows is not None:
        keep = rows < s0
        rows, slab = rows[keep], slab[keep]
    spec = q3.LayerSpec.of(cfg)
    dw = dev_weights(w, cfg.dtype)
    kc, vc = q3.kv_cache_alloc(spec, s0 + 9)
    args = (rows, dev(slab, cfg.dtype)) if rows is not None else (None, None)
    y_kv = q3.layer_prefill_kv(spec, dw, dev(x), dev_i32(pos), kc, vc, *args)
    y = q3.layer_prefill(spec, dw, dev(x), dev_i32(pos), *args)
    torch.cuda.synchronize()
    assert torch.equal(y_kv, y)
    assert not torch.any(kc[:, s0:] != 0) and not torch.any(vc[:, s0:] != 0)
    _, k_ref, v_ref = oracle.prefill_kv(x, w, cfg, pos)
    act = spec.act_dtype
    ek = rel_err(host(kc[:, :s0]).transpose(1, 0, 2), k_ref)
    ev = rel_err(host(vc[:, :s0]).transpose(1, 0, 2), v_ref)
    log_err(f"prefill_kv[{name},S{s0}] k", ek)
    log_err(f"prefill_kv[{name},S{s0}] v", ev)
    assert ek <= CACHE_TOL[act] and ev <= CACHE_TOL[act], (ek, ev)


@pytest.mark.parametrize("name,s0,steps,act", [("tiny_f32", 20, 6, ""), ("qwen3vl_2b_text", 300, 3, ""),
                                               ("qwen3vl_2b_image", 1500, 3, ""), ("qwen3vl_2b_text", 0, 2, ""),
                                               # bf16 operands and cache
                                               ("qwen3vl_2b_text", 200, 2, "bf16")])
def test_decode_steps_continue_the_prefill(name, s0, steps, act):
    """Prefill s0 tokens with the cache, then decode tokens s0 .. s0+steps-1 one at a time: every
    decode output equals the oracle's prefill row of that position (image positions included)."""
    cfg, w, x, pos = _layer_case(name)
    full = s0 + steps
    spec = q3.LayerSpec.of(cfg, act)
    dw = dev_weights(w, cfg.dtype)
    kc, vc = q3.kv_cache_alloc(spec, full + 3)
    if s0 > 0:
        q3.layer_prefill_kv(spec, dw, dev(x[:s0]), dev_i32(pos[:, :s0]), kc, vc)
    outs = []
    ws = torch.empty(q3.layer_decode_workspace_bytes(spec, full + 3), dtype=torch.uint8, device="cuda")
    for t in range(s0, full):
        xt = dev(x[t])
        y = q3.layer_decode(spec, dw, xt, dev_i32(pos[:, t]), kc, vc, t, out=xt, workspace=ws)  # in place
        outs.append(host(y))
    ref = oracle.layer_prefill_rows(x[:full], w, cfg, pos[:, :full], np.arange(s0, full))
    err = rel_err(np.stack(outs), ref)
    log_err(f"layer_decode[{name},S0={s0},+{steps}{',' + act if act else ''}]", err)
    print(f"{name}: decode after {s0}: max|err|/rms = {err:.3e}")
    assert err <= TOL[cfg.dtype]
    # the rows the decode steps appended are the oracle's k', v of those positions
    _, k_ref, v_ref = oracle.prefill_kv(x[:full], w, cfg, pos[:, :full])
    act = spec.act_dtype
    ek = rel_err(host(kc[:, s0:full]).transpose(1, 0, 2), k_ref[s0:full])
    ev = rel_err(host(vc[:, s0:full]).transpose(1, 0, 2), v_ref[s0:full])
    assert ek <= CACHE_TOL[act] and ev <= CACHE_TOL[act], (ek, ev)


def test_decode_8b_after_a_4096_token_prefill():
    """The 8B layer shape at full size: prefill 4096 tokens with the cache, then decode token 4096
    (the configuration the bench times); its output is the oracle's row 4096."""
    cfg, w, x, pos = _layer_case("qwen3vl_8b_stack4", seq=4097)
    s0 = 4096
    spec = q3.LayerSpec.of(cfg)
    dw = dev_weights(w, cfg.dtype)
    kc, vc = q3.kv_cache_alloc(spec, 8192)
    q3.layer_prefill_kv(spec, dw, dev(x[:s0]), dev_i32(pos[:, :s0]), kc, vc)
    y = host(q3.layer_decode(spec, dw, dev(x[s0]), dev_i32(pos[:, s0]), kc, vc, s0))
    ref = oracle.layer_prefill_rows(x, w, cfg, pos, np.array([s0]))[0]
    err = rel_err(y, ref)
    log_err("layer_decode[8b,S0=4096]", err)
    print(f"8B decode after 4096: max|err|/rms = {err:.3e}")
    assert err <= TOL[cfg.dtype]
