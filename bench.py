"""Benchmark: prefill tokens/s per decoder layer on the Qwen3-VL-8B-shaped 4-layer stack.

One step = the whole hot path (RMSNorm, QKV, q/k norm + MRoPE, causal GQA attention, o-proj +
residual, RMSNorm, SwiGLU FFN + residual) for all 4 layers over one 4096-token sequence, with
seeded synthetic bf16 weight values (stored once at load as fp16 with the projection matrices
in 16x32 tiles: the same numbers in the products' operand format, read as whole 1 KiB blocks)
and inputs already resident in HBM. The same stack with the bf16 weights as given and with
row-major fp16 weights, the measured MFMA and copy peaks, the streaming kernels' HBM rates on
rotated inputs and the wider paths (whole model, bidirectional attention, decode, Q4_0) are
extra fields. Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E (published)
DOMINANT = "gemm_gate_up_swiglu"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gate_up_swiglu_8b.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="qwen3vl_8b_stack4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-model", action="store_true",
                    help="skip the whole-model (embedding + stack + LM head) measurement")
    ap.add_argument("--vocab", type=int, default=151936)
    ap.add_argument("--no-quant", action="store_true",
                    help="skip the Q4_0-weight layer measurement")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the KV-cache decode measurement")
    ap.add_argument("--no-bidirectional", action="store_true",
                    help="skip the bidirectional-attention (vision encoder shape) measurement")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))


def kernel_sources_digest():
    """Digest of the GEMM kernel source, to tell whether stored counter data is still current."""
    p = os.path.join(ROOT, "transformer_lm_prefill_amd", "csrc", "gemm_mfma.h")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic():
    """(HBM bytes per launch, algorithmic bytes per launch) of the dominant kernel from the
    committed rocprofv3 counter summary, or (None, None) if there is none or the kernel source
    has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    if t.get("kernel_source_sha256_16") != kernel_sources_digest():
        return None, None
    return t.get("bytes_per_launch"), t.get("algorithmic_bytes_per_launch")


def cpu_baseline(cfg, w0, x, pos, n_tok, min_s=10.0, max_reps=8):
    """The float64 oracle (untuned) on the first n_tok tokens of layer 1, timed on this host.
    The pass is repeated until at least min_s seconds of CPU work (or max_reps passes)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    reps = 0
    t = time.perf_counter()
    while True:
        oracle.layer_prefill(x[:n_tok], w0, cfg, pos[:, :n_tok])
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_s or reps >= max_reps:
            break
    return {"value": n_tok * reps / dt, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"layer 1 of the stack on its first {n_tok} tokens, {reps} passes "
                      f"(float64 numpy oracle, {dt:.1f} s)"}


def model_prefill_extra(cfg, layers, pos, stream, vocab, spec=None):
    """The whole-model path on the same layers: embedding lookup, the layer stack, final
    RMSNorm and an untied LM head over `vocab` rows, for the last position's logits. Weights of
    the embedding table and head are seeded random (torch generator) in the layers' element
    type (fp16 for tiled layers)."""
    import torch

    import transformer_lm_prefill_amd as q3
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    spec = spec or q3.LayerSpec.of(cfg)
    wdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f16t": torch.float16, "f32": torch.float32}[spec.dtype]
    emb = (torch.randn(vocab, cfg.hidden, device=dev, generator=g) * 0.02).to(wdt)
    head = (torch.randn(vocab, cfg.hidden, device=dev, generator=g) * 0.02).to(wdt)
    norm = (1 + 0.1 * torch.randn(cfg.hidden, device=dev, generator=g)).to(wdt)
    tokens = torch.randint(0, vocab, (cfg.seq_len,), generator=torch.Generator().manual_seed(5)).tolist()
    ws = torch.empty(q3.model_workspace_bytes(spec, len(layers), vocab, cfg.seq_len), dtype=torch.uint8,
                     device=dev)
    out = torch.empty(vocab, dtype=torch.float32, device=dev)

    def run():
        q3.model_prefill_logits_last(spec, layers, emb, norm, head, tokens, pos, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    n = 3
    t = time.perf_counter()
    for _ in range(n):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / n
    q3.timing_enable(True)
    run()
    torch.cuda.synchronize()
    kt = q3.timing_collect()
    q3.timing_enable(False)
    head_ms = kt["lm_head"][1] / kt["lm_head"][0]
    head_bytes = vocab * cfg.hidden * (4 if wdt == torch.float32 else 2)
    emb_ms = kt["embed_gather"][1] / kt["embed_gather"][0]

    # generation after the prompt: the prefill leaves every layer's cache, then single tokens
    n_dec = 16
    caches = [q3.kv_cache_alloc(spec, cfg.seq_len + n_dec) for _ in layers]
    q3.model_prefill_logits_last(spec, layers, emb, norm, head, tokens, pos, out=out, workspace=ws, caches=caches)
    dws = torch.empty(q3.model_decode_workspace_bytes(spec, len(layers), vocab, cfg.seq_len + n_dec),
                      dtype=torch.uint8, device=dev)
    dpos = torch.arange(cfg.seq_len, cfg.seq_len + n_dec, dtype=torch.int32, device=dev).repeat(3, 1).t().contiguous()
    new_tok = torch.randint(0, vocab, (n_dec,), generator=torch.Generator().manual_seed(6)).tolist()

    def gen():
        for i in range(n_dec):
            q3.model_decode_logits(spec, layers, emb, norm, head, new_tok[i], dpos[i], caches, cfg.seq_len + i,
                                   out=out, workspace=dws)

    gen()
    torch.cuda.synchronize()
    t = time.perf_counter()
    gen()
    torch.cuda.synchronize()
    dec_ms = (time.perf_counter() - t) * 1e3 / n_dec
    return {"workload": f"{cfg.name}: {len(layers)} layers, seq {cfg.seq_len}, vocab {vocab} untied head",
            "weights": spec.dtype,
            "ms": round(ms, 4), "tokens_per_s": round(cfg.seq_len / (ms * 1e-3), 1),
            # the kernels alone (one call, event-timed): "ms" is wall time per call and also holds
            # the token ids' host-side marshalling and their copy to the device
            "kernels_ms": round(sum(v[1] for v in kt.values()), 4),
            "lm_head": {"avg_ms": round(head_ms, 4), "bound": "hbm",
                        "GB_per_s": round(head_bytes / (head_ms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(head_bytes / (head_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "embed_gather_ms": round(emb_ms, 4),
            "decode_after_prompt": {"tokens": n_dec, "ms_per_token": round(dec_ms, 4),
                                    "tokens_per_s": round(1e3 / dec_ms, 1)},
            "finite_logits": bool(torch.isfinite(out).all().item())}


def bidirectional_extra():
    """Bidirectional (no mask) GQA attention on two fp16 shapes: a vision-encoder block over a
    64x64 patch grid (4096 patches, 16 heads of 64, rotary tables applied first) and the text
    layer's head layout (32/8 heads of 128) over 4096 tokens. Seeded N(0,1) q, k, v."""
    import torch

    import transformer_lm_prefill_amd as q3
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    res = {}
    for name, s, nh, nkv, hd in (("vision_4096x16x64", 4096, 16, 16, 64),
                                 ("text_heads_4096x32x8x128", 4096, 32, 8, 128)):
        qkv = torch.randn(s, (nh + 2 * nkv) * hd, device=dev, generator=g).to(torch.float16)
        q = qkv[:, :nh * hd].view(s, nh, hd)
        k = qkv[:, nh * hd:(nh + nkv) * hd].view(s, nkv, hd)
        v = qkv[:, (nh + nkv) * hd:].view(s, nkv, hd)
        qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
        out = torch.empty_like(qc)
        q3.gqa_bidirectional_attention(qc, kc, vc, out=out)
        torch.cuda.synchronize()
        n = 10
        q3.timing_enable(True)
        for _ in range(n):
            q3.gqa_bidirectional_attention(qc, kc, vc, out=out)
        torch.cuda.synchronize()
        kt = q3.timing_collect()
        q3.timing_enable(False)
        ms = kt["attention_bidirectional"][1] / kt["attention_bidirectional"][0]
        tf = 4.0 * s * s * nh * hd / (ms * 1e-3) / 1e12
        res[name] = {"avg_ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        if hd == 64:
            cos, sin = q3.vision_rope_tables((1, 64, 64), hd, 10000.0, 2, layout="2d")
            q3.timing_enable(True)
            for _ in range(n):
                q3.vision_rope_tables((1, 64, 64), hd, 10000.0, 2, layout="2d")
                q3.apply_rope_tables(q, cos, sin, pairing="split")
                q3.apply_rope_tables(k, cos, sin, pairing="split")
            torch.cuda.synchronize()
            kt = q3.timing_collect()
            q3.timing_enable(False)
            res[name]["rope"] = {k2: round(v2[1] / v2[0], 4) for k2, v2 in kt.items()}
    return res


def decode_extra(cfg, layers, x0, pos, n_tokens=16):
    """Decode after a full prompt: every layer's cache is filled by a prefill of the S-token
    prompt through the stack, then n_tokens new tokens go through all layers one at a time
    (positions S, S+1, ...). Also decode attention alone over 4096 and 32768 cached keys."""
    import torch

    import transformer_lm_prefill_amd as q3
    dev = torch.device("cuda:0")
    S, L = cfg.seq_len, len(layers)
    spec = q3.LayerSpec.of(cfg)
    cap = S + n_tokens
    caches = [q3.kv_cache_alloc(spec, cap) for _ in range(L)]
    h = torch.empty_like(x0)
    ws = torch.empty(q3.layer_workspace_bytes(spec, S), dtype=torch.uint8, device=dev)
    q3.layer_prefill_kv(spec, layers[0], x0, pos, *caches[0], out=h, workspace=ws)
    for li in range(1, L):
        q3.layer_prefill_kv(spec, layers[li], h, pos, *caches[li], out=h, workspace=ws)
    del ws
    dws = torch.empty(q3.layer_decode_workspace_bytes(spec, cap), dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    xs = torch.randn(n_tokens, cfg.hidden, device=dev, generator=g)
    tpos = torch.arange(S, S + n_tokens, dtype=torch.int32, device=dev).repeat(3, 1).t().contiguous()
    y = torch.empty(cfg.hidden, device=dev)

    def token(i):
        y.copy_(xs[i])
        for li in range(L):
            q3.layer_decode(spec, layers[li], y, tpos[i], *caches[li], S + i, out=y, workspace=dws)

    token(0)   # warm-up (rewrites row S of every cache with the same values later)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(n_tokens):
        token(i)
    torch.cuda.synchronize()
    ms_tok = (time.perf_counter() - t) * 1e3 / n_tokens
    q3.timing_enable(True)
    for i in range(n_tokens):
        token(i)
    torch.cuda.synchronize()
    kt = q3.timing_collect()
    q3.timing_enable(False)
    H, F, qd, kvd = cfg.hidden, cfg.ffn, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    wbytes = {"gemv_qkv": (qd + 2 * kvd) * H * 2, "gemv_o_resid": H * qd * 2,
              "gemv_gate_up_swiglu": 2 * F * H * 2, "gemv_down_resid": H * F * 2}
    kern = {}
    for k, (n, tot) in kt.items():
        avg = tot / n
        e = {"avg_ms": round(avg, 4)}
        if k in wbytes:
            e["GB_per_s"] = round(wbytes[k] / (avg * 1e-3) / 1e9, 1)
            e["frac_of_hbm_peak"] = round(wbytes[k] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        kern[k] = e
    layer_bytes = sum(wbytes.values()) + 2 * (S + n_tokens // 2) * kvd * 2
    res = {"workload": f"{cfg.name}: {L} layers, {n_tokens} tokens decoded after a {S}-token prompt, "
                       f"fp16 cache", "ms_per_token": round(ms_tok, 4),
           "tokens_per_s": round(1e3 / ms_tok, 1), "ms_per_token_layer": round(ms_tok / L, 4),
           "weight_and_cache_GB_per_s": round(layer_bytes * L / (ms_tok * 1e-3) / 1e9, 1),
           "kernels": kern}
    # decode attention alone at the 8B head layout
    attn = {}
    for length in (4096, 32768):
        kc = torch.randn(cfg.n_kv_heads, length, cfg.head_dim, device=dev, generator=g).to(torch.float16)
        vc = torch.randn(cfg.n_kv_heads, length, cfg.head_dim, device=dev, generator=g).to(torch.float16)
        q = torch.randn(cfg.n_heads, cfg.head_dim, device=dev, generator=g)
        wsa = torch.empty(q3.decode_attention_workspace_bytes(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, length),
                          dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        q3.gqa_decode_attention(q, kc, vc, length, out=out, workspace=wsa)
        torch.cuda.synchronize()
        q3.timing_enable(True)
        for _ in range(20):
            q3.gqa_decode_attention(q, kc, vc, length, out=out, workspace=wsa)
        torch.cuda.synchronize()
        kt = q3.timing_collect()
        q3.timing_enable(False)
        ms = kt["decode_attention"][1] / kt["decode_attention"][0]
        b = 2 * length * cfg.n_kv_heads * cfg.head_dim * 2
        attn[f"len_{length}"] = {"avg_ms": round(ms, 4), "GB_per_s": round(b / (ms * 1e-3) / 1e9, 1),
                                 "frac_of_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del kc, vc
    res["decode_attention"] = attn
    return res


def quant_extra(cfg, x0, pos, n_tokens=16):
    """One 8B-shaped layer with every projection in Q4_0 blocks (seeded random codes and scales):
    the prefill of the S-token prompt (expansion + MFMA products) and decode steps after it
    (matrix-vector products on the quantized bytes)."""
    import numpy as np
    import torch

    import synth
    import transformer_lm_prefill_amd as q3
    dev = torch.device("cuda:0")
    S = cfg.seq_len
    norms, proj = synth.make_quant_layer_weights(cfg, 0)
    wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dn = {n: torch.from_numpy(a).to(dev).to(wdt) for n, a in norms.items()}
    dp = {n: (f, torch.from_numpy(np.ascontiguousarray(d)).to(dev), None) for n, (f, d, _) in proj.items()}
    qbytes = {n: d.numel() for n, (_, d, _) in dp.items()}
    spec = q3.LayerSpec.of(cfg)
    cap = S + n_tokens
    kc, vc = q3.kv_cache_alloc(spec, cap)
    ws = torch.empty(q3.layer_quant_workspace_bytes(spec, S), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x0)

    def prefill():
        q3.layer_prefill_quant(spec, dn, dp, x0, pos, k_cache=kc, v_cache=vc, out=y, workspace=ws)

    prefill()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(3):
        prefill()
    torch.cuda.synchronize()
    ms_pre = (time.perf_counter() - t) * 1e3 / 3
    q3.timing_enable(True)
    prefill()
    torch.cuda.synchronize()
    kt = q3.timing_collect()
    q3.timing_enable(False)
    res = {"workload": f"{cfg.name} layer 1 with Q4_0 projections (18 bytes per 32 weights), seq {S}",
           "prefill": {"ms": round(ms_pre, 4), "tokens_per_s": round(S / (ms_pre * 1e-3), 1),
                       "dequant_ms": round(kt["dequant"][1], 4) if "dequant" in kt else 0.0,
                       "q4_0_decoded_in_products": "dequant" not in kt,
                       "kernels_ms": {k: round(v[1], 4) for k, v in kt.items()}}}
    del ws
    dws = torch.empty(q3.layer_decode_workspace_bytes(spec, cap), dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    xs = torch.randn(n_tokens, cfg.hidden, device=dev, generator=g)
    tpos = torch.arange(S, S + n_tokens, dtype=torch.int32, device=dev).repeat(3, 1).t().contiguous()
    out = torch.empty(cfg.hidden, device=dev)

    def decode_all():
        for i in range(n_tokens):
            q3.layer_decode_quant(spec, dn, dp, xs[i], tpos[i], kc, vc, S + i, out=out, workspace=dws)

    decode_all()
    torch.cuda.synchronize()
    t = time.perf_counter()
    decode_all()
    torch.cuda.synchronize()
    ms_tok = (time.perf_counter() - t) * 1e3 / n_tokens
    q3.timing_enable(True)
    decode_all()
    torch.cuda.synchronize()
    kt = q3.timing_collect()
    q3.timing_enable(False)
    gbytes = {"gemv_qkv": qbytes["wq"] + qbytes["wk"] + qbytes["wv"], "gemv_o_resid": qbytes["wo"],
              "gemv_gate_up_swiglu": qbytes["w_gate"] + qbytes["w_up"], "gemv_down_resid": qbytes["w_down"]}
    kern = {}
    for k, (n, tot) in kt.items():
        avg = tot / n
        e = {"avg_ms": round(avg, 4)}
        if k in gbytes:
            e["GB_per_s"] = round(gbytes[k] / (avg * 1e-3) / 1e9, 1)
            e["frac_of_hbm_peak"] = round(gbytes[k] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        kern[k] = e
    res["decode"] = {"ms_per_token_layer": round(ms_tok, 4), "tokens_per_s_layer": round(1e3 / ms_tok, 1),
                     "quantized_weight_MB": round(sum(gbytes.values()) / 1e6, 1), "kernels": kern}
    return res


def measured_peaks():
    """What this GPU delivers under load, next to the published peaks: the MFMA throughput probe
    (fp16 32x32x16, no memory traffic; also the shader clock it ran at) and a plain 1 GiB
    device-to-device copy (torch)."""
    import torch

    import transformer_lm_prefill_amd as q3
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg, iters = 8 * cus, 2000
    q3.mfma_probe(wg, 100)
    runs = [q3.mfma_probe(wg, iters) for _ in range(3)]
    ms, flop, ghz = min(runs, key=lambda r: r[0])
    tf = flop / (ms * 1e-3) / 1e12
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    cms = e0.elapsed_time(e1) / reps
    gbs = 2 * n / (cms * 1e-3) / 1e9
    return {"mfma_probe_f16": {"tflops": round(tf, 1), "frac_of_published_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                               "shader_clock_ghz": round(ghz, 3), "launch_ms": round(ms, 4),
                               "what": f"{wg} workgroups x 4 waves x {iters} x 8 independent 32x32x16 fp16 MFMAs"},
            "copy_1GiB": {"GB_per_s": round(gbs, 1), "frac_of_published_peak": round(gbs / HBM_PEAK_GBS, 4),
                          "what": "torch device-to-device copy of 1 GiB (read + write counted)"}}


def streaming_rotated(cfg):
    """HBM rate of the two streaming kernels of the layer with inputs that the 256 MB MALL cannot
    hold: each launch works on the next of several copies of its operands (> 512 MB in all),
    timed per launch with events on the library's stream (the 8B shapes, S = seq_len)."""
    import torch

    import transformer_lm_prefill_amd as q3
    dev = torch.device("cuda:0")
    S, H = cfg.seq_len, cfg.hidden
    nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    res = {}
    # RMSNorm: fp32 [S, H] in, fp16 [S, H] out: S*H*(4 + 2) bytes per launch
    ncopy = 10
    xs = [torch.randn(S, H, device=dev, generator=g) for _ in range(ncopy)]
    ys = [torch.empty(S, H, dtype=torch.float16, device=dev) for _ in range(ncopy)]
    w = (1 + 0.1 * torch.randn(H, device=dev, generator=g)).to(torch.bfloat16)
    for i in range(ncopy):
        q3.rms_norm_rows(xs[i], w, 1e-6, out=ys[i])
    torch.cuda.synchronize()
    q3.timing_enable(True)
    for _ in range(3):
        for i in range(ncopy):
            q3.rms_norm_rows(xs[i], w, 1e-6, out=ys[i])
    torch.cuda.synchronize()
    kt = q3.timing_collect()
    q3.timing_enable(False)
    ms = kt["rmsnorm"][1] / kt["rmsnorm"][0]
    b = S * H * 6
    res["rmsnorm"] = {"avg_ms": round(ms, 4), "bytes": b, "GB_per_s": round(b / (ms * 1e-3) / 1e9, 1),
                      "frac_of_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "rotation": f"{ncopy} input/output pairs, {ncopy * S * H * 6 / 2**20:.0f} MiB"}
    del xs, ys
    # q/k RMSNorm + MRoPE in place on fp16 q [S, nh, hd] and k [S, nkv, hd]: read + write both
    ncopy = 14
    qs = [torch.randn(S, nh, hd, device=dev, generator=g).to(torch.float16) for _ in range(ncopy)]
    ks = [torch.randn(S, nkv, hd, device=dev, generator=g).to(torch.float16) for _ in range(ncopy)]
    qn = (1 + 0.1 * torch.randn(hd, device=dev, generator=g)).to(torch.bfloat16)
    kn = (1 + 0.1 * torch.randn(hd, device=dev, generator=g)).to(torch.bfloat16)
    pos = torch.arange(S, dtype=torch.int32, device=dev).repeat(3, 1).contiguous()
    for i in range(ncopy):
        q3.qk_norm_mrope(qs[i], ks[i], qn, kn, pos, 1e-6, cfg.theta, cfg.sections)
    torch.cuda.synchronize()
    q3.timing_enable(True)
    for _ in range(3):
        for i in range(ncopy):
            q3.qk_norm_mrope(qs[i], ks[i], qn, kn, pos, 1e-6, cfg.theta, cfg.sections)
    torch.cuda.synchronize()
    kt = q3.timing_collect()
    q3.timing_enable(False)
    ms = kt["qk_norm_mrope"][1] / kt["qk_norm_mrope"][0]
    b = 2 * S * (nh + nkv) * hd * 2
    res["qk_norm_mrope"] = {"avg_ms": round(ms, 4), "bytes": b, "GB_per_s": round(b / (ms * 1e-3) / 1e9, 1),
                            "frac_of_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "rotation": f"{ncopy} q/k pairs, {ncopy * S * (nh + nkv) * hd * 2 / 2**20:.0f} MiB"}
    return res


def run_stack(q3, spec, layers, x0, pos, rows, ds, S, L, steps, warmup):
    """Warm-up, then the timed region of `steps` whole steps (every kernel of all L layers), then
    the same steps again with each launch bracketed by events on the library's stream."""
    import torch
    dev = x0.device
    h = torch.empty_like(x0)
    ws = torch.empty(q3.layer_workspace_bytes(spec, S), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        q3.layer_prefill(spec, layers[0], x0, pos, rows, ds, out=h, workspace=ws)
        for li in range(1, L):
            q3.layer_prefill(spec, layers[li], h, pos, out=h, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # ---- timed region: K whole steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    # ---- per-kernel durations
    q3.timing_enable(True)
    torch.cuda.synchronize()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    med = {}
    kt = q3.timing_collect(medians=med)
    q3.timing_enable(False)
    finite = bool(torch.isfinite(h).all().item())
    return {"wall_s": wall, "gpu_ms": gpu_ms, "kt": kt, "median": med, "finite": finite}


def stack_summary(r, cfg, S, L, steps):
    kt = r["kt"]
    gemm_flops = cfg.gemm_flops() * L * steps
    attn_flops = cfg.attn_flops() * L * steps
    gemm_ms = sum(v[1] for k, v in kt.items() if k.startswith("gemm"))
    attn_ms = sum(v[1] for k, v in kt.items() if k == "attention")
    gemm_tf = gemm_flops / (gemm_ms * 1e-3) / 1e12
    attn_tf = attn_flops / (attn_ms * 1e-3) / 1e12
    per_kernel_flops = {"gemm_qkv": 2.0 * S * cfg.hidden * (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim,
                        "gemm_o_resid": 2.0 * S * cfg.n_heads * cfg.head_dim * cfg.hidden,
                        "gemm_gate_up_swiglu": 2.0 * S * cfg.hidden * 2 * cfg.ffn,
                        "gemm_down_resid": 2.0 * S * cfg.ffn * cfg.hidden,
                        "attention": cfg.attn_flops()}
    kernels = {}
    for k, (n, tot) in kt.items():
        e = {"launches": n, "avg_ms": round(tot / n, 4), "median_ms": round(r["median"][k], 4)}
        if k in per_kernel_flops:
            tf = per_kernel_flops[k] / (tot / n * 1e-3) / 1e12
            e["tflops"] = round(tf, 1)
            e["frac_of_peak"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        kernels[k] = e
    return {"tokens_per_s_layer": round(S * L * steps / r["wall_s"], 1),
            "ms_per_step": round(r["wall_s"] * 1e3 / steps, 4),
            "gpu_event_ms_per_step": round(r["gpu_ms"] / steps, 4),
            "gemm_tflops": round(gemm_tf, 1), "gemm_frac_of_peak": round(gemm_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "attn_tflops_causal": round(attn_tf, 1), "attn_frac_of_peak": round(attn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            # the same time against the work of all S x S pairs (as if nothing were masked)
            "attn_tflops_dense_equivalent": round(attn_tf * 2.0 * S / (S + 1), 1),
            "kernels": kernels, "finite_output": r["finite"]}


def main():
    args = parse()
    if args.copy_calib:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sequence sharding is designed, not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import transformer_lm_prefill_amd as q3

    cfg = synth.get_config(args.config)
    dev = torch.device("cuda:0")
    S, L = cfg.seq_len, cfg.n_layers
    spec = q3.LayerSpec.of(cfg)

    def to(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        return t.to(torch.bfloat16) if dt == "bf16" else t

    host_layers = []
    layers = []
    for li in range(L):
        w = synth.make_layer_weights(cfg, li)
        if li == 0:
            host_layers.append(w)
        layers.append({n: to(a, cfg.dtype) for n, a in w.items()})
        del w
    x_host = synth.make_x(cfg)
    pos_host = synth.make_positions(cfg)
    x0 = to(x_host, "f32")
    pos = torch.from_numpy(pos_host).to(dev)
    rows_h, ds_h = synth.make_deepstack(cfg)
    rows = rows_h  # host row list (checked by the library before any launch)

    # The weights are generated as bf16 values (the workload's format). Loading stores them once
    # as fp16, the format of the matrix products, with the projection matrices in the tiled
    # layout (qwen3_tile_weights: 16-row x 32-column tiles of 1 KiB): every such bf16 value of
    # magnitude in [2^-14, 65504] is an fp16 value, so this re-encodes the same numbers; the
    # kernels then read operand-format weights as whole 1 KiB blocks instead of converting each
    # bf16 tile in their inner loop.
    prepared, spec_run = layers, spec
    prep_ms = None
    if cfg.dtype == "bf16":
        torch.cuda.synchronize()
        t = time.perf_counter()
        prepared = [q3.tile_layer_weights(lw) for lw in layers]
        torch.cuda.synchronize()
        prep_ms = (time.perf_counter() - t) * 1e3
        spec_run = q3.LayerSpec(**{**spec.__dict__, "dtype": "f16t"})
    ds = None if ds_h is None else to(ds_h, cfg.dtype).to(torch.float16 if cfg.dtype == "bf16" else torch.float32)

    r = run_stack(q3, spec_run, prepared, x0, pos, rows, ds, S, L, args.steps, args.warmup)
    head = stack_summary(r, cfg, S, L, args.steps)
    kt = r["kt"]
    n_dom, ms_dom = kt[DOMINANT]
    dom_flops = 2.0 * S * cfg.hidden * 2 * cfg.ffn     # one launch: gate and up products
    dom_avg_ms = ms_dom / n_dom
    achieved = dom_flops / (dom_avg_ms * 1e-3) / 1e12
    traffic, traffic_alg = stored_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": DOMINANT,
                "avg_launch_ms": round(dom_avg_ms, 4)}
    if traffic and traffic_alg:
        # counter bytes (L2 misses, MALL hits included) over the bytes the product must move once
        roofline["traffic_algorithmic"] = traffic_alg
        roofline["traffic_ratio"] = round(traffic / traffic_alg, 2)

    def extra(skip, fn, *a):
        """A secondary measurement; a failure is reported in its field, not by losing the line."""
        if skip:
            return None
        try:
            return fn(*a)
        except Exception as e:  # noqa: BLE001
            print(f"bench.py: {fn.__name__} failed: {e!r}", file=sys.stderr)
            return {"error": repr(e)}
        finally:
            torch.cuda.synchronize()

    def as_given():
        ds_b = None if ds_h is None else to(ds_h, cfg.dtype)
        rb = run_stack(q3, spec, layers, x0, pos, rows, ds_b, S, L, args.steps, args.warmup)
        out = stack_summary(rb, cfg, S, L, args.steps)
        out["what"] = "the same stack with the bf16 weights as given (each weight tile converted to fp16 in the GEMM loop)"
        return out

    def row_major_f16():
        plain = [{n: t_.to(torch.float16) for n, t_ in lw.items()} for lw in layers]
        rp = run_stack(q3, q3.LayerSpec(**{**spec.__dict__, "dtype": "f16"}), plain, x0, pos, rows, ds, S, L,
                       args.steps, args.warmup)
        out = stack_summary(rp, cfg, S, L, args.steps)
        out["what"] = "the same stack with the fp16 weights row-major (not tiled)"
        return out

    bf16_in_kernel = extra(cfg.dtype != "bf16", as_given)
    f16_row_major = extra(cfg.dtype != "bf16", row_major_f16)
    # the whole model on the headline's weights (tiled layers; its decode steps read them too)
    model = extra(args.no_model, model_prefill_extra, cfg, prepared, pos, None, args.vocab, spec_run)
    del prepared
    peaks = extra(False, measured_peaks)
    streaming = extra(False, streaming_rotated, cfg)
    bidir = extra(args.no_bidirectional, bidirectional_extra)
    decode = extra(args.no_decode, decode_extra, cfg, layers, x0, pos)
    quant = extra(args.no_quant, quant_extra, cfg, x0, pos)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, host_layers[0], x_host, pos_host, args.cpu_sample_tokens)

    out = {
        "metric": "layer prefill tokens/s + attn/GEMM TFLOP/s (% bf16 MFMA peak), 8B shape seq 4096",
        "value": head["tokens_per_s_layer"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "weights_dtype": ("bf16 values, stored once at load as fp16 with the projection matrices in "
                          "16x32 tiles (qwen3_tile_weights; exact re-encoding; "
                          f"{prep_ms:.1f} ms for the {L} layers, outside the timed region)"
                          if prep_ms is not None else cfg.dtype),
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights, 1+N(0,0.1) norms; random-init)",
        "config": {"workload": f"{cfg.name}: {L} decoder layers, hidden {cfg.hidden}, "
                               f"{cfg.n_heads}/{cfg.n_kv_heads} heads, head_dim {cfg.head_dim}, "
                               f"ffn {cfg.ffn}, seq {S}, text-only positions",
                   "layers": L, "seq_len": S, "tokens_per_step": S, "parallelism": "none (1 GPU)"},
        "gpu_event_ms_per_step": head["gpu_event_ms_per_step"],
        "gemm_tflops": head["gemm_tflops"],
        "gemm_frac_of_peak": head["gemm_frac_of_peak"],
        "attn_tflops_causal": head["attn_tflops_causal"],
        "attn_frac_of_peak": head["attn_frac_of_peak"],
        "attn_tflops_dense_equivalent": head["attn_tflops_dense_equivalent"],
        "kernels": head["kernels"],
        "finite_output": head["finite_output"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "streaming_kernels_rotated_inputs": streaming,
        "bf16_weights_in_kernel": bf16_in_kernel,
        "f16_row_major_weights": f16_row_major,
        "model_prefill_logits_last": model,
        "bidirectional_attention": bidir,
        "decode": decode,
        "quantized_q4_0": quant,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
