"""Host-side checks of bench.py (no GPU): the one-GPU rule, the work each reported TFLOP/s figure
divides by, and the gating of the stored counter traffic by the kernel source digest."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


# Algorithmic work per layer in GFLOP (2 per multiply-add; causal attention counts the pairs
# j <= s only), as tabulated for the workloads: GEMMs and attention of the 2B layer at 1024 and
# 2048 tokens, the 8B layer at 4096 and the 32B layer at 8192.
@pytest.mark.parametrize("name,seq,gemm_gf,attn_gf", [
    ("qwen3vl_2b_text", 1024, 103.08, 4.30),
    ("qwen3vl_2b_image", 2048, 206.16, 17.19),
    ("qwen3vl_8b_stack4", 4096, 1580.55, 137.47),
    ("qwen3_32b_encoder", 8192, 7988.64, 1099.65),
])
def test_layer_work_matches_the_tabulated_counts(name, seq, gemm_gf, attn_gf):
    cfg = synth.get_config(name)
    assert cfg.seq_len == seq
    assert cfg.gemm_flops() / 1e9 == pytest.approx(gemm_gf, abs=0.006)
    assert cfg.attn_flops() / 1e9 == pytest.approx(attn_gf, abs=0.006)


def _fake_run(kt_ms, steps, wall_s):
    """A run_stack result with given total milliseconds per kernel (one launch each per step)."""
    return {"kt": {k: (steps, ms) for k, ms in kt_ms.items()},
            "median": {k: ms / steps for k, ms in kt_ms.items()},
            "wall_s": wall_s, "gpu_ms": wall_s * 1e3, "finite": True}


def test_stack_summary_rates():
    """Each kernel's TFLOP/s is its own product's work over its average launch time: at 1 ms per
    launch the figures equal the work in GFLOP (206.2 QKV, 137.4 o-proj, 824.6 gate/up,
    412.3 down, 137.5 causal attention at the 8B shape)."""
    cfg = synth.get_config("qwen3vl_8b_stack4")
    S, L, steps = cfg.seq_len, cfg.n_layers, 2
    names = ["gemm_qkv", "gemm_o_resid", "gemm_gate_up_swiglu", "gemm_down_resid", "attention"]
    n_launch = L * steps
    r = _fake_run({k: 1.0 * n_launch for k in names}, n_launch, wall_s=0.01)
    out = bench.stack_summary(r, cfg, S, L, steps)
    k = out["kernels"]
    assert k["gemm_qkv"]["tflops"] == pytest.approx(206.2, abs=0.06)
    assert k["gemm_o_resid"]["tflops"] == pytest.approx(137.4, abs=0.06)
    assert k["gemm_gate_up_swiglu"]["tflops"] == pytest.approx(824.6, abs=0.06)
    assert k["gemm_down_resid"]["tflops"] == pytest.approx(412.3, abs=0.06)
    assert k["attention"]["tflops"] == pytest.approx(137.5, abs=0.06)
    assert k["gemm_gate_up_swiglu"]["frac_of_peak"] == pytest.approx(824.6 / 2500, abs=1e-4)
    # the GEMM figure is the four products' total work over their total time (4 ms per layer-step)
    assert out["gemm_tflops"] == pytest.approx(1580.55 / 4, abs=0.06)
    # attention: causal work over its time; the dense-equivalent figure counts all S x S pairs
    assert out["attn_tflops_causal"] == pytest.approx(137.47, abs=0.06)
    assert out["attn_tflops_dense_equivalent"] == pytest.approx(137.47 * 2 * S / (S + 1), abs=0.1)
    # tokens per second per layer: S tokens through L layers per step over the wall time
    assert out["tokens_per_s_layer"] == pytest.approx(S * L * steps / 0.01, rel=1e-6)


def test_stored_traffic_only_for_the_measured_kernel_source(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: t["kernel_source_sha256_16"])
    assert bench.stored_traffic() == (t["bytes_per_launch"], t["algorithmic_bytes_per_launch"])
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0" * 16)
    assert bench.stored_traffic() == (None, None)


def test_traffic_record_is_consistent():
    """The stored HBM bytes are the copy-calibrated counter readings, and the algorithmic bytes
    of the gate/up product at the 8B shape: yn [4096, 4096] and the two [12288, 4096] weight
    matrices read once, a [4096, 12288] written once, all 16-bit."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    c = t["copy_calibration"]
    assert c["fetch_scale"] == pytest.approx(c["bytes"] / 1024 / c["fetch_kib"], rel=1e-3)
    assert c["write_scale"] == pytest.approx(c["bytes"] / 1024 / c["write_kib"], rel=1e-3)
    scaled = (t["fetch_kib_per_launch"] * c["bytes"] / 1024 / c["fetch_kib"]
              + t["write_kib_per_launch"] * c["bytes"] / 1024 / c["write_kib"]) * 1024
    assert t["bytes_per_launch"] == pytest.approx(scaled, rel=1e-6)
    S, H, F = 4096, 4096, 12288
    assert t["algorithmic_bytes_per_launch"] == 2 * (S * H + 2 * F * H + S * F)
    assert len(t["kernel_source_sha256_16"]) == 16
