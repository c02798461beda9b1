"""Helpers shared by the GPU tests: device copies of seeded inputs and the error metric."""

import numpy as np

import json
import os

# max |gpu - oracle| / RMS(oracle) for a whole layer output (fp32 residual stream), by the
# layer's weight dtype
TOL = {"f32": 1e-4, "bf16": 2e-2}
# the same bound for a single step whose output is stored in a 16-bit format: the output
# rounding alone can reach half an ulp of the largest element (2^-8 relative for bf16,
# 2^-11 for fp16, with elements up to ~5x the RMS), plus the step's own arithmetic error
TOL16 = {"bf16": 2e-2, "f16": 4e-3, "f32": 2e-6}


# A 16-bit output differs from the exact value by its own rounding (at most half an ulp:
# 2^-8 of the value for bf16, 2^-11 for fp16, round to nearest even) plus the arithmetic error
# of the step, allowed up to ALLOW16 x RMS(exact).
HALF_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
ALLOW16 = {"bf16": 6e-3, "f16": 1e-3, "f32": 2e-6}
# Attention stores its probabilities in fp16 without rescaling them on every new row maximum
# (lazy rescaling), so every probability, the row maximum's included, carries one fp16 rounding
# (relative 2^-12); a dominant weight w perturbed by that moves the output by up to
# 2^-12 * w * |v_max - o|, a few 1e-4 of RMS. fp16 allowance 2e-3; bf16 operands rescale on every
# increase (their largest probability stays exactly 1) and keep the single-step allowance.
ALLOW_ATTN16 = {"bf16": ALLOW16["bf16"], "f16": 2e-3, "f32": ALLOW16["f32"]}


def err16(gpu, ref, fmt):
    """max over elements of (|gpu - ref| - half_ulp(fmt) * |ref|) / RMS(ref)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape and np.all(np.isfinite(gpu))
    excess = np.abs(gpu - ref) - HALF_ULP[fmt] * np.abs(ref)
    return float(np.max(excess) / np.sqrt(np.mean(ref * ref)))


def log_err(name, err):
    """Append a measured error to the file named by $Q3_PARITY_LOG (if set)."""
    path = os.environ.get("Q3_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": name, "max_abs_err_over_rms": err}) + "\n")


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    return float(np.max(np.abs(gpu - ref)) / np.sqrt(np.mean(ref * ref)))


def dev(a, dtype="f32"):
    """Host float32 array (bf16-exact values for bf16) -> contiguous CUDA tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    conv = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    return t.to(conv).contiguous()


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def dev_weights(w, dtype):
    return {n: dev(a, dtype) for n, a in w.items()}
