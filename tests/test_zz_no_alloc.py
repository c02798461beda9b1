"""gqa_decode_attention_noalloc (the decode attention for callers that cannot allocate) against
the workspace form gqa_decode_attention, through the C ABI: two calls in a row on the library's
fixed per-GPU scratch array, the second with a smaller input, each bit-identical to the
workspace form (same kernels) and within the decode-attention bound of the oracle."""

import ctypes

import numpy as np
import pytest

import oracle
from util import dev, host, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402
from transformer_lm_prefill_amd import _lib  # noqa: E402

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _round(a, fmt):
    return torch.from_numpy(np.asarray(a, np.float32)).to(TDT[fmt]).to(torch.float64).numpy()


def _case(seed, cdt, nh, nkv, hd, length, cap):
    r = np.random.Generator(np.random.SFC64(seed))
    q = 2.0 * r.standard_normal((nh, hd))
    k = _round(r.standard_normal((nkv, cap, hd)), cdt)
    v = _round(r.standard_normal((nkv, cap, hd)), cdt)
    kd, vd = dev(k, cdt), dev(v, cdt)
    if length < cap:
        kd[:, length:] = float("nan")
        vd[:, length:] = float("nan")
    return q, k, v, dev(q, "f32"), kd, vd


def test_noalloc_matches_workspace_form_on_two_calls():
    # first call: the 8B head layout over 4097 cached keys (two key tiles per split, a ragged
    # last tile); second call: a smaller input (fewer heads, head_dim 64, 130 keys, bf16 cache),
    # so the fixed array still holds the first call's larger partial results
    for seed, cdt, nh, nkv, hd, length, cap in ((1, "f16", 32, 8, 128, 4097, 5000),
                                               (2, "bf16", 10, 2, 64, 130, 140)):
        q, k, v, qd, kd, vd = _case(seed, cdt, nh, nkv, hd, length, cap)
        got = q3.gqa_decode_attention_noalloc(qd, kd, vd, length)
        want = q3.gqa_decode_attention(qd, kd, vd, length)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (cdt, nh, nkv, hd, length)
        kc, vc = k[:, :length].transpose(1, 0, 2), v[:, :length].transpose(1, 0, 2)
        err = rel_err(host(got), oracle.decode_attention(_round(q, cdt), kc, vc))
        assert err <= 2e-5, err


def test_noalloc_rejects_partials_beyond_the_fixed_array():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the size check fails first
    # 16384 query heads over 1024 KV heads need 8 MiB + 128 KiB of partial results
    need = lib.gqa_decode_attention_workspace_bytes(16384, 1024, 128, 64)
    assert need > (8 << 20)
    rc = lib.gqa_decode_attention_noalloc(fake, fake, fake, 64, 64, 16384, 1024, 128, 0.1, _lib.QWEN3_F16, fake,
                                          None)
    assert rc == 2 and "8 MiB" in lib.qwen3_last_error().decode()
