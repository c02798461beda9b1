"""GPU: the library's per-kernel timing record (launch counts, summed and median launch times)."""

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import transformer_lm_prefill_amd as q3  # noqa: E402


def test_timing_record_counts_sums_and_medians():
    x = torch.randn(4096, 4096, device="cuda", dtype=torch.float32)
    w = torch.ones(4096, device="cuda", dtype=torch.bfloat16)
    q3.timing_collect()  # drop anything recorded before
    q3.timing_enable(True)
    try:
        for _ in range(7):
            q3.rms_norm_rows(x, w, 1e-6, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        med = {}
        kt = q3.timing_collect(medians=med)
    finally:
        q3.timing_enable(False)
    assert list(kt) == ["rmsnorm"] and list(med) == ["rmsnorm"]
    n, total = kt["rmsnorm"]
    assert n == 7
    # each launch moves 96 MiB: well above event resolution, well below a second
    assert 0.0 < med["rmsnorm"] < 1000.0
    assert 0.0 < total < 7 * 1000.0
    # one launch's median cannot exceed the sum of all seven launches
    assert med["rmsnorm"] <= total
    # nothing is left after a collect, and a disabled record stays empty
    q3.rms_norm_rows(x, w, 1e-6, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert q3.timing_collect() == {}
