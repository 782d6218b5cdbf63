"""CPU tests of the measurement tooling: the profiled-kernel classifier that keys the
HBM-traffic and SQ-counter summaries (and the benchmark's traffic lookup)."""
import pytest

from exact_attention_102_amd.traffic import classify


@pytest.mark.parametrize("name,expected", [
    ("void fa::fwd_kernel<128, 128, 32, 4, 3, false, false>(fa::FwdArgs)", ("fwd", "full")),
    ("void fa::fwd_kernel<128, 128, 32, 4, 3, true, false>(fa::FwdArgs)", ("fwd", "causal")),
    ("void fa::dq_kernel<128, 128, 64, 8, 2, false, false>(fa::BwdArgs)", ("dq", "full")),
    ("void fa::dkdv_kernel<128, 128, 32, 8, true, true, 2, true, false>(fa::BwdArgs)", ("dkdv_atomic", "causal")),
    ("void fa::dkdv_kernel<256, 256, 32, 4, false, false, 2, false, false>(fa::BwdArgs)", ("dkdv", "full")),
    # wide kernels: <D, DV, BQ, waves, CAUSAL, ATOMIC>
    ("void fa::dkdv_wide_kernel<128, 128, 32, 4, false, true>(fa::BwdArgs)", ("dkdv_atomic", "full")),
    ("void fa::dkdv_wide_kernel<128, 128, 64, 4, true, false>(fa::BwdArgs)", ("dkdv", "causal")),
    ("void fa::dkdv_wide_kernel<128, 96, 32, 4, true, true>(fa::BwdArgs)", ("dkdv_atomic", "causal")),
    ("void fa::preprocess_kernel<128>(fa::PreArgs)", ("preprocess", None)),
])
def test_classify(name, expected):
    assert classify(name) == expected


@pytest.mark.parametrize("name", [
    # dropout kernels (last template argument true) are timed by their own report
    "void fa::fwd_kernel<128, 128, 64, 4, 2, false, true>(fa::FwdArgs)",
    "void fa::dkdv_kernel<128, 128, 64, 4, false, false, 0, false, true>(fa::BwdArgs)",
    "void elementwise_copy_kernel(float*)",
])
def test_classify_skips(name):
    assert classify(name) is None
