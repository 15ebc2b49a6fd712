"""Host-side checks of the benchmark script: the one-GPU rule, the roofline
arithmetic and the lookup of the committed HBM counters.  Nothing here
touches a GPU."""
import os
import subprocess
import sys

import pytest

import bench
import sparse_mixture_experts_32_amd as M
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_and_flops_at_the_decode_shape():
    w = W.WORKLOADS["decode_bf16_T8"]
    counts = [1, 0, 0, 3, 2, 1, 5, 4]                     # 6 experts with rows
    a = bench.algorithmic(w, counts)
    wbytes = 4096 * 14336 * 2
    assert a["n_active"] == 6
    assert a["swiglu_bytes"] == 6 * 2 * wbytes + 2 * 8 * 4096 + 16 * 14336 * 2
    assert a["swiglu_flops"] == 16 * 4 * 4096 * 14336
    assert a["layer_flops"] == 16 * 6 * 4096 * 14336 + 2 * 8 * 4096 * 8


def test_roofline_object_is_bytes_over_time_against_the_hbm_peak():
    w = W.WORKLOADS["decode_bf16_T8"]
    a = bench.algorithmic(w, [1, 0, 0, 3, 2, 1, 5, 4])
    plan = dict(streaming=True, swiglu_splits=1)
    r = bench.roofline_for(w, a, {"expert_swiglu": 0.25}, plan)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(a["swiglu_bytes"] / 0.25e-3 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
    assert r["kernel"] == "stream_sk_kernel"


def test_roofline_object_is_flops_over_time_against_the_mfma_peak():
    w = W.WORKLOADS["prefill_bf16_T4096_zipf"]
    a = bench.algorithmic(w, [3511, 1757, 1170, 878, 702, 585, 502, 439])
    plan = dict(streaming=False, swiglu_splits=0)
    r = bench.roofline_for(w, a, {"expert_swiglu": 1.7}, plan)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(a["swiglu_flops"] / 1.7e-3 / 1e12, rel=1e-3)
    assert r["kernel"] == "tiled_gemm_kernel<256, true, 256, false>"
    if "sclk_ghz" in r:          # while the committed counters match the kernel source
        assert 1.0 < r["sclk_ghz"] < 2.5
        assert r["peak_at_sclk"] == pytest.approx(2500.0 * r["sclk_ghz"] / 2.4, rel=1e-3)
        assert r["frac_at_sclk"] == pytest.approx(r["achieved"] / r["peak_at_sclk"], rel=1e-3)


def test_w1w3_kernel_name_follows_the_plan():
    assert bench.swiglu_kernel(dict(streaming=True, swiglu_splits=0))[0] == "stream_gemm_kernel<1, 1>"
    assert bench.swiglu_kernel(dict(streaming=True, swiglu_splits=3))[0] == "stream_sk_kernel"
    assert bench.swiglu_kernel(dict(streaming=False, swiglu_splits=0))[1] == "expert_tiled_bf16.hip"
    assert bench.swiglu_kernel(M.plan_for(512, 4096, 14336, 8, 2, M.BF16))[0] == "tiled_mixed_kernel"
    assert (bench.swiglu_kernel(M.plan_for(4096, 4096, 14336, 8, 2, M.BF16))[0]
            == "tiled_gemm_kernel<256, true, 256, false>")


def test_committed_counters_are_found_only_for_their_kernel_and_workload():
    """The headline's plan names the per-matrix streaming kernel; the committed
    counter rows carry the sha256 of the source they were taken with, so a
    row is found while that source is unchanged and never for another
    workload."""
    plan = M.plan_for(8, 4096, 14336, 8, 2, M.BF16)
    assert plan["streaming"]
    got = bench.measured_traffic("decode_bf16_T8", plan)
    if got is not None:           # None only while the kernel changed since profiling
        # the decode workload routes to 7 experts: 7 x 2 x 117.4 MB = 1.644 GB
        # of W1/W3 weights, plus the token rows and partial sums
        assert 1.60e9 < got < 1.75e9
    assert bench.measured_traffic("no_such_workload", plan) is None


def test_attention_clock_comes_from_the_committed_counters_of_its_source():
    """The prefill attention row of the committed counters carries the clock
    the part held under the kernel; decode's dispatches are too short for one.
    None for any other kernel or workload."""
    got = bench.attn_sclk("swa_attn_kernel<2>", "attn_prefill_bf16_T4096")
    if got is not None:          # None only while swa_attention.hip changed since profiling
        assert 1.0 < got < 2.5
    assert bench.attn_sclk("swa_attn_kernel<1>", "attn_decode_bf16_B8") is None
    assert bench.attn_sclk("swa_attn_kernel<2>", "no_such_workload") is None
