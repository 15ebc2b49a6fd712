"""moe_forward_noalloc (the allocation-free variant of moe_forward, whose
workspace is the library's static device scratch) against moe_forward with a
caller's workspace, through the C ABI: bit for bit, on consecutive calls that
reuse the one scratch with different shapes and plans."""
from __future__ import annotations

import sys

import pytest
import torch

import sparse_mixture_experts_32_amd as M
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()
    return torch.device("cuda:0")


def _inputs(dev, T, d, d_ff, name="mid_bf16_T512"):
    w = W.scaled(W.WORKLOADS[name], T=T, d=d, d_ff=d_ff)
    return W.layer_inputs(w, dev), w


def _both(inp, K, y_dtype, accumulate=False, y0=None):
    args = (inp["x"], inp["W_g"], inp["W1"], inp["W3"], inp["W2"], K)
    y_ref = None if y0 is None else y0.clone()
    y_new = None if y0 is None else y0.clone()
    y_ref = M.moe_forward(*args, y=y_ref, y_dtype=y_dtype, accumulate=accumulate)
    y_new = M.moe_forward_noalloc(*args, y=y_new, y_dtype=y_dtype, accumulate=accumulate)
    torch.cuda.synchronize()
    return y_ref, y_new


@pytest.mark.parametrize("d,d_ff,T1,T2", [(1024, 2048, 200, 8), (4096, 14336, 40, 8)])
def test_noalloc_matches_forward_on_consecutive_calls(dev, d, d_ff, T1, T2):
    """First call with T1 tokens (tiled plan), then T2 < T1 tokens (streaming
    plan, with W1/W3 partial sums in the scratch), then T1 again: every call
    equals moe_forward bit for bit."""
    for T in (T1, T2, T1):
        inp, w = _inputs(dev, T, d, d_ff)
        plan = M.plan_for(T, d, d_ff, w.E, w.K, M.BF16)
        need = M.workspace_size(T, d, d_ff, w.E, w.K, M.BF16)
        say("noalloc T=%d d=%d d_ff=%d plan %s workspace %d bytes" % (T, d, d_ff, plan, need))
        assert need <= M.NOALLOC_SCRATCH_BYTES
        for y_dtype in (torch.float32, torch.bfloat16):
            y_ref, y_new = _both(inp, w.K, y_dtype)
            assert torch.equal(y_ref, y_new), (T, y_dtype)
        h = torch.randn((T, d), generator=torch.Generator().manual_seed(T)).to(dev, torch.bfloat16)
        y_ref, y_new = _both(inp, w.K, torch.bfloat16, accumulate=True, y0=h)
        assert torch.equal(y_ref, y_new), (T, "accumulate")


def test_noalloc_fp32_layer(dev):
    w = W.WORKLOADS["tiny_f32_T64"]
    for T in (64, 5):
        inp = W.layer_inputs(w, dev, T=T)
        say("noalloc fp32 T=%d" % T)
        y_ref, y_new = _both(inp, w.K, torch.float32)
        assert torch.equal(y_ref, y_new)


def test_noalloc_rejects_oversized_shape_and_keeps_working(dev):
    d, d_ff = 4096, 14336
    need = M.workspace_size(4096, d, d_ff, 8, 2, M.BF16)
    assert need > M.NOALLOC_SCRATCH_BYTES
    inp, w = _inputs(dev, 16, 256, 256)
    big = torch.empty((4096, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(big)
    with pytest.raises(M.MoeError) as ei:
        M.moe_forward_noalloc(big, torch.empty((d, 8), dtype=torch.bfloat16, device=dev),
                              [torch.empty((d, d_ff), dtype=torch.bfloat16, device=dev)] * 8,
                              [torch.empty((d, d_ff), dtype=torch.bfloat16, device=dev)] * 8,
                              [torch.empty((d_ff, d), dtype=torch.bfloat16, device=dev)] * 8,
                              2, y=y)
    assert ei.value.status == 3 and "static scratch" in str(ei.value)
    y_ref, y_new = _both(inp, w.K, torch.float32)
    assert torch.equal(y_ref, y_new)


def test_noalloc_graph_replay(dev):
    """The caller it is for: a step captured in a HIP graph.  Every replay,
    with eager calls of other shapes between replays, equals the eager
    moe_forward result bit for bit."""
    inp, w = _inputs(dev, 8, 512, 1024)
    other, _ = _inputs(dev, 100, 512, 1024)
    args = (inp["x"], inp["W_g"], inp["W1"], inp["W3"], inp["W2"], w.K)
    y_ref = M.moe_forward(*args, y_dtype=torch.float32)
    y = torch.empty_like(y_ref)
    M.moe_forward_noalloc(*args, y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_forward_noalloc(*args, y=y)
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), rep
        M.moe_forward_noalloc(other["x"], other["W_g"], other["W1"], other["W3"], other["W2"],
                              w.K, y_dtype=torch.float32)
        torch.cuda.synchronize()
