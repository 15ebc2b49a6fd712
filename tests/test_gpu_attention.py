"""Parity of the sliding-window grouped-query attention kernels (through the C
ABI) with the float64 attention oracle, on the GPU.

Inputs are seeded (``workloads.attn_inputs``); the oracle receives the same
bf16 values upcast exactly.  Bar: for every (token, head) output row,
max|o - o_ref| <= 1e-2 * rms(o_ref row), on the fp32 output.  Reading behind
it: q, k, v and the cache are bf16 and the products accumulate in fp32 like
the MoE's bf16 layer, whose bar is 1e-2 of rms; the one extra rounding is of
the softmax weights to bf16 before the P.V product, a relative error of at
most 2^-9 per weight, so the error of a row scales with that row's own size.
Rows differ in size by the window they see (a token with 2 keys has |o| ~ 1,
one with 4096 keys |o| ~ 1/64), hence the bar per row rather than over the
whole tensor.  The bf16 output must equal round-to-nearest-even of the fp32
output bit for bit, and the rolling-buffer append is an exact copy.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import sparse_mixture_experts_32_amd as M
import workloads as W
from oracle import swa_oracle as A

pytestmark = pytest.mark.gpu

TOL = 1e-2


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()
    return torch.device("cuda:0")


def np64(t):
    return t.detach().double().cpu().numpy()


def rel(got, ref):
    """max over (token, head) rows of max|got - ref| / rms(ref row)."""
    d = np.abs(got - ref).max(axis=-1)
    r = np.sqrt(np.mean(ref ** 2, axis=-1))
    return float(np.max(d / r))


def small(**kw):
    base = W.AttnWorkload("attn_small", 1, 8, 16, 8, 2, (0,), 20240210)
    return dataclasses.replace(base, **kw)


def run_both(inp, Wn):
    o32 = M.swa_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                          inp["pos0"], Wn, out_dtype=torch.float32)
    o16 = M.swa_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                          inp["pos0"], Wn)
    torch.cuda.synchronize()
    return o32, o16


def oracle_rows(inp, w, b, rows=None):
    return A.swa_chunk_attention(np64(inp["q"][b]), np64(inp["k_new"][b]), np64(inp["v_new"][b]),
                                 np64(inp["k_cache"][b]), np64(inp["v_cache"][b]),
                                 int(w.pos0[b]), w.W, rows=rows)


CASES = [
    dict(B=2, T=5, W=16, H=8, KVH=2, pos0=(0, 37)),            # empty and wrapped cache
    dict(B=1, T=16, W=16, H=4, KVH=4, pos0=(3,)),               # MHA (group 1), chunk = W
    dict(B=3, T=33, W=64, H=8, KVH=4, pos0=(0, 64, 1000)),      # group 2, ragged tile
    dict(B=1, T=100, W=128, H=32, KVH=8, pos0=(130,)),          # two query tiles per wave
    dict(B=2, T=1, W=4096, H=8, KVH=2, pos0=(5000, 10)),        # decode, key splits
    dict(B=1, T=64, W=64, H=4, KVH=1, pos0=(1,)),               # one kv head for 4 heads
    dict(B=2, T=1, W=1, H=4, KVH=1, pos0=(0, 9)),               # W = 1: each token alone
    dict(B=1, T=2, W=2, H=8, KVH=2, pos0=(5,)),                 # W = 2, chunk = W
    dict(B=8, T=1, W=512, H=32, KVH=8, pos0=(700,) * 4 + (100,) * 4),    # 2 key splits
    dict(B=8, T=1, W=1024, H=32, KVH=8, pos0=(5000,) * 4 + (1023,) * 4),  # 4 key splits
    dict(B=1, T=128, W=2048, H=32, KVH=8, pos0=(3000,)),      # two tiles per wave + key splits
    dict(B=1, T=1, W=32768, H=8, KVH=2, pos0=(100000,)),      # large window, 16 key splits
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dW%dH%dKV%d" % (
    c["B"], c["T"], c["W"], c["H"], c["KVH"]))
def test_attention_vs_oracle(dev, case):
    w = small(**case)
    say("attention", case)
    inp = W.attn_inputs(w, dev)
    o32, o16 = run_both(inp, w.W)
    worst = 0.0
    for b in range(w.B):
        ref = oracle_rows(inp, w, b)
        worst = max(worst, rel(np64(o32[b]), ref))
    say("max|d|/rms = %.2e" % worst)
    assert worst <= TOL
    # bf16 store = round-to-nearest-even of the fp32 result, bit for bit
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_attention_deterministic(dev):
    w = small(B=2, T=1, W=4096, H=8, KVH=2, pos0=(5000, 4100))
    inp = W.attn_inputs(w, dev)
    a, _ = run_both(inp, w.W)
    b, _ = run_both(inp, w.W)
    assert torch.equal(a, b)


def test_workspace_reused_across_shapes(dev):
    """One workspace serves shapes with different split counts and tile grids
    in turn (each call overwrites what the previous left): every output
    equals the call with a fresh workspace bit for bit."""
    shapes = [small(B=8, T=1, W=4096, H=32, KVH=8, pos0=(8191,) * 8),     # 8 splits
              small(B=2, T=1, W=4096, H=8, KVH=2, pos0=(5000, 10)),       # 16 splits
              small(B=1, T=128, W=2048, H=32, KVH=8, pos0=(3000,)),       # two-tile kernel
              small(B=8, T=1, W=1024, H=32, KVH=8, pos0=(5000,) * 8)]     # 4 splits
    need = max(M.swa_workspace_size(w.B, w.T, w.W, w.H, w.KVH) for w in shapes)
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=dev)   # not zero on purpose
    for w in shapes + shapes[:1]:
        say("shared workspace", w.B, w.T, w.W, w.H, w.KVH)
        assert M.swa_workspace_size(w.B, w.T, w.W, w.H, w.KVH) > 0
        inp = W.attn_inputs(w, dev)
        args = (inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["pos0"],
                w.W)
        shared = M.swa_attention(*args, out_dtype=torch.float32, workspace=ws)
        fresh = M.swa_attention(*args, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(shared, fresh)


def test_cache_append_bit_exact(dev):
    for T, Wn, pos in [(5, 16, (14, 0)), (20, 16, (3, 30)), (1, 4096, (8191, 4096))]:
        w = small(B=2, T=T, W=Wn, H=4, KVH=2, pos0=pos)
        inp = W.attn_inputs(w, dev)
        kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
        exp_k, exp_v = kc.cpu().clone(), vc.cpu().clone()
        for b in range(w.B):
            for t in range(max(0, T - Wn), T):
                s = A.rolling_slot(pos[b] + t, Wn)
                exp_k[b, s] = inp["k_new"][b, t].cpu()
                exp_v[b, s] = inp["v_new"][b, t].cpu()
        M.swa_cache_append(inp["k_new"], inp["v_new"], inp["pos0"], kc, vc)
        torch.cuda.synchronize()
        assert torch.equal(kc.cpu(), exp_k) and torch.equal(vc.cpu(), exp_v), (T, Wn)


@pytest.mark.parametrize("chunk", [16, 10, 1])
def test_chunked_prefill_through_rolling_cache(dev, chunk):
    """The pages' procedure end to end on the GPU: chunks attend to the cache,
    then are appended; the outputs equal sliding-window attention over the
    whole sequence (float64 oracle)."""
    Tn, Wn, H, KVH = 70, 16, 8, 2
    w = small(B=1, T=Tn, W=Tn, H=H, KVH=KVH, pos0=(0,))
    full = W.attn_inputs(w, dev)                       # q, k_new, v_new of the whole sequence
    kc = torch.zeros((1, Wn, KVH, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    outs = []
    for c0 in range(0, Tn, chunk):
        c1 = min(Tn, c0 + chunk)
        pos0 = torch.tensor([c0], dtype=torch.int32, device=dev)
        q, kn, vn = (full[n][:, c0:c1].contiguous() for n in ("q", "k_new", "v_new"))
        outs.append(M.swa_attention(q, kn, vn, kc, vc, pos0, Wn, out_dtype=torch.float32))
        M.swa_cache_append(kn, vn, pos0, kc, vc)
    torch.cuda.synchronize()
    got = np64(torch.cat(outs, dim=1)[0])
    ref = A.swa_attention(np64(full["q"][0]), np64(full["k_new"][0]), np64(full["v_new"][0]), Wn)
    err = rel(got, ref)
    say("chunked prefill chunk=%d: max|d|/rms = %.2e" % (chunk, err))
    assert err <= TOL


def test_full_size_decode(dev):
    w = W.ATTN_WORKLOADS["attn_decode_bf16_B8"]
    say("full decode", w.name)
    inp = W.attn_inputs(w, dev)
    o32, o16 = run_both(inp, w.W)
    worst = max(rel(np64(o32[b]), oracle_rows(inp, w, b)) for b in range(w.B))
    say("decode B8 W4096: max|d|/rms = %.2e" % worst)
    assert worst <= TOL
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_full_size_prefill_sampled(dev):
    w = W.ATTN_WORKLOADS["attn_prefill_bf16_T4096"]
    say("full prefill", w.name)
    inp = W.attn_inputs(w, dev)
    o32, o16 = run_both(inp, w.W)
    rows = sorted({0, 1, 15, 16, 31, 32, 63, 64, 1000, 2047, 2048, 3071, 4094, 4095} |
                  set(np.random.default_rng(3).choice(w.T, 10, replace=False).tolist()))
    ref = oracle_rows(inp, w, 0, rows=rows)
    err = rel(np64(o32[0][rows]), ref)
    say("prefill T4096 (sampled %d tokens): max|d|/rms = %.2e" % (len(rows), err))
    assert err <= TOL
    assert torch.equal(o16, o32.to(torch.bfloat16))
