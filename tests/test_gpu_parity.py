"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Inputs come from the seeded generators in ``workloads``; the oracle gets the
same bytes (upcast exactly to float) and never sees a HIP output.  Rules and
tolerances: ``tests/parity.py``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import sparse_mixture_experts_32_amd as M
import workloads as W
from oracle import moe_oracle as O
from tests import parity as PY

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


class LazyNp:
    """Converts expert matrices to float numpy only when the oracle asks."""

    def __init__(self, ts):
        self.ts = ts

    def __len__(self):
        return len(self.ts)

    def __getitem__(self, e):
        return PY.to_np(self.ts[e])


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()
    return torch.device("cuda:0")


def small(name="mid_bf16_T512", **kw):
    return W.scaled(W.WORKLOADS[name], **kw)


def run_forward(inp, K, y_dtype=torch.float32, y=None, accumulate=False):
    x = inp["x"]
    T, d = x.shape
    E = len(inp["W1"])
    d_ff = inp["W1"][0].shape[1]
    dt = M.BF16 if x.dtype == torch.bfloat16 else M.F32
    ws = torch.empty(max(M.workspace_size(T, d, d_ff, E, K, dt), 1), dtype=torch.uint8,
                     device=x.device)
    y = M.moe_forward(x, inp["W_g"], inp["W1"], inp["W3"], inp["W2"], K, y=y, y_dtype=y_dtype,
                      accumulate=accumulate, workspace=ws)
    torch.cuda.synchronize()
    views = M.workspace_views(ws, T, d, d_ff, E, K, dt) if T > 0 else {}
    return y, {k: v.clone() for k, v in views.items()}


def oracle(inp, K, faithful, tokens=None):
    x = PY.to_np(inp["x"])
    if tokens is not None:
        x = x[tokens]
    return O.moe_forward(x, PY.to_np(inp["W_g"]), LazyNp(inp["W1"]), LazyNp(inp["W3"]),
                         LazyNp(inp["W2"]), K, faithful=faithful)


def check_layer(inp, K, tokens=None, bf16_store=True):
    x = inp["x"]
    is_bf16 = x.dtype == torch.bfloat16
    T = x.shape[0]
    E = len(inp["W1"])
    y32, v = run_forward(inp, K, torch.float32)
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    y_ref, aux = oracle(inp, K, faithful=is_bf16, tokens=rows)
    set_ok = PY.check_routing(v["topk_idx"].cpu().numpy()[rows], v["topk_w"].cpu().numpy()[rows],
                              aux["idx"], aux["w"], aux["logits"], K)
    err = PY.rel_err(PY.to_np(y32)[rows], y_ref, set_ok)
    tol = PY.TOL_BF16 if is_bf16 else PY.TOL_F32
    say("rel err %.3e (tol %.0e) over %d decided of %d tokens" % (err, tol, set_ok.sum(), len(rows)))
    assert err <= tol
    if tokens is None:
        keep = np.zeros(T, dtype=bool)
        keep[rows[set_ok]] = True
        PY.check_permutation(v["offsets"].cpu().numpy(), v["sorted_token"].cpu().numpy(),
                             aux["idx"], E, K, keep)
    if is_bf16 and bf16_store:
        yb, _ = run_forward(inp, K, torch.bfloat16)
        assert torch.equal(yb, PY.bf16_rne_of(y32))
    return y32, v, err


# ---------------------------------------------------------------- router
# T >= 1024 with 8 experts takes the many-token router (4 tokens per workgroup,
# the features split over its 4 wavefronts), fewer tokens the general one; the
# small batches cover decode sizes, and d = 6144 gives k-loops with a ragged
# number of chunks per thread (and per wavefront in the many-token router)
@pytest.mark.parametrize("dtype,T,K,d", [("bf16", 300, 2, 256), ("f32", 300, 2, 256),
                                         ("bf16", 1500, 2, 256), ("bf16", 1027, 1, 256),
                                         ("bf16", 1100, 4, 256), ("f32", 1100, 2, 256),
                                         ("bf16", 1, 2, 256), ("bf16", 8, 8, 256),
                                         ("bf16", 13, 4, 512), ("bf16", 32, 2, 6144),
                                         ("bf16", 21, 3, 4096), ("f32", 8, 2, 256),
                                         ("bf16", 1030, 2, 6144), ("bf16", 1024, 2, 4096)])
def test_router_small(dev, dtype, T, K, d):
    w = small(T=T, d=d, d_ff=128, dtype=dtype)
    say("router", dtype, w.T, w.d, K)
    W_g, _, _, _ = W.expert_weights(w, dev, experts=[])
    x = W.make_x(w, W_g, dev)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    idx, wt = M.moe_router_topk(x, W_g, K, logits=logits)
    torch.cuda.synchronize()
    l64 = O.router_logits(PY.to_np(x), PY.to_np(W_g))
    assert np.abs(PY.to_np(logits) - l64).max() <= 1e-5 * (1 + np.abs(l64).max())
    ref_idx = O.topk_select(l64, K)
    PY.check_routing(idx.cpu().numpy(), wt.cpu().numpy(), ref_idx, O.gate_weights(l64, ref_idx),
                     l64, K)


@pytest.mark.parametrize("T", [32, 512, 1100])
def test_router_ties_lower_index_wins(dev, T):
    """Columns 5 and 7 of W_g copy column 2, so logits 2, 5, 7 tie exactly (in
    fp32 on the GPU and in float64 in the oracle).  Where the distinct logit
    values around the selection are more than 1e-3 apart, the GPU must make
    the oracle's choice, which resolves the tie towards the lower index."""
    w = small(T=T, d=128, d_ff=128, E=8)
    say("router ties")
    W_g, _, _, _ = W.expert_weights(w, dev, experts=[])
    W_g[:, 5] = W_g[:, 2]
    W_g[:, 7] = W_g[:, 2]
    x = W.make_x(w, W_g, dev)
    idx, _ = M.moe_router_topk(x, W_g, 2)
    torch.cuda.synchronize()
    l64 = O.router_logits(PY.to_np(x), PY.to_np(W_g))
    assert np.array_equal(l64[:, 2], l64[:, 5]) and np.array_equal(l64[:, 2], l64[:, 7])
    distinct = -np.sort(-l64[:, [0, 1, 2, 3, 4, 6]], axis=1)
    ok = (distinct[:, 0] - distinct[:, 1] > 1e-3) & (distinct[:, 1] - distinct[:, 2] > 1e-3)
    ref = O.topk_select(l64, 2)
    got = idx.cpu().numpy()
    assert np.array_equal(got[ok], ref[ok])
    both = ok & (ref[:, 0] == 2) & (ref[:, 1] == 5)          # tie inside the selection
    cut = ok & (ref[:, 1] == 2)                              # tie straddles the cut
    assert both.any() and cut.any()
    assert not np.any(got[ok] == 7)


# ---------------------------------------------------------------- dispatch
def random_routing(T, E, K, seed, skew=None):
    g = torch.Generator().manual_seed(seed)
    if skew is not None:
        idx = torch.stack([torch.randperm(E, generator=g)[:K] for _ in range(T)]) if T else \
            torch.empty((0, K), dtype=torch.int64)
        idx[:, 0] = skew
        idx[:, 1:] = torch.where(idx[:, 1:] == skew, (skew + 1) % E, idx[:, 1:])
        if K > 2:
            return None
        return idx
    if T == 0:
        return torch.empty((0, K), dtype=torch.int64)
    scores = torch.rand((T, E), generator=g)
    return torch.argsort(scores, dim=1)[:, :K]


# pairs held in registers for 2048 < P <= 16384 and E <= 16 (4, 8 or 16
# rounds of 1024), streamed otherwise
@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (7, 8, 2), (1000, 8, 2), (5000, 8, 2),
                                   (333, 64, 4), (64, 1, 1), (129, 8, 8), (2048, 16, 1),
                                   (1500, 8, 2), (3000, 16, 2), (8192, 8, 2), (9000, 8, 2),
                                   (1100, 32, 3)])
def test_permute_bit_exact(dev, T, E, K):
    say("permute", T, E, K)
    idx = random_routing(T, E, K, seed=T * 131 + E * 7 + K)
    off, st, pos = M.moe_route_permute(idx.to(torch.int32).to(dev), E)
    torch.cuda.synchronize()
    counts, r_off, r_st, r_sr, r_pos = O.route_tables(idx.numpy(), E)
    assert off.cpu().numpy().tolist() == r_off.tolist()
    assert st.cpu().numpy().tolist() == r_st.tolist()
    assert pos.cpu().numpy().tolist() == r_pos.tolist()


def test_permute_all_to_one_expert(dev):
    say("permute skew")
    idx = random_routing(3000, 8, 2, seed=5, skew=3)
    off, st, pos = M.moe_route_permute(idx.to(torch.int32).to(dev), 8)
    torch.cuda.synchronize()
    _, r_off, r_st, _, r_pos = O.route_tables(idx.numpy(), 8)
    assert off.cpu().tolist() == r_off.tolist()
    assert st.cpu().tolist() == r_st.tolist() and pos.cpu().numpy().tolist() == r_pos.tolist()


# ---------------------------------------------------------------- layer
def test_layer_tiny_f32(dev):
    w = W.WORKLOADS["tiny_f32_T64"]
    say("layer", w.name)
    check_layer(W.layer_inputs(w, dev), w.K)


@pytest.mark.parametrize("T,d,d_ff", [(300, 256, 384), (24, 384, 256), (1, 256, 128),
                                      (129, 512, 640), (65, 128, 128), (700, 256, 256)])
def test_layer_bf16_small(dev, T, d, d_ff):
    w = small(T=T, d=d, d_ff=d_ff)
    say("layer bf16", T, d, d_ff)
    check_layer(W.layer_inputs(w, dev), w.K)


@pytest.mark.parametrize("T,d,d_ff", [(8, 2048, 1024), (3, 1024, 2048), (32, 512, 1536),
                                      (8, 1024, 512), (1, 1024, 1024), (5, 1024, 2560),
                                      (16, 768, 2048)])
def test_layer_bf16_streaming_splits(dev, T, d, d_ff):
    """Small batches take the weight-streaming kernels with K split over
    workgroups (partial sums added in split order)."""
    w = small(T=T, d=d, d_ff=d_ff)
    plan = M.plan_for(T, d, d_ff, w.E, w.K, M.BF16)
    say("layer streaming", T, d, d_ff, plan)
    assert plan["streaming"]
    check_layer(W.layer_inputs(w, dev), w.K)


@pytest.mark.parametrize("E,K", [(8, 1), (8, 8), (64, 4), (1, 1), (16, 3)])
def test_layer_bf16_k_and_e(dev, E, K):
    w = small(T=200, d=256, d_ff=256, E=E, K=K)
    say("layer E K", E, K)
    check_layer(W.layer_inputs(w, dev), K)


# decode-sized batches take the streaming kernels with any number of
# experts: with many, most experts hold no rows and the worst-case grid has a
# token tile per expert; with one or two, an expert's rows span several
# 16-row token tiles, each streaming the expert's weights
@pytest.mark.parametrize("T,d,d_ff,E,K", [(8, 512, 1024, 16, 3), (16, 512, 512, 64, 4),
                                          (5, 1024, 512, 64, 4), (21, 256, 1024, 16, 3),
                                          (40, 512, 1024, 1, 1), (32, 512, 512, 2, 2),
                                          (64, 256, 512, 1, 1)])
def test_layer_bf16_streaming_experts(dev, T, d, d_ff, E, K):
    w = small(T=T, d=d, d_ff=d_ff, E=E, K=K)
    plan = M.plan_for(T, d, d_ff, E, K, M.BF16)
    say("layer streaming E K", T, E, K, plan)
    assert plan["streaming"]
    check_layer(W.layer_inputs(w, dev), K)


def test_layer_f32_general_sizes(dev):
    w = small(T=77, d=96, d_ff=200, dtype="f32")
    say("layer f32 ragged", w.T, w.d, w.d_ff)
    check_layer(W.layer_inputs(w, dev), 2)


def test_layer_skewed_routing_prefill_recipe(dev):
    w = small(name="prefill_bf16_T4096_zipf", T=1500, d=256, d_ff=256)
    say("layer zipf small")
    check_layer(W.layer_inputs(w, dev), 2)


def test_empty_batch(dev):
    w = small(T=4, d=128, d_ff=128)
    inp = W.layer_inputs(w, dev)
    inp["x"] = inp["x"][:0]
    y, _ = run_forward(inp, 2)
    assert y.shape == (0, 128)


# (640, 256, 384): tiled; (8, 1024, 1024): per-matrix streaming W1/W3 +
# finish; (16, 768, 2048): fused streaming W1/W3
@pytest.mark.parametrize("T,d,d_ff", [(640, 256, 384), (8, 1024, 1024), (16, 768, 2048)])
def test_deterministic_and_stages_match_forward(dev, T, d, d_ff):
    w = small(T=T, d=d, d_ff=d_ff)
    say("determinism", T, d, d_ff, M.plan_for(T, d, d_ff, w.E, w.K, M.BF16))
    inp = W.layer_inputs(w, dev)
    y1, v1 = run_forward(inp, 2)
    y2, v2 = run_forward(inp, 2)
    assert torch.equal(y1, y2)
    for k in v1:
        if k != "scratch":
            assert torch.equal(v1[k], v2[k]), k
    idx, wt = M.moe_router_topk(inp["x"], inp["W_g"], 2)
    off, st, pos = M.moe_route_permute(idx, w.E)
    H = M.moe_expert_swiglu(inp["x"], inp["W1"], inp["W3"], 2, off, st)
    Ob = M.moe_expert_down(H, inp["W2"], w.T, 2, off)
    y3 = M.moe_combine(Ob, wt, pos)
    torch.cuda.synchronize()
    assert torch.equal(idx, v1["topk_idx"]) and torch.equal(wt, v1["topk_w"])
    assert torch.equal(off, v1["offsets"]) and torch.equal(st, v1["sorted_token"])
    assert torch.equal(pos, v1["pos"])
    assert torch.equal(y3, y1)
    assert torch.equal(H, v1["H"]) and torch.equal(Ob, v1["O"])


def test_scaling_w2_scales_output_exactly(dev):
    w = small(T=200, d=256, d_ff=256)
    inp = W.layer_inputs(w, dev)
    y, _ = run_forward(inp, 2)
    inp2 = dict(inp, W2=[2 * t for t in inp["W2"]])
    y2, _ = run_forward(inp2, 2)
    assert torch.equal(y2, 2 * y)


def test_accumulate_adds_residual_then_rounds(dev):
    w = small(T=100, d=256, d_ff=256)
    inp = W.layer_inputs(w, dev)
    y32, _ = run_forward(inp, 2)
    h = torch.randn((w.T, w.d), generator=torch.Generator(device=dev).manual_seed(3),
                    device=dev).to(torch.bfloat16)
    yacc = h.clone()
    run_forward(inp, 2, y_dtype=torch.bfloat16, y=yacc, accumulate=True)
    assert torch.equal(yacc, (h.float() + y32).to(torch.bfloat16))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm(dev, dtype):
    g = torch.Generator(device=dev).manual_seed(11)
    h = (torch.randn((33, 4096), generator=g, device=dev) * 3)
    h = h.to(torch.bfloat16) if dtype == "bf16" else h
    out = M.moe_rmsnorm(h)
    torch.cuda.synchronize()
    ref = O.rmsnorm(PY.to_np(h), 1e-5)
    err = np.abs(PY.to_np(out) - ref).max()
    assert err <= (2.0 ** -7 * np.abs(ref).max() if dtype == "bf16" else 1e-5)


# ---------------------------------------------------------------- full size
def _full(name, dev, tokens, check_perm_all=True):
    w = W.WORKLOADS[name] if isinstance(name, str) else name
    name = w.name
    say("full size", name)
    inp = W.layer_inputs(w, dev)
    y32, v = run_forward(inp, w.K)
    yb, _ = run_forward(inp, w.K, torch.bfloat16)
    assert torch.equal(yb, PY.bf16_rne_of(y32))
    # routing of every token (the router is cheap in float64)
    l64 = O.router_logits(PY.to_np(inp["x"]), PY.to_np(inp["W_g"]))
    ref_idx = O.topk_select(l64, w.K)
    set_ok = PY.check_routing(v["topk_idx"].cpu().numpy(), v["topk_w"].cpu().numpy(), ref_idx,
                              O.gate_weights(l64, ref_idx), l64, w.K)
    if check_perm_all:
        PY.check_permutation(v["offsets"].cpu().numpy(), v["sorted_token"].cpu().numpy(),
                             ref_idx, w.E, w.K, set_ok)
    rows = np.asarray(tokens)
    y_ref, aux = oracle(inp, w.K, faithful=True, tokens=rows)
    keep = set_ok[rows]
    err = PY.rel_err(PY.to_np(y32)[rows], y_ref, keep)
    say("%s: rel err %.3e over %d sampled tokens" % (name, err, keep.sum()))
    assert err <= PY.TOL_BF16
    y_exact, _ = oracle(inp, w.K, faithful=False, tokens=rows[:8])
    say("%s: rel err vs exact (reported) %.3e" % (name, PY.rel_err(PY.to_np(y32)[rows[:8]],
                                                                   y_exact, keep[:8])))


def test_full_decode_T8(dev):
    _full("decode_bf16_T8", dev, tokens=range(8))


@pytest.mark.parametrize("T", [1, 2, 4])
def test_full_decode_small_batches(dev, T):
    """Mixtral shape at 1, 2 and 4 tokens: the streaming plan takes the
    per-matrix W1/W3 form with 1 and 2 K splits and the fused form, and
    splits W2 7, 4 and 2 ways."""
    w = W.scaled(W.WORKLOADS["decode_bf16_T8"], name="decode_bf16_T%d" % T, T=T)
    plan = M.plan_for(w.T, w.d, w.d_ff, w.E, w.K, M.BF16)
    say("full decode", T, plan)
    assert plan["streaming"]
    _full(w, dev, tokens=range(T))


def test_tiled_operand_past_32_bit_offsets_takes_grouped_kernels(dev):
    """d_ff = 65536 at T = 16500 (K = 2) makes H 33000 rows x 128 KB: its byte
    offsets pass 2^32, beyond the tiled kernel's 32-bit lane offsets, so the
    W2 product goes to the grouped kernels.  Tokens whose sorted rows lie past
    that point are checked against the oracle."""
    w = small(T=16500, d=256, d_ff=65536)
    say("32-bit offset limit", w.T, w.d, w.d_ff, M.plan_for(w.T, w.d, w.d_ff, w.E, w.K, M.BF16))
    inp = W.layer_inputs(w, dev)
    _, v = run_forward(inp, w.K)
    pos = v["pos"].cpu().numpy()
    del v
    late = np.nonzero(pos.max(axis=1).astype(np.int64) * w.d_ff * 2 >= 2 ** 32)[0]
    assert late.size > 0
    tokens = np.concatenate([late[:: max(1, late.size // 8)][:8], [0, w.T - 1]])
    check_layer(inp, w.K, tokens=np.unique(tokens), bf16_store=False)


def test_full_T512_sampled(dev):
    _full("mid_bf16_T512", dev, tokens=np.random.default_rng(1).choice(512, 32, replace=False))


def test_full_prefill_T4096_sampled(dev):
    rng = np.random.default_rng(2)
    _full("prefill_bf16_T4096_zipf", dev, tokens=np.sort(rng.choice(4096, 32, replace=False)))


# ---------------------------------------------------------------- stack (pre-norm blocks)
def _stack_inputs(w, dev, layers):
    blocks = []
    for b in range(layers):
        W_g, W1s, W3s, W2s = W.expert_weights(w, dev, block=b)
        blocks.append((W_g, W1s, W3s, W2s))
    h0 = W.make_x(w, blocks[0][0], dev)
    return h0, blocks


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stack_small_vs_oracle(dev, dtype):
    """h <- h + MoE(RMSNorm(h)) over 4 blocks, tokens whose routing is decided
    at every block.  Reading of the per-layer bar for a stack: every block
    may move its own output by up to the layer tolerance (1e-2 of rms for
    bf16, 1e-4 for fp32) and the residual stream carries each block's
    deviation forward (RMSNorm is scale invariant, so nothing amplifies it),
    hence max|dh| <= L x tol x rms(h); the norm-wise error must stay within
    one layer's tolerance."""
    layers = 4
    tol = PY.TOL_BF16 if dtype == "bf16" else PY.TOL_F32
    w = small(name="stack32_bf16_T4096", T=200, d=256, d_ff=256, dtype=dtype)
    say("stack small", dtype)
    h0, blocks = _stack_inputs(w, dev, layers)
    h = h0.clone()
    M.moe_stack_forward(h, blocks, w.K)
    torch.cuda.synchronize()
    np_blocks = [(PY.to_np(Wg), LazyNp(W1), LazyNp(W3), LazyNp(W2)) for Wg, W1, W3, W2 in blocks]
    h_ref, margins = O.stack_forward(PY.to_np(h0), np_blocks, w.K, faithful=(dtype == "bf16"))
    ok = np.ones(w.T, dtype=bool)
    for m_rank, m_cut in margins:
        ok &= m_cut > PY.DECIDED_GAP
    assert ok.sum() > w.T // 2
    d = PY.to_np(h)[ok] - h_ref[ok]
    rms = np.sqrt(np.mean(h_ref[ok] ** 2))
    max_rel = np.abs(d).max() / rms
    l2_rel = np.sqrt(np.mean(d ** 2)) / rms
    say("stack small %s: max %.2e, l2 %.2e of rms over %d of %d tokens decided at every block"
        % (dtype, max_rel, l2_rel, ok.sum(), w.T))
    assert max_rel <= layers * tol and l2_rel <= tol


@pytest.mark.parametrize("T", [8, 300])
def test_stack_graph_replay_matches_eager(dev, T):
    """A whole stack step captured in one HIP graph: every replay, with eager
    work and synchronisations between replays, gives the eager result bit for
    bit (the library allocates and memsets nothing, so the captured step is
    only its kernels).  T = 8 takes the streaming kernels, T = 300 the tiled
    ping-pong ones."""
    w = small(name="stack32_bf16_T4096", T=T, d=256, d_ff=512, dtype="bf16")
    say("stack graph replay", T, M.plan_for(T, 256, 512, w.E, w.K, M.BF16))
    h0, blocks = _stack_inputs(w, dev, 3)
    ws = torch.empty(M.workspace_size(w.T, w.d, w.d_ff, w.E, w.K, M.BF16), dtype=torch.uint8,
                     device=dev)
    h = h0.clone()
    xn = torch.empty_like(h)
    M.moe_stack_forward(h, blocks, w.K, workspace=ws, xn=xn)
    torch.cuda.synchronize()
    eager = h.clone()
    g = torch.cuda.CUDAGraph()
    h.copy_(h0)
    with torch.cuda.graph(g):
        M.moe_stack_forward(h, blocks, w.K, workspace=ws, xn=xn)
    for rep in range(4):
        h.copy_(h0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, eager), "replay %d" % rep
        # eager work between replays that reuses the same workspace
        h.copy_(h0)
        M.moe_stack_forward(h, blocks[:1], w.K, workspace=ws, xn=xn)
        torch.cuda.synchronize()


def test_full_stack32_T4096(dev):
    """The 32-block stack at Mixtral shape (90 GB of expert weights): block 0
    against the oracle on sampled tokens, then all 32 blocks run; the result
    must be finite and its RMS must grow as residual sums do."""
    w = W.WORKLOADS["stack32_bf16_T4096"]
    say("full stack32")
    h0, blocks = _stack_inputs(w, dev, w.layers)
    h = h0.clone()
    M.moe_stack_forward(h, blocks[:1], w.K)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(w.T, 16, replace=False))
    Wg, W1, W3, W2 = blocks[0]
    xn_ref = O.rmsnorm(PY.to_np(h0)[rows], 1e-5, faithful=True)
    y_ref, aux = O.moe_forward(xn_ref, PY.to_np(Wg), LazyNp(W1), LazyNp(W3), LazyNp(W2), w.K,
                               faithful=True)
    h1_ref = O.bf16_round(PY.to_np(h0)[rows] + y_ref)
    ok = O.routing_margins(aux["logits"], w.K)[1] > PY.DECIDED_GAP
    diff = np.abs(PY.to_np(h)[rows] - h1_ref)[ok]
    rms = np.sqrt(np.mean(h1_ref ** 2))
    say("stack32 block 0: max diff/rms %.2e over %d decided of 16" % (diff.max() / rms, ok.sum()))
    assert np.all(diff <= 1e-2 * rms + 2.0 ** -8 * np.abs(h1_ref[ok]))
    rms1 = h.float().pow(2).mean().sqrt().item()
    M.moe_stack_forward(h, blocks[1:], w.K)
    torch.cuda.synchronize()
    assert torch.isfinite(h.float()).all()
    rms32 = h.float().pow(2).mean().sqrt().item()
    say("stack32 rms h0 %.3f, h1 %.3f, h32 %.3f" % (h0.float().pow(2).mean().sqrt().item(), rms1,
                                                    rms32))
    assert rms32 > rms1
