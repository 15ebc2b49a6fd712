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
        # exact upcast on the device, one copy of float64 to the host
        return self.ts[e].detach().double().cpu().numpy()


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


@pytest.mark.parametrize("T,E,K,splits", [(37, 4, 2, 1), (1500, 8, 2, 2)])
def test_dropped_pairs_add_nothing(dev, T, E, K, splits):
    """Expert indices outside [0, E) (written by the router only for
    non-finite logits) are dropped: the dispatch leaves them out of every
    segment and gives them pos = -1, and the combine adds nothing for them.
    T = 37 takes the streaming dispatch, T = 1500 (3000 pairs) the held one."""
    say("dropped pairs", T, E, K, splits)
    idx = random_routing(T, E, K, seed=T + 17)
    planted = [(3, K - 1, E), (10, 0, -1), (20, 0, E + 2), (20, K - 1, -7), (T - 1, 0, 1 << 20)]
    for t, r, v in planted:
        idx[t, r] = v
    off, st, pos = M.moe_route_permute(idx.to(torch.int32).to(dev), E)
    torch.cuda.synchronize()
    idx_np = idx.numpy()
    kept = [(p // K, p % K) for p in range(T * K) if 0 <= idx_np[p // K, p % K] < E]
    order = sorted(range(len(kept)), key=lambda i: idx_np[kept[i]])     # stable
    ref_off = np.zeros(E + 1, dtype=np.int64)
    for t, r in kept:
        ref_off[idx_np[t, r] + 1] += 1
    ref_off = np.cumsum(ref_off)
    ref_pos = np.full((T, K), -1, dtype=np.int64)
    for dest, i in enumerate(order):
        ref_pos[kept[i]] = dest
    assert off.cpu().numpy().tolist() == ref_off.tolist()
    assert st.cpu().numpy()[:len(kept)].tolist() == [kept[i][0] for i in order]
    assert pos.cpu().numpy().tolist() == ref_pos.tolist()
    # combine: a dropped pair contributes exactly what a kept pair of weight
    # zero would (s = w0*o0, then s = fma(w, o, s), and fma(0, o, s) = s)
    g = torch.Generator(device="cpu").manual_seed(T)
    O_ = torch.randn((splits, T * K, 256), generator=g).to(dev)
    wts = torch.rand((T, K), generator=g).to(dev)
    y_drop = M.moe_combine(O_, wts, pos)
    dropped = pos < 0
    y_zero = M.moe_combine(O_, torch.where(dropped, torch.zeros_like(wts), wts),
                           torch.where(dropped, torch.zeros_like(pos), pos))
    h = torch.randn((T, 256), generator=g).to(dev).to(torch.bfloat16)
    h_drop = M.moe_combine(O_, wts, pos, y=h.clone(), accumulate=True)
    h_zero = M.moe_combine(O_, torch.where(dropped, torch.zeros_like(wts), wts),
                           torch.where(dropped, torch.zeros_like(pos), pos), y=h.clone(),
                           accumulate=True)
    torch.cuda.synchronize()
    assert torch.isfinite(y_drop).all()
    assert torch.equal(y_drop, y_zero) and torch.equal(h_drop, h_zero)
    assert torch.all(y_drop[20] == 0)                  # both of token 20's pairs dropped


@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (2, 8, 2), (37, 4, 2), (5000, 8, 2),
                                   (70000, 8, 1), (3000, 64, 4)])
def test_routing_stats_bit_exact(dev, T, E, K):
    """Expert loads and first-choice repeats of consecutive tokens, on
    routings with planted same-expert runs and out-of-range entries."""
    say("routing stats", T, E, K)
    idx = random_routing(T, E, K, seed=T * 7 + E + K)
    g = torch.Generator().manual_seed(T + 1)
    run = torch.rand(T, generator=g) < 0.4            # token repeats its predecessor's row
    for t in range(1, T):
        if run[t]:
            idx[t] = idx[t - 1]
    if T > 3:
        idx[T // 2, 0] = -1
        idx[T // 3, K - 1] = E
    counts, repeats = M.moe_routing_stats(idx.to(torch.int32).to(dev), E)
    torch.cuda.synchronize()
    r_counts, r_repeats = O.routing_stats(idx.numpy(), E)
    assert counts.cpu().numpy().tolist() == r_counts.tolist()
    assert int(repeats.item()) == r_repeats


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


@pytest.mark.parametrize("T,d,d_ff", [(300, 320, 448), (24, 256, 320), (200, 192, 512),
                                      (1, 64, 64)])
def test_layer_bf16_multiples_of_64(dev, T, d, d_ff):
    """bf16 shapes that are multiples of 64 but not of 128 (d or d_ff) take
    the general grouped kernels: 128-column W1/W3 tiles when d_ff is an odd
    multiple of 64, 64-column W2 tiles when d is."""
    w = small(T=T, d=d, d_ff=d_ff)
    plan = M.plan_for(T, d, d_ff, w.E, w.K, M.BF16)
    say("layer bf16 multiples of 64", T, d, d_ff, plan)
    assert not plan["streaming"] and plan["down_splits"] == 1
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


@pytest.mark.parametrize("T,d,d_ff,units_past_grid", [(8, 2048, 4608, True),
                                                      (7, 2048, 4608, True),
                                                      (8, 4096, 9216, True),
                                                      (8, 1024, 4608, True),
                                                      (8, 1024, 3072, False)])
def test_layer_bf16_streaming_persistent_grid(dev, T, d, d_ff, units_past_grid):
    """The per-matrix W1/W3 product over its persistent grid of 224
    workgroups.  When the units (busy token tile, 256 features, matrix)
    outnumber the workgroups, every workgroup takes the same number of
    256-row chunks (to one), so units are cut at workgroup boundaries and
    their head and tail partial sums are added by the finish (units of 8, 16
    and 4 chunks); with fewer units (at most 192 at d_ff = 3072) each is cut
    into the same number of pieces."""
    w = small(T=T, d=d, d_ff=d_ff)
    plan = M.plan_for(T, d, d_ff, w.E, w.K, M.BF16)
    say("layer streaming persistent", T, d, d_ff, plan)
    assert plan["streaming"] and plan["swiglu_splits"] > 0
    y32, v, _ = check_layer(W.layer_inputs(w, dev), w.K)
    units = int(((v["offsets"].diff() + 15) // 16).sum().item()) * (d_ff // 256) * 2
    assert (units >= 224) == units_past_grid, units


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
# finish; (16, 768, 2048): fused streaming W1/W3; (130, 49152, 1024) over 3
# experts: tiled W2 with its last round of tiles split along K (576 tiles)
@pytest.mark.parametrize("T,d,d_ff,E", [(640, 256, 384, 8), (8, 1024, 1024, 8),
                                        (16, 768, 2048, 8), (130, 49152, 1024, 3)])
def test_deterministic_and_stages_match_forward(dev, T, d, d_ff, E):
    w = small(T=T, d=d, d_ff=d_ff, E=E)
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


def test_w2_split_tail_every_row(dev):
    """A W2 product of at least one whole round of tiles.  d = 49152 gives 192
    feature tiles of 256 columns; 130 tokens top-2 over 3 experts fill 3
    token tiles (at most 130 rows each), 576 tiles in all: 512 run over the
    whole of K, and the 64 of the last, partial round are cut into 4 K pieces
    whose sums the fix-up adds.  Every token is checked against the oracle."""
    w = small(T=130, d=49152, d_ff=1024, E=3)
    plan = M.plan_for(w.T, w.d, w.d_ff, w.E, w.K, M.BF16)
    say("W2 split tail", w.T, w.d, w.d_ff, w.E, plan)
    assert not plan["streaming"] and plan["down_splits"] == 1 and plan["down_scratch_bytes"] > 0
    inp = W.layer_inputs(w, dev)
    _, v = run_forward(inp, w.K)
    counts = np.diff(v["offsets"].cpu().numpy())
    tiles = int(np.sum((counts + 255) // 256)) * (w.d // 256)
    say("expert rows", counts.tolist(), "tiles", tiles)
    assert tiles % 256 != 0 and tiles > 256           # a whole round and a split tail
    del v
    check_layer(inp, w.K)


@pytest.mark.parametrize("counts", [(0, 1, 128, 129, 256, 257, 100, 153),
                                    (512, 0, 0, 0, 0, 0, 0, 512),
                                    (128,) * 8])
def test_tile_shape_per_expert_boundaries(dev, counts):
    """The W1/W3 product with a tile shape per expert (128 x 512 tiles for
    experts of at most 128 rows, 256 x 256 otherwise) and the K-split W2
    product, on routing built by hand: experts of 0, 1, 128, 129, 256 and 257 rows; only
    256-row tiles; only the wide shape.  Token i takes the experts of entries
    i and i + T of the sorted label list (distinct, since no expert holds T
    or more pairs).  Each expert's output rows (the W2 slices summed) are
    compared with the oracle's expert on the same token rows."""
    E, K = len(counts), 2
    P = sum(counts)
    T = P // K
    w = small(T=T, d=512, d_ff=512, E=E)
    plan = M.plan_for(T, w.d, w.d_ff, E, K, M.BF16)
    say("tile shape per expert", counts, plan)
    assert plan["swiglu_mixed"] and not plan["streaming"]
    labels = np.repeat(np.arange(E), counts)
    idx_np = np.stack([labels[:T], labels[T:]], axis=1).astype(np.int32)
    assert np.all(idx_np[:, 0] != idx_np[:, 1])
    inp = W.layer_inputs(w, dev)
    off, st, pos = M.moe_route_permute(torch.from_numpy(idx_np).to(dev), E)
    H = M.moe_expert_swiglu(inp["x"], inp["W1"], inp["W3"], K, off, st)
    Ob = M.moe_expert_down(H, inp["W2"], T, K, off)
    torch.cuda.synchronize()
    r_counts, r_off, r_st, _, r_pos = O.route_tables(idx_np, E)
    assert off.cpu().numpy().tolist() == list(r_off)
    assert st.cpu().numpy().tolist() == list(r_st)
    o_sum = PY.to_np(Ob).sum(axis=0)     # [splits, P, d]: the slices' sum
    x = PY.to_np(inp["x"])
    W1s, W3s, W2s = LazyNp(inp["W1"]), LazyNp(inp["W3"]), LazyNp(inp["W2"])
    for e in range(E):
        lo, hi = int(r_off[e]), int(r_off[e + 1])
        if lo == hi:
            continue
        ref = O.swiglu_expert(x[r_st[lo:hi]], W1s[e], W3s[e], W2s[e], faithful=True)
        err = PY.rel_err(o_sum[lo:hi], ref)
        say("expert %d: %d rows, rel err %.3e" % (e, hi - lo, err))
        assert err <= PY.TOL_BF16, e


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


def _stack_layerwise(blocks, stacks, K, tol, faithful, label):
    """Block-by-block parity of pre-norm stacks, h <- h + MoE(RMSNorm(h))
    ("【DL輪読会】Mixtral of Experts" slides, "Architecture – 全体").

    ``stacks`` maps a name to (h0 on the GPU, rows to compare).  For every
    block l and stack, the GPU's block input h_l (bf16 or fp32) goes to the
    oracle's RMSNorm, and the GPU's normalised rows must be within one
    rounding of the oracle's (the fp32 and float64 normalisations may round
    an element to neighbouring bf16 values).  The GPU's normalised rows then
    go to the oracle's MoE of block l (the block's weights as the GPU holds
    them, upcast exactly), and the GPU's fp32 MoE output of the block must
    match it on the sampled rows whose routing is decided: expert sets, gate
    weights and outputs at the layer tolerances.
    The stack step (moe_stack_forward over that one block) must equal
    round(h_l + y_l) of that output bit for bit, and the whole stack run in
    one call must equal the block-by-block result bit for bit, and the
    per-block statistics it reports must hold each block's expert loads.
    Returns the per-block errors of every stack."""
    hs = {name: h0.clone() for name, (h0, _) in stacks.items()}
    errs = {name: [] for name in stacks}
    block_loads = {name: [] for name in stacks}
    for l, (Wg, W1, W3, W2) in enumerate(blocks):
        h_in, y_gpu, xn_gpu, gidx, gw, split = [], [], [], [], [], {}
        for name, (_, rows) in stacks.items():
            h = hs[name]
            sel = torch.as_tensor(rows, device=h.device)
            h_in.append(PY.to_np(h[sel]))
            xn = M.moe_rmsnorm(h)
            y32, v = run_forward(dict(x=xn, W_g=Wg, W1=W1, W3=W3, W2=W2), K)
            expect = (h.float() + y32).to(h.dtype)
            M.moe_stack_forward(h, [(Wg, W1, W3, W2)], K)
            torch.cuda.synchronize()
            assert torch.equal(h, expect), (label, name, l)
            split[name] = (sum(len(a) for a in y_gpu), len(rows))
            y_gpu.append(PY.to_np(y32[sel]))
            xn_gpu.append(PY.to_np(xn[sel]))
            block_loads[name].append(v["offsets"].diff().cpu().numpy().tolist())
            gidx.append(v["topk_idx"][sel].cpu().numpy())
            gw.append(v["topk_w"][sel].cpu().numpy())
            del v
        x_ref = O.rmsnorm(np.concatenate(h_in), 1e-5, faithful=faithful)
        xn_g = np.concatenate(xn_gpu)
        rel = 2.0 ** -7 if faithful else 1e-6
        assert np.all(np.abs(xn_g - x_ref) <= rel * np.abs(x_ref) + 1e-30), (label, l)
        y_ref, aux = O.moe_forward(xn_g, PY.to_np(Wg), LazyNp(W1), LazyNp(W3), LazyNp(W2), K,
                                   faithful=faithful)
        ok = PY.check_routing(np.concatenate(gidx), np.concatenate(gw), aux["idx"], aux["w"],
                              aux["logits"], K)
        y_g = np.concatenate(y_gpu)
        line = []
        for name, (a, n) in split.items():
            sl = slice(a, a + n)
            err = PY.rel_err(y_g[sl], y_ref[sl], ok[sl])
            errs[name].append(err)
            line.append("%s %.2e (%d/%d decided)" % (name, err, ok[sl].sum(), n))
            assert err <= tol, (label, name, l, err)
        say("%s block %d: %s" % (label, l, ", ".join(line)))
    for name, (h0, _) in stacks.items():
        h = h0.clone()
        E = len(blocks[0][1])
        stats = torch.full((len(blocks), E + 1), -1, dtype=torch.int32, device=h.device)
        M.moe_stack_forward(h, blocks, K, stats=stats)
        torch.cuda.synchronize()
        assert torch.equal(h, hs[name]), (label, name, "whole stack in one call")
        st = stats.cpu().numpy()
        T = h.shape[0]
        assert np.all(st[:, :E].sum(axis=1) == T * K) and np.all(st[:, E] >= 0)
        assert np.all(st[:, E] <= max(T - 1, 0))
        assert st[:, :E].tolist() == block_loads[name]
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stack_small_layerwise(dev, dtype):
    """Four blocks, 200 tokens (tiled plan for bf16) and the first 8 of them
    (streaming plan), every token compared at every block."""
    w = small(name="stack32_bf16_T4096", T=200, d=256, d_ff=256, dtype=dtype)
    say("stack small", dtype)
    h0, blocks = _stack_inputs(w, dev, 4)
    stacks = {"T200": (h0, np.arange(200)), "T8": (h0[:8].clone(), np.arange(8))}
    tol = PY.TOL_BF16 if dtype == "bf16" else PY.TOL_F32
    errs = _stack_layerwise(blocks, stacks, w.K, tol, dtype == "bf16", "stack small " + dtype)
    say("stack small %s: max per-block error %.2e" % (dtype, max(max(e) for e in errs.values())))


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
    ws = torch.empty(M.stack_workspace_size(w.T, w.d, w.d_ff, w.E, w.K, M.BF16),
                     dtype=torch.uint8, device=dev)
    h = h0.clone()
    M.moe_stack_forward(h, blocks, w.K, workspace=ws)
    torch.cuda.synchronize()
    eager = h.clone()
    g = torch.cuda.CUDAGraph()
    h.copy_(h0)
    with torch.cuda.graph(g):
        M.moe_stack_forward(h, blocks, w.K, workspace=ws)
    for rep in range(4):
        h.copy_(h0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, eager), "replay %d" % rep
        # eager work between replays that reuses the same workspace
        h.copy_(h0)
        M.moe_stack_forward(h, blocks[:1], w.K, workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("E,K,T,d,d_ff", [(6, 2, 8, 512, 256), (16, 4, 8, 512, 256),
                                          (8, 2, 1, 512, 256), (8, 2, 2, 4096, 14336),
                                          (8, 2, 4, 4096, 14336), (8, 2, 8, 4096, 14336),
                                          (8, 2, 1100, 512, 256), (8, 3, 700, 384, 256)])
def test_stack_glue_and_separate_launches_agree(dev, E, K, T, d, d_ff):
    """The stack joins small-batch blocks with one glue launch when it can
    (8 | E); otherwise the previous block's combine and the RMSNorm share one
    launch and the router follows (E = 6, and the tiled batches of 700 and
    1100 tokens, the latter with the many-token router).  Either way the
    stack equals moe_rmsnorm + moe_forward(accumulate) block by block, bit
    for bit.  The Mixtral-shape cases give the W2 product 4 and 2 slices (the
    glue's all-loads-first combine); K = 4, K = 3 and 7 slices (T = 1) take
    its general loop."""
    w = small(name="stack32_bf16_T4096", T=T, d=d, d_ff=d_ff, E=E, K=K)
    say("stack glue", E, K, T, d, d_ff, M.plan_for(T, d, d_ff, E, K, M.BF16))
    h0, blocks = _stack_inputs(w, dev, 3)
    h = h0.clone()
    for blk in blocks:
        xn = M.moe_rmsnorm(h)
        M.moe_forward(xn, *blk, K, y=h, accumulate=True)
    ref = h.clone()
    h = h0.clone()
    M.moe_stack_forward(h, blocks, K)
    torch.cuda.synchronize()
    assert torch.equal(h, ref)


@pytest.mark.timeout(900)
def test_full_stack32_layerwise(dev):
    """The 32-block stack at Mixtral shape (90 GB of expert weights), block by
    block against the oracle: the prefill stack of 4096 tokens (tiled
    kernels) on 16 sampled tokens and the decode stack of 8 tokens
    (streaming kernels) on all of them, at every one of the 32 blocks."""
    w = W.WORKLOADS["stack32_bf16_T4096"]
    say("full stack32 layerwise")
    h0, blocks = _stack_inputs(w, dev, w.layers)
    rows = np.sort(np.random.default_rng(5).choice(w.T, 16, replace=False))
    h8 = W.make_x(w, blocks[0][0], dev, T=8)
    stacks = {"T4096": (h0, rows), "T8": (h8, np.arange(8))}
    errs = _stack_layerwise(blocks, stacks, w.K, PY.TOL_BF16, True, "stack32")
    for name, e in errs.items():
        say("stack32 %s: per-block error max %.2e, median %.2e" % (name, max(e), np.median(e)))
