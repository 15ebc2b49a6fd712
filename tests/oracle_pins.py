"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` raises AssertionError on failure.  They are collected as
tests by ``test_oracle_pins.py`` and re-run against deliberately broken copies
of the oracle by ``test_oracle_mutations.py`` (a planted mistake must make at
least one check fail).

Sources of the pinned facts (page title, section):

* "从Mistral 7B到MoE模型Mixtral 8x7B的全面解析：从原理分析到代码解读"
  (aiqianji.com blog), *Mixtral 全面解析* below: section 2.1.1 (gate and sum
  equations, TopK rule), section 2.1.2 (46.7B total / 12.9B active
  parameters), section 3.2.1 code block A (printed routing weights), sections
  3.2.2-3.2.3 code blocks B and C (one expert's dispatch), code block D (the
  SwiGLU expert), section 3.2.5 code block E (zero-initialised accumulator).
* "【DL輪読会】Mixtral of Experts" (docswell slides), slide
  "Architecture – Mixture of Experts (Router)": logits 1.4 and 0.7 give the
  printed top-2 weights 0.7 and 0.3 (one decimal).
* "MistralAI开源全球首个..." part 04 of the zikao35.com blog: checkpoint size
  86.99 GB.
"""

from __future__ import annotations

import math
import os

import numpy as np

from oracle import moe_oracle as O
from oracle import scalar as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def tiny_layer(seed, T=6, d=5, d_ff=7, E=4, scale_w2=1.0):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    W_g = r.standard_normal((d, E))
    W1s = [r.standard_normal((d, d_ff)) / math.sqrt(d) for _ in range(E)]
    W3s = [r.standard_normal((d, d_ff)) / math.sqrt(d) for _ in range(E)]
    W2s = [scale_w2 * r.standard_normal((d_ff, d)) / math.sqrt(d_ff) for _ in range(E)]
    return x, W_g, W1s, W3s, W2s


def read_golden_block_a():
    rows = []
    with open(os.path.join(GOLDEN, "routing_weights_code_block_a.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return np.array(rows)


def read_golden_blocks_bc():
    out = {}
    with open(os.path.join(GOLDEN, "dispatch_code_blocks_bc.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                out[key] = [int(v) for v in vals]
    return out


# --- bfloat16 rounding ------------------------------------------------------
def check_bf16_round_hand_cases():
    # spacing of bf16 just above 1.0 is 2**-7
    cases = {
        1.0: 1.0,
        1.0 + 2.0 ** -8: 1.0,                       # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,       # tie -> even (mantissa ...10)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,  # above the tie -> up
        -(1.0 + 2.0 ** -8 + 2.0 ** -20): -(1.0 + 2.0 ** -7),
        3.0: 3.0,
        0.1: 0.10009765625,                          # 0x3DCD
        float.fromhex("0x1.fep127"): float.fromhex("0x1.fep127"),
        float.fromhex("0x1.ffp127"): math.inf,       # rounds past the largest finite
        2.0 ** -130 * 1.3: 2.0 ** -133 * round(1.3 * 8),   # subnormal quantum 2**-133
        0.0: 0.0,
    }
    for a, want in cases.items():
        got = float(O.bf16_round(np.array([a]))[0])
        assert got == want, (a, got, want)


def check_bf16_round_vs_torch():
    """Library special case: for float32 inputs, torch's float32 -> bfloat16
    conversion is round-to-nearest-even, the same function."""
    import torch
    r = _rng(1)
    v = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-8, 8, 20000),
                        r.standard_normal(2000)]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = O.bf16_round(v.astype(np.float64))
    assert np.array_equal(got, want)


# --- router -------------------------------------------------------------------
def check_router_logits_worked_example():
    # x = (1, 2, 3), W_g columns (1,0,1) and (0,1,1) -> l = (4, 5), by hand
    x = np.array([[1.0, 2.0, 3.0]])
    W_g = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    assert np.array_equal(O.router_logits(x, W_g), np.array([[4.0, 5.0]]))
    # a unit token picks out one row of W_g
    r = _rng(2)
    W_g = r.standard_normal((6, 3))
    x = np.zeros((1, 6))
    x[0, 4] = 1.0
    assert np.array_equal(O.router_logits(x, W_g)[0], W_g[4])


def check_topk_hand_cases():
    l = np.array([[1.0, 3.0, 3.0, 2.0]])
    assert O.topk_select(l, 1).tolist() == [[1]]
    assert O.topk_select(l, 2).tolist() == [[1, 2]]
    assert O.topk_select(l, 3).tolist() == [[1, 2, 3]]
    l = np.array([[0.5, 0.5, 0.5, 0.5]])
    assert O.topk_select(l, 2).tolist() == [[0, 1]]
    l = np.array([[-1.0, 7.0, -3.0, 7.5, 0.0]])
    assert O.topk_select(l, 2).tolist() == [[3, 1]]


def check_topk_vs_bruteforce():
    """Brute force over all K-subsets (scalar oracle) on logits drawn from a
    small set of values, so that ties are frequent."""
    r = _rng(3)
    for trial in range(300):
        E = int(r.integers(2, 7))
        K = int(r.integers(1, E + 1))
        l = r.integers(-2, 3, E).astype(np.float64) * 0.5
        want = S.topk_bruteforce(list(l), K)
        got = O.topk_select(l[None, :], K)[0].tolist()
        assert got == want, (l, K, got, want)


def _logits_for_weights(w0, w1, E, perm):
    """Logits over E experts whose top-2 softmax is (w0, w1): l_top = 0,
    l_second = ln(w1 / w0), every other expert one unit below the second."""
    second = math.log(w1 / w0)
    l = np.full(E, second - 1.0)
    l[perm[0]] = 0.0
    l[perm[1]] = second
    return l


def check_gate_block_a():
    """Code block A: rows sum to 1 over exactly 2 experts, col0 >= 1/2 >=
    col1.  Rebuilding logits from each printed pair (others NOT at -inf) and
    re-gating must reproduce the printed weights, which only holds if the
    gate is a softmax over the selected two alone (renormalised)."""
    W = read_golden_block_a()
    assert W.shape == (16, 2)
    assert np.all(np.abs(W.sum(axis=1) - 1.0) <= 1e-4)
    assert np.all(W[:, 0] >= 0.5) and np.all(W[:, 1] <= 0.5)
    r = _rng(4)
    E = 8
    for w0, w1 in W:
        perm = r.permutation(E)
        l = _logits_for_weights(w0, w1, E, perm)[None, :]
        idx = O.topk_select(l, 2)
        assert idx[0].tolist() == [perm[0], perm[1]] or (w0 == w1)
        g = O.gate_weights(l, idx)[0]
        assert abs(g[0] - w0) <= 6e-5 and abs(g[1] - w1) <= 6e-5, (g, w0, w1)
        G = O.gate_dense(l, idx)[0]
        assert np.count_nonzero(G) == 2 and abs(G.sum() - 1.0) < 1e-15


def check_gate_closed_form():
    """For K = 2: w0 = 1 / (1 + e^D), w1 = e^D / (1 + e^D), D = l1 - l0 <= 0."""
    r = _rng(5)
    l = r.standard_normal((200, 8)) * 3
    idx = O.topk_select(l, 2)
    w = O.gate_weights(l, idx)
    D = np.take_along_axis(l, idx[:, 1:2], 1) - np.take_along_axis(l, idx[:, 0:1], 1)
    assert np.all(D <= 0)
    assert np.allclose(w[:, 0:1], 1 / (1 + np.exp(D)), rtol=0, atol=1e-15)
    assert np.allclose(w[:, 1:2], np.exp(D) / (1 + np.exp(D)), rtol=0, atol=1e-15)


def check_router_slide_figure():
    """Router slide: selected logits 1.4 and 0.7 are printed as weights 0.7
    and 0.3 (one decimal).  A weak sanity check, not a precise pin."""
    l = np.array([[1.4, 0.7, 0.3, 0.2, 0.1, 0.6, 0.1, 0.1]])
    idx = O.topk_select(l, 2)
    assert idx[0].tolist() == [0, 1]
    w = O.gate_weights(l, idx)[0]
    assert round(w[0], 1) == 0.7 and round(w[1], 1) == 0.3


# --- dispatch tables ----------------------------------------------------------
def check_dispatch_blocks_bc():
    g = read_golden_blocks_bc()
    T, K, E, e_star = 16, 2, 8, 5
    idx = np.zeros((T, K), dtype=np.int64)
    others = [e for e in range(E) if e != e_star]
    for t in range(T):           # two distinct non-target experts per token
        idx[t] = [others[t % 7], others[(t + 3) % 7]]
    for r_, row in ((0, g["mask_rank0"]), (1, g["mask_rank1"])):
        for t, on in enumerate(row):
            if on:
                idx[t, r_] = e_star
    counts, offsets, st, sr, pos = O.route_tables(idx, E)
    seg = slice(offsets[e_star], offsets[e_star + 1])
    assert st[seg].tolist() == g["top_x"]
    assert sr[seg].tolist() == g["idx"]
    assert counts[e_star] == 3


def check_dispatch_invariants():
    """Counting-sort invariants, and each segment equals the expert's pairs
    listed in pair order by numpy's nonzero (an independent method)."""
    r = _rng(6)
    for trial in range(40):
        T = int(r.integers(0, 40))
        E = int(r.integers(1, 10))
        K = int(r.integers(1, E + 1))
        idx = np.array([r.permutation(E)[:K] for _ in range(T)], dtype=np.int64).reshape(T, K)
        counts, offsets, st, sr, pos = O.route_tables(idx, E)
        assert counts.sum() == T * K and offsets[0] == 0 and offsets[-1] == T * K
        assert np.all(np.diff(offsets) == counts)
        flat = idx.reshape(-1)
        for e in range(E):
            pairs = np.nonzero(flat == e)[0]
            seg = slice(offsets[e], offsets[e + 1])
            assert st[seg].tolist() == (pairs // K).tolist()
            assert sr[seg].tolist() == (pairs % K).tolist()
            assert np.all(np.diff(st[seg]) > 0)
        assert sorted(pos.reshape(-1).tolist()) == list(range(T * K))
        for t in range(T):
            for k in range(K):
                assert st[pos[t, k]] == t and sr[pos[t, k]] == k


# --- expert -----------------------------------------------------------------
SIGMOID_2 = 0.88079707797788244    # 1 / (1 + e^-2), table value
SIGMOID_3 = 0.95257412682243322    # 1 / (1 + e^-3), table value


def check_silu_closed_forms():
    z = np.array([0.0, 2.0, 3.0, -2.0, 40.0, -40.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 2 * SIGMOID_2) < 1e-15 and abs(s[2] - 3 * SIGMOID_3) < 1e-15
    assert abs(s[3] - (-2) * (1 - SIGMOID_2)) < 1e-15
    assert abs(s[4] - 40.0) < 1e-15 and abs(s[5]) < 1e-15
    r = _rng(7)
    v = r.standard_normal(100) * 5
    assert np.allclose(O.silu(v) - O.silu(-v), v, rtol=0, atol=1e-13)


def check_swiglu_branch_order():
    """1x1 expert: x = 1, W1 = 2, W3 = 3, W2 = 1 gives SiLU(2) * 3, while the
    branches swapped would give SiLU(3) * 2 (code block D gates w1)."""
    out = O.swiglu_expert(np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]),
                          np.array([[1.0]]))
    assert abs(out[0, 0] - 3 * 2 * SIGMOID_2) < 1e-14
    assert abs(out[0, 0] - 2 * 3 * SIGMOID_3) > 0.4
    # an output projection with two columns keeps them apart: W2 = [[1, -2]]
    out = O.swiglu_expert(np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]),
                          np.array([[1.0, -2.0]]))
    assert np.allclose(out, [[6 * SIGMOID_2, -12 * SIGMOID_2]], rtol=0, atol=1e-14)


def check_swiglu_hand_matrix():
    """d = 2, d_ff = 2 by hand: x = (1, -1), W1 = [[1, 0], [0, 2]],
    W3 = [[1, 1], [1, -1]], W2 = [[1, 0], [0, 1]] -> a = (1, -2), b = (0, 2),
    h = (0, SiLU(-2) * 2), y = h."""
    x = np.array([[1.0, -1.0]])
    W1 = np.array([[1.0, 0.0], [0.0, 2.0]])
    W3 = np.array([[1.0, 1.0], [1.0, -1.0]])
    W2 = np.eye(2)
    out = O.swiglu_expert(x, W1, W3, W2)
    want = np.array([[0.0, 2 * (-2) * (1 - SIGMOID_2)]])
    assert np.allclose(out, want, rtol=0, atol=1e-14)


# --- whole layer --------------------------------------------------------------
def check_scalar_vs_numpy():
    """Two independent writings of the definition (sum over all experts with
    dense gates, brute-force TopK) agree on tiny random layers."""
    for seed in range(4):
        x, W_g, W1s, W3s, W2s = tiny_layer(100 + seed, T=5, d=4, d_ff=6, E=5)
        for K in (1, 2, 3, 5):
            y, aux = O.moe_forward(x, W_g, W1s, W3s, W2s, K)
            ys, sel, _ = S.layer(x.tolist(), W_g.tolist(), [w.tolist() for w in W1s],
                                 [w.tolist() for w in W3s], [w.tolist() for w in W2s], K)
            assert np.allclose(y, np.array(ys), rtol=0, atol=1e-12)
            assert aux["idx"].tolist() == sel


def check_k_equals_e_dense():
    x, W_g, W1s, W3s, W2s = tiny_layer(8, T=7, d=6, d_ff=5, E=5)
    y, _ = O.moe_forward(x, W_g, W1s, W3s, W2s, K=5)
    assert np.allclose(y, O.dense_mixture(x, W_g, W1s, W3s, W2s), rtol=0, atol=1e-12)


def check_one_hot_router():
    x, W_g, W1s, W3s, W2s = tiny_layer(9, T=5, d=6, d_ff=5, E=4)
    j = 2
    single = O.swiglu_expert(x, W1s[j], W3s[j], W2s[j])
    y1, aux = O.moe_forward(x, W_g, W1s, W3s, W2s, K=1)
    sel = aux["idx"][:, 0]
    for t in range(x.shape[0]):
        one = O.swiglu_expert(x[t:t + 1], W1s[sel[t]], W3s[sel[t]], W2s[sel[t]])[0]
        assert np.allclose(y1[t], one, rtol=1e-14, atol=1e-15)
    # K = 2 with a 60-unit margin towards expert j: the second expert weighs e^-60
    W_g2 = np.zeros_like(W_g)
    x2 = x.copy()
    x2[:, 0] = 1.0
    W_g2[0, j] = 60.0
    W_g2[0, (j + 1) % 4] = 0.0
    y2, aux2 = O.moe_forward(x2, W_g2, W1s, W3s, W2s, K=2)
    single2 = O.swiglu_expert(x2, W1s[j], W3s[j], W2s[j])
    assert np.all(aux2["idx"][:, 0] == j)
    assert np.allclose(y2, single2, rtol=1e-14, atol=1e-24)
    del single


def check_identical_experts():
    x, W_g, W1s, W3s, W2s = tiny_layer(10, T=9, d=6, d_ff=5, E=6)
    W1s = [W1s[0]] * 6
    W3s = [W3s[0]] * 6
    W2s = [W2s[0]] * 6
    single = O.swiglu_expert(x, W1s[0], W3s[0], W2s[0])
    for K in (1, 2, 4):
        y, _ = O.moe_forward(x, W_g, W1s, W3s, W2s, K)
        assert np.allclose(y, single, rtol=0, atol=1e-13)


def check_zero_init_block_e():
    """Code block E: the accumulator starts at zero and only routed pairs are
    added.  With every expert but j producing zeros, tokens that did not pick
    j come out exactly zero, the others not."""
    x, W_g, W1s, W3s, W2s = tiny_layer(11, T=12, d=6, d_ff=5, E=5)
    j = 3
    W2s = [w if e == j else np.zeros_like(w) for e, w in enumerate(W2s)]
    y, aux = O.moe_forward(x, W_g, W1s, W3s, W2s, K=2)
    routed = np.any(aux["idx"] == j, axis=1)
    assert routed.any() and (~routed).any()
    assert np.all(y[~routed] == 0.0)
    assert np.all(np.abs(y[routed]).max(axis=1) > 0)


def check_scaling_and_relabelling():
    x, W_g, W1s, W3s, W2s = tiny_layer(12, T=10, d=6, d_ff=5, E=5)
    y, aux = O.moe_forward(x, W_g, W1s, W3s, W2s, K=2)
    y2, _ = O.moe_forward(x, W_g, W1s, W3s, [2 * w for w in W2s], K=2)
    assert np.array_equal(y2, 2 * y)
    perm = np.array([3, 0, 4, 1, 2])          # new expert e' = old perm[e']
    inv = np.argsort(perm)
    yp, auxp = O.moe_forward(x, W_g[:, perm], [W1s[p] for p in perm], [W3s[p] for p in perm],
                             [W2s[p] for p in perm], K=2)
    assert np.allclose(yp, y, rtol=0, atol=1e-14)
    assert np.array_equal(perm[auxp["idx"]], aux["idx"])
    del inv
    tperm = _rng(13).permutation(x.shape[0])
    yt, _ = O.moe_forward(x[tperm], W_g, W1s, W3s, W2s, K=2)
    assert np.array_equal(yt, y[tperm])


def check_faithful_close_to_exact():
    x, W_g, W1s, W3s, W2s = tiny_layer(14, T=16, d=32, d_ff=48, E=4)
    ye, _ = O.moe_forward(x, W_g, W1s, W3s, W2s, K=2)
    yf, _ = O.moe_forward(x, W_g, W1s, W3s, W2s, K=2, faithful=True)
    rel = np.abs(yf - ye).max() / np.sqrt(np.mean(ye ** 2))
    assert 0 < rel < 2e-2


def _one_expert(W1, W3, W2):
    """One expert, so with K = 1 the gate weight is exactly 1 whatever the
    router says (softmax over a single selected logit)."""
    d = np.asarray(W1).shape[0]
    return np.zeros((d, 1)), [np.asarray(W1, float)], [np.asarray(W3, float)], \
        [np.asarray(W2, float)]


def check_faithful_rounds_h_hand():
    """Faithful mode rounds the SwiGLU product H to bfloat16 before the W2
    projection (code block D run in bfloat16 stores H in the activation
    dtype), and nothing else inside the expert.  Hand case, d = 1, d_ff = 2:
      x = [1]; W1 = [[64, 64]] so a = 64 and SiLU(64) = 64 / (1 + e^-64) = 64
      exactly in binary64 (e^-64 < 2^-53); W3 = [[(1 + 3 2^-9) / 64,
      (1 + 2^-9) / 64]] so H = [1 + 3 2^-9, 1 + 2^-9] exactly; W2 = [[1], [-1]].
      bf16 spacing above 1 is 2^-7: bf16(1 + 3 2^-9) = 1 + 2^-7 (three
      quarters of a spacing rounds up), bf16(1 + 2^-9) = 1 (a quarter rounds
      down).  Faithful y = 2^-7; exact y = 2 2^-9 = 2^-8.  Rounding the
      expert output instead of H would give bf16(2^-8) = 2^-8."""
    W_g, W1s, W3s, W2s = _one_expert([[64.0, 64.0]],
                                     [[(1 + 3 * 2.0 ** -9) / 64, (1 + 2.0 ** -9) / 64]],
                                     [[1.0], [-1.0]])
    x = np.array([[1.0]])
    yf, aux = O.moe_forward(x, W_g, W1s, W3s, W2s, K=1, faithful=True)
    ye, _ = O.moe_forward(x, W_g, W1s, W3s, W2s, K=1, faithful=False)
    assert aux["w"][0, 0] == 1.0
    assert yf[0, 0] == 2.0 ** -7, yf
    assert ye[0, 0] == 2.0 ** -8, ye
    # same case with W2 = I (d_ff = d = 2): faithful y is bf16(H) itself
    W_g2, W1s2, W3s2, W2s2 = _one_expert([[64.0, 64.0], [0.0, 0.0]],
                                         [[(1 + 3 * 2.0 ** -9) / 64, (1 + 2.0 ** -9) / 64],
                                          [0.0, 0.0]], np.eye(2))
    yf2, _ = O.moe_forward(np.array([[1.0, 0.0]]), W_g2, W1s2, W3s2, W2s2, K=1, faithful=True)
    assert yf2.tolist() == [[1.0 + 2.0 ** -7, 1.0]], yf2


def check_stack_prenorm_hand():
    """One pre-norm block in the order of the slide "Architecture – 全体"
    (RMSNorm, then the mixture of experts, then the residual add), by hand
    with eps = 0, one expert and K = 1:
      h0 = [2, -2]: mean(h0^2) = 4, RMSNorm(h0) = [1, -1]
      W1 = [[64], [0]]: a = 64, SiLU(64) = 64 exactly; W3 = [[0.5], [0]]: b = 0.5
      H = 32; W2 = [[1/64, 1/32]]: MoE = [0.5, 1]; h1 = h0 + MoE = [2.5, -1].
    A block that fed h0 itself to the MoE would get a = 128 and h1 = [4, 2].
    Faithful mode rounds the new residual stream to bfloat16: with
    W2 = [[3 2^-13, 1/32]] the MoE adds [3 2^-8, 1]; 2 + 3 2^-8 is three
    quarters of a bf16 spacing (2^-6) above 2, so h1 = [2 + 2^-6, -1]
    (exact mode: [2 + 3 2^-8, -1])."""
    h0 = np.array([[2.0, -2.0]])
    blk = _one_expert([[64.0], [0.0]], [[0.5], [0.0]], [[1 / 64, 1 / 32]])
    h1, _ = O.stack_forward(h0, [blk], K=1, eps=0.0)
    assert h1.tolist() == [[2.5, -1.0]], h1
    blk = _one_expert([[64.0], [0.0]], [[0.5], [0.0]], [[3 * 2.0 ** -13, 1 / 32]])
    h1e, _ = O.stack_forward(h0, [blk], K=1, eps=0.0)
    h1f, _ = O.stack_forward(h0, [blk], K=1, eps=0.0, faithful=True)
    assert h1e.tolist() == [[2.0 + 3 * 2.0 ** -8, -1.0]], h1e
    assert h1f.tolist() == [[2.0 + 2.0 ** -6, -1.0]], h1f


def check_stack_two_blocks_hand():
    """Two blocks applied in order, each reading the residual stream the
    previous one left (eps = 0, one expert, K = 1):
      block 1 on h0 = [2, -2]: RMSNorm = [1, -1], W1 = [[64], [0]] (a = 64),
        W3 = [[0.5], [0]] (H = 32), W2 = [[0, 1/8]]: adds [0, 4] -> h1 = [2, 2]
      block 2 on h1: RMSNorm = [1, 1], W1 = [[32], [32]] (a = 64),
        W3 = [[0.5], [0.5]] (H = 64), W2 = [[1/64, 1/64]]: adds [1, 1] -> [3, 3].
    Both blocks reading h0, or the blocks in reverse order, give [2, 2]
    (block 2 sees RMSNorm(h0) = [1, -1], a = 0, SiLU(0) = 0)."""
    h0 = np.array([[2.0, -2.0]])
    b1 = _one_expert([[64.0], [0.0]], [[0.5], [0.0]], [[0.0, 1 / 8]])
    b2 = _one_expert([[32.0], [32.0]], [[0.5], [0.5]], [[1 / 64, 1 / 64]])
    h2, margins = O.stack_forward(h0, [b1, b2], K=1, eps=0.0)
    assert h2.tolist() == [[3.0, 3.0]], h2
    assert len(margins) == 2


def check_stack_scale_invariance():
    """With eps = 0, RMSNorm(c h) = RMSNorm(h) for c > 0, exactly in binary64
    when c is a power of two; so one pre-norm block adds the same MoE output
    to c h0 as to h0 (the block's input is normalised before the MoE, slide
    "Architecture – 全体").  A block whose MoE read anything that is not
    scale invariant fails this."""
    x, W_g, W1s, W3s, W2s = tiny_layer(17, T=6, d=6, d_ff=5, E=4)
    h1, _ = O.stack_forward(x, [(W_g, W1s, W3s, W2s)], K=2, eps=0.0)
    y = h1 - x
    assert np.abs(y).max() > 1e-3
    for c in (2.0 ** 5, 2.0 ** -3):
        hc, _ = O.stack_forward(c * x, [(W_g, W1s, W3s, W2s)], K=2, eps=0.0)
        assert np.allclose(hc - c * x, y, rtol=0, atol=1e-13 * max(c, 1.0))


def check_rmsnorm_closed_form():
    for c in (0.5, -3.0, 1e-3):
        h = np.full((1, 16), c)
        out = O.rmsnorm(h, eps=1e-5)
        assert np.allclose(out, c / math.sqrt(c * c + 1e-5), rtol=1e-15, atol=0)
    h = _rng(15).standard_normal((4, 4096)) * 7
    out = O.rmsnorm(h)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, atol=1e-6)


def check_stack_residual_only():
    """With every W2 zero the MoE adds nothing and the stack returns h0."""
    x, W_g, W1s, W3s, W2s = tiny_layer(16, T=5, d=6, d_ff=5, E=4)
    zero = [np.zeros_like(w) for w in W2s]
    h, margins = O.stack_forward(x, [(W_g, W1s, W3s, zero)] * 3, K=2)
    assert np.array_equal(h, x) and len(margins) == 3


def check_margins_hand():
    m_rank, m_cut = O.routing_margins(np.array([[1.0, 4.0, 2.5, 2.0]]), K=2)
    assert m_rank[0] == 1.5 and m_cut[0] == 0.5


# --- routing statistics ----------------------------------------------------------
def check_routing_stats_hand():
    """Hand case: first choices 0 0 1 1 1 2 0 repeat at t = 1, 3, 4 (three
    repeats in six consecutive pairs); the second choices (1 2 2 0 2 3 3) would
    give two (t = 2, 6).  Every pair counts towards its expert's load."""
    idx = np.array([[0, 1], [0, 2], [1, 2], [1, 0], [1, 2], [2, 3], [0, 3]])
    counts, repeats = O.routing_stats(idx, 4)
    assert repeats == 3
    assert counts.tolist() == [4, 4, 4, 2]
    # an index outside [0, E) counts nowhere and breaks a run
    idx2 = np.array([[0, 1], [-1, 2], [-1, 0], [0, 7]])
    counts2, repeats2 = O.routing_stats(idx2, 4)
    assert repeats2 == 0 and counts2.tolist() == [3, 1, 1, 0]
    assert O.routing_stats(np.zeros((1, 2), dtype=int), 3)[1] == 0


def check_routing_stats_random_rate():
    """"Mixtral of Experts" (xyznot.com), limitations: random assignment
    repeats the first choice 12.5 % of the time with 8 experts, i.e. 1/E.
    Uniform random first choices over 200001 tokens must land within five
    binomial standard deviations of 1/8; the loads sum to T*K."""
    T, E, K = 200_001, 8, 2
    r = _rng(31)
    scores = r.random((T, E))
    idx = np.argsort(scores, axis=1)[:, :K]
    counts, repeats = O.routing_stats(idx, E)
    rate = repeats / (T - 1)
    sigma = math.sqrt((1 / E) * (1 - 1 / E) / (T - 1))
    assert abs(rate - 1 / E) < 5 * sigma, rate
    assert counts.sum() == T * K
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=E))


# --- shapes -------------------------------------------------------------------
def mixtral_param_counts(d, d_ff, E, K, layers=32, vocab=32000, n_q=32, n_kv=8, head=128):
    attn = d * n_q * head + 2 * d * n_kv * head + n_q * head * d
    expert = 3 * d * d_ff
    per_layer_shared = attn + d * E + 2 * d          # router, two RMSNorm gains
    total = layers * (per_layer_shared + E * expert) + 2 * vocab * d + d
    active = layers * (per_layer_shared + K * expert) + 2 * vocab * d + d
    return total, active


def check_shapes_closed_form(d=4096, d_ff=14336, E=8, K=2):
    """Mixtral 全面解析 section 2.1.2: 46.7B total and 12.9B active
    parameters; zikao35 part 04: an 86.99 GB checkpoint.  The layer shapes used
    here reproduce those to every printed digit."""
    total, active = mixtral_param_counts(d, d_ff, E, K)
    assert total == 46_702_792_704 and active == 12_879_925_248
    assert round(total / 1e9, 1) == 46.7 and round(active / 1e9, 1) == 12.9
    assert round(total * 2 / 2 ** 30, 2) == 86.99


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_") and callable(v)]
