"""Plain float64 CPU oracle of the Mixtral sparse-MoE layer forward.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Slow and obvious on
purpose: numpy matmuls are the only library primitives, there is no blocking,
fusion or reordering beyond what the definition states.

Pages cited (by title and section):

* "从Mistral 7B到MoE模型Mixtral 8x7B的全面解析：从原理分析到代码解读"
  (aiqianji.com blog, called *Mixtral 全面解析* below):
  section 2.1.1 (expert-layer sum, the gate G(x) = Softmax(TopK(x W_g)) and
  the TopK masking rule, the Mixtral instance with Top2 and SwiGLU experts),
  section 2.1.4 (the router is a bias-free linear layer from hidden_dim to
  num_experts), section 3.1.1 (routing weights: softmax in float, top-k,
  renormalise), section 3.1.2 and code blocks B, C (expert-major dispatch),
  code block D (expert = w2(act(w1 h) * w3 h)), code block E (zero-initialised
  accumulator, index_add).
* "Mixtral of Experts" (xyznot.com paper page), section "Method with key
  equations": shapes (hidden 4096, 8 experts, SwiGLU width 14336, K = 2) and
  the same gate and sum equations.
* "【DL輪読会】Mixtral of Experts" (docswell slides), slide
  "Architecture – 全体": RMSNorm before the mixture-of-experts block.

Readings where the pages are silent (each also listed in the design doc):

* TopK keeps exactly K coordinates; ties go to the lower expert index
  (key (-logit, index)).
* The gate weights are the softmax of the TopK-masked logits, i.e. a softmax
  over the K selected logits only; the pages' code reaches the same numbers by
  softmax over all experts followed by renormalisation over the selected K.
* The activation is SiLU (Swish with beta = 1); W1 is the activated branch and
  W3 the linear branch.
* Weights are stored row-major in the pages' ``x . W`` orientation:
  ``W_g [d, E]``, ``W1[e], W3[e] [d, d_ff]``, ``W2[e] [d_ff, d]``.
* "faithful" mode rounds the SwiGLU product H to bfloat16 (round to nearest,
  ties to even) before the W2 projection, as the pages' eager code does when
  activations are bfloat16; "exact" mode does no intermediate rounding.
* The expert outputs of one token are summed in rank order (rank 0 first).
* Dispatch is dropless: every (token, expert) pair is computed.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "router_logits",
    "topk_select",
    "gate_dense",
    "gate_weights",
    "route_tables",
    "silu",
    "swiglu_expert",
    "moe_forward",
    "dense_mixture",
    "rmsnorm",
    "stack_forward",
    "routing_margins",
    "routing_stats",
]


def _f64(a) -> np.ndarray:
    out = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(out)):
        raise ValueError("oracle inputs must be finite")
    return out


# ---------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even), written from the format:
# 8 significant bits (7 stored + the implicit one), the exponent range of
# IEEE binary32, gradual underflow with quantum 2**-133.
# ---------------------------------------------------------------------------
_BF16_MAX = float.fromhex("0x1.fep127")
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_QUANTUM = 2.0 ** -133


def bf16_round(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    Returned as float64 holding exactly representable bfloat16 values.
    Values beyond the largest finite bfloat16 after rounding become +-inf.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    tiny = np.abs(a) < _BF16_MIN_NORMAL
    # normal range: scale the significand to 8 integer bits and round half-even
    mant, expo = np.frexp(np.where(tiny, 1.0, a))  # a = mant * 2**expo, 0.5 <= |mant| < 1
    out_norm = np.ldexp(np.rint(mant * 256.0) / 256.0, expo)
    # subnormal range: fixed quantum
    out_tiny = np.rint(a / _BF16_SUBNORMAL_QUANTUM) * _BF16_SUBNORMAL_QUANTUM
    out = np.where(tiny, out_tiny, out_norm)
    # the largest finite bf16 is 0x1.fe p127; anything that rounds above it overflows
    return np.where(np.abs(out) > _BF16_MAX, np.copysign(np.inf, out), out)


# ---------------------------------------------------------------------------
# Router (Mixtral 全面解析 section 2.1.4: bias-free linear layer; section 2.1.1:
# logits l = x . W_g in R^n)
# ---------------------------------------------------------------------------
def router_logits(x, W_g) -> np.ndarray:
    """l[t, e] = sum_k x[t, k] * W_g[k, e], in float64, no bias."""
    return _f64(x) @ _f64(W_g)


def topk_select(logits, K: int) -> np.ndarray:
    """Indices of the K largest logits per token, in rank order.

    Mixtral 全面解析 section 2.1.1 (TopK keeps the top-K coordinates of l).
    Rank order is the key (-l_i, i): larger logit first, lower expert index
    first among equal logits.  ``np.argsort(..., kind="stable")`` of -l keeps
    equal keys in index order, which is exactly that key.
    """
    logits = np.asarray(logits, dtype=np.float64)
    E = logits.shape[1]
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :K].astype(np.int64)


def gate_dense(logits, idx) -> np.ndarray:
    """G(x) = Softmax(TopK(l)) as a dense [T, E] matrix.

    Mixtral 全面解析 section 2.1.1: TopK(l)_i = l_i for the selected
    coordinates and -inf elsewhere; the softmax then gives exp(-inf) = 0 to
    every other expert.  The max subtraction is the usual overflow guard and
    does not change the value.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    masked = np.full((T, E), -np.inf)
    rows = np.arange(T)[:, None]
    masked[rows, idx] = logits[rows, idx]
    m = masked.max(axis=1, keepdims=True)
    ex = np.exp(masked - m)
    return ex / ex.sum(axis=1, keepdims=True)


def gate_weights(logits, idx) -> np.ndarray:
    """Per-rank gate weights w[t, r] = G(x_t)[idx[t, r]] (Mixtral 全面解析
    section 3.1.1 keeps them as a [tokens, top_k] table summing to 1)."""
    G = gate_dense(logits, idx)
    return np.take_along_axis(G, idx, axis=1)


# ---------------------------------------------------------------------------
# Expert-major dispatch tables (Mixtral 全面解析 section 3.1.2, code blocks
# B and C: for every expert, which (rank, token) pairs it processes)
# ---------------------------------------------------------------------------
def route_tables(idx, E: int):
    """Stable counting sort of the (token, rank) pairs by expert.

    Pairs are numbered p = t*K + r.  Returns
      counts[E]         pairs per expert,
      offsets[E+1]      exclusive prefix sum of counts,
      sorted_token[P]   token of the pair at each sorted position,
      sorted_rank[P]    rank of the pair at each sorted position,
      pos[T, K]         sorted position of pair (t, r).
    Inside one expert's segment the pairs keep their original order p, i.e.
    tokens ascending (Python's ``sorted`` is stable).
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    flat = [int(v) for v in idx.reshape(-1)]
    if any(v < 0 or v >= E for v in flat):
        raise ValueError("expert index out of range")
    counts = np.zeros(E, dtype=np.int64)
    for v in flat:
        counts[v] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    order = sorted(range(T * K), key=lambda p: flat[p])
    sorted_token = np.array([p // K for p in order], dtype=np.int64)
    sorted_rank = np.array([p % K for p in order], dtype=np.int64)
    pos = np.empty(T * K, dtype=np.int64)
    for dest, p in enumerate(order):
        pos[p] = dest
    return counts, offsets, sorted_token, sorted_rank, pos.reshape(T, K)


# ---------------------------------------------------------------------------
# SwiGLU expert (Mixtral 全面解析 code block D; Mixtral of Experts, Method)
# ---------------------------------------------------------------------------
def silu(z) -> np.ndarray:
    """Swish with beta = 1: z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows, W1, W3, W2, faithful: bool = False) -> np.ndarray:
    """E(x) = (SiLU(x W1) * (x W3)) W2 for a block of token rows.

    W1 is the activated branch and W3 the linear one (code block D applies the
    activation to w1's output).  In faithful mode the product H is rounded to
    bfloat16 before the last projection.
    """
    x_rows = _f64(x_rows)
    a = x_rows @ _f64(W1)
    b = x_rows @ _f64(W3)
    h = silu(a) * b
    if faithful:
        h = bf16_round(h)
    return h @ _f64(W2)


# ---------------------------------------------------------------------------
# The layer (Mixtral 全面解析 section 2.1.1: y = sum_i G(x)_i * SwiGLU_i(x),
# only experts with a non-zero gate are evaluated; section 3.1.2 and code
# block E: expert-major loop into a zero-initialised accumulator)
# ---------------------------------------------------------------------------
def moe_forward(x, W_g, W1s, W3s, W2s, K: int, faithful: bool = False):
    """Forward of one sparse-MoE layer.

    Returns (y, aux) with y [T, d] float64 and aux holding the routing:
    logits, idx [T, K], w [T, K], counts, offsets, sorted_token, sorted_rank,
    pos.  Experts are visited in index order as in the pages' loop; every
    routed pair's expert output is kept and the token's K contributions are
    summed afterwards in rank order.
    """
    x = _f64(x)
    T, d = x.shape
    E = len(W1s)
    logits = router_logits(x, W_g)
    idx = topk_select(logits, K)
    w = gate_weights(logits, idx)
    counts, offsets, sorted_token, sorted_rank, pos = route_tables(idx, E)
    contrib = np.zeros((T, K, d))
    for e in range(E):
        tok, rank = np.nonzero(idx == e)
        if tok.size == 0:
            continue  # an expert with no routed token is never evaluated
        contrib[tok, rank] = swiglu_expert(x[tok], W1s[e], W3s[e], W2s[e], faithful)
    y = np.zeros((T, d))
    for r in range(K):
        y = y + w[:, r:r + 1] * contrib[:, r]
    aux = dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
               sorted_token=sorted_token, sorted_rank=sorted_rank, pos=pos)
    return y, aux


def dense_mixture(x, W_g, W1s, W3s, W2s) -> np.ndarray:
    """The K = E special case written independently: every expert evaluated
    and weighted by the plain softmax of all logits (Mixtral 全面解析 section
    2.1.1: with K = n no coordinate is masked)."""
    x = _f64(x)
    logits = x @ _f64(W_g)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    y = np.zeros_like(x)
    for e in range(len(W1s)):
        a = x @ _f64(W1s[e])
        b = x @ _f64(W3s[e])
        y = y + p[:, e:e + 1] * ((a / (1.0 + np.exp(-a)) * b) @ _f64(W2s[e]))
    return y


# ---------------------------------------------------------------------------
# Pre-norm block glue ("【DL輪読会】Mixtral of Experts", slide
# "Architecture – 全体": RMSNorm then the mixture of experts, with a residual)
# ---------------------------------------------------------------------------
def rmsnorm(h, eps: float = 1e-5, faithful: bool = False) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) per row, unit gain."""
    h = _f64(h)
    out = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    return bf16_round(out) if faithful else out


def stack_forward(h0, blocks, K: int, eps: float = 1e-5, faithful: bool = False):
    """h_{l+1} = h_l + MoE_l(RMSNorm(h_l)) over a list of blocks.

    ``blocks`` is a sequence of (W_g, W1s, W3s, W2s).  In faithful mode the
    normalised input, H and the new residual stream are rounded to bfloat16,
    as a bfloat16 stack stores them.  Returns the final h and the per-block
    routing margins (see ``routing_margins``)."""
    h = _f64(h0)
    margins = []
    for (W_g, W1s, W3s, W2s) in blocks:
        xn = rmsnorm(h, eps, faithful)
        y, aux = moe_forward(xn, W_g, W1s, W3s, W2s, K, faithful)
        margins.append(routing_margins(aux["logits"], K))
        h = h + y
        if faithful:
            h = bf16_round(h)
    return h, margins


def routing_margins(logits, K: int):
    """Per token, the gaps between consecutive sorted logits around the
    selection: (m_rank, m_cut) where m_rank is the smallest gap among the K
    selected (it decides the rank order) and m_cut = l_(K) - l_(K+1) (it
    decides the selected set; +inf when K = E)."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
    T, E = s.shape
    if K >= 2:
        m_rank = np.min(s[:, :K - 1] - s[:, 1:K], axis=1)
    else:
        m_rank = np.full(T, np.inf)
    m_cut = s[:, K - 1] - s[:, K] if K < E else np.full(T, np.inf)
    return m_rank, m_cut


# ---------------------------------------------------------------------------
# Routing statistics ("Mixtral of Experts" (xyznot.com), limitations: the
# first choice of consecutive tokens repeats more often than the 1/E of random
# routing; "杀疯了的开源专家模型 Mixtral 8x7B 论文公开啦！" (redian.news), 实验:
# per layer, consecutive tokens are often assigned the same expert)
# ---------------------------------------------------------------------------
def routing_stats(idx, E: int):
    """(counts[E], repeats) of one layer's routing table idx [T, K]:
    counts[e] = pairs routed to expert e; repeats = number of tokens t >= 1
    whose first choice idx[t, 0] equals idx[t - 1, 0].  Indices outside
    [0, E) count nowhere and never repeat."""
    idx = np.asarray(idx)
    T = idx.shape[0]
    counts = np.zeros(E, dtype=np.int64)
    for v in idx.reshape(-1):
        if 0 <= v < E:
            counts[v] += 1
    repeats = 0
    for t in range(1, T):
        if idx[t, 0] == idx[t - 1, 0] and 0 <= idx[t, 0] < E:
            repeats += 1
    return counts, repeats
