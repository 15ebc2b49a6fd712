"""Pure-Python scalar oracle for tiny shapes.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

This writes the layer the way the gate equation states it, token by token and
expert by expert, with Python floats (IEEE binary64) and no numpy:

  l = x . W_g;  TopK(l)_i = l_i for the K selected coordinates, -inf else;
  G = softmax(TopK(l));  y = sum over ALL n experts of G_i * E_i(x),
  skipping the experts whose gate is exactly zero.

("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section 2.1.1,
expert-layer sum, gate G(x) and the TopK rule; code block D for the SwiGLU
expert.)  The selected set is found by brute force over all K-subsets, the
reading being: a subset S is a valid top-K set when every selected logit is
>= every unselected one; among valid subsets take the one whose sorted index
tuple is smallest (lower expert index wins ties).
"""

from __future__ import annotations

import itertools
import math


def _dot(u, v):
    s = 0.0
    for a, b in zip(u, v):
        s += a * b
    return s


def _col(M, j):
    return [row[j] for row in M]


def topk_bruteforce(l, K):
    """Brute force over all K-subsets (see module docstring); returns the
    subset ordered by rank, i.e. by (-l_i, i)."""
    n = len(l)
    best = None
    for S in itertools.combinations(range(n), K):
        inside = min(l[i] for i in S)
        outside = max((l[j] for j in range(n) if j not in S), default=-math.inf)
        if inside >= outside:
            if best is None or S < best:
                best = S
    return sorted(best, key=lambda i: (-l[i], i))


def layer_token(x_t, W_g, W1s, W3s, W2s, K):
    """y for one token, plus (selected experts in rank order, dense gate)."""
    n = len(W1s)
    l = [_dot(x_t, _col(W_g, e)) for e in range(n)]
    S = topk_bruteforce(l, K)
    masked = [l[i] if i in S else -math.inf for i in range(n)]
    m = max(masked)
    ex = [math.exp(v - m) if v != -math.inf else 0.0 for v in masked]
    tot = sum(ex)
    G = [v / tot for v in ex]
    d = len(x_t)
    y = [0.0] * d
    for i in range(n):
        if G[i] == 0.0:
            continue  # a zero gate means the expert is not evaluated
        W1, W3, W2 = W1s[i], W3s[i], W2s[i]
        d_ff = len(W1[0])
        h = []
        for f in range(d_ff):
            a = _dot(x_t, _col(W1, f))
            b = _dot(x_t, _col(W3, f))
            h.append(a / (1.0 + math.exp(-a)) * b)
        for j in range(d):
            y[j] += G[i] * _dot(h, _col(W2, j))
    return y, S, G


def layer(x, W_g, W1s, W3s, W2s, K):
    """Apply ``layer_token`` to every row of x (lists of lists of floats)."""
    ys, sel, gates = [], [], []
    for x_t in x:
        y, S, G = layer_token(list(x_t), W_g, W1s, W3s, W2s, K)
        ys.append(y)
        sel.append(S)
        gates.append(G)
    return ys, sel, gates
