"""Plain float64 CPU oracle of the attention sub-block in front of the MoE:
grouped-query attention over a sliding window, with a rolling-buffer cache
and chunked prefill.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Loops over query
tokens and heads with numpy dot products; no blocking or fusion.

Pages cited (by title and section):

* "从Mistral 7B到MoE模型Mixtral 8x7B的全面解析：从原理分析到代码解读"
  (aiqianji.com blog, *全面解析* below):
  section 1.1 (GQA: 32 query heads, 8 key/value heads, head dimension 128,
  the query heads are 4x the key/value heads; window size 4096, and the
  example that the 5000th token attends to tokens 905..5000),
  section 1.2.1 (sliding-window attention: a token attends to at most W
  tokens of the previous layer, itself included -- the W = 3 example),
  section 1.2.2 (rolling-buffer cache: size W, the keys and values of
  timestep i live in slot i mod W; the W = 3 "The cat sat on the mat"
  example), section 1.2.3 (prefill in chunks of the window size: each chunk
  attends to the cache through the sliding window and to itself through a
  causal mask, and not to tokens that fell out of the window).
* "Mixtral of Experts" (xyznot.com paper page), section "Abstract": Mixtral
  has the same architecture as Mistral 7B apart from the expert layers.

Readings where the pages are silent (each also listed in the design doc):

* Attention weights are the softmax over the window of the query-key inner
  products scaled by 1/sqrt(head_dim); the output is the weighted sum of the
  values (the pages name the inner products and the window only).
* Query head h reads key/value head h // (n_heads / n_kv_heads): consecutive
  groups of 4 query heads share one key/value head.
* No positional rotation is applied inside the sub-block: the pages do not
  describe one; queries and keys arrive as given.
* A chunk attends to the cache as it was before the chunk, then its own keys
  and values are written to the cache (slot = position mod W); a chunk is at
  most W tokens long, so nothing a chunk's queries need is overwritten first.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rolling_slot",
    "window_keys",
    "kv_head_of",
    "swa_attention",
    "swa_chunk_attention",
    "rolling_prefill",
]


def rolling_slot(position: int, W: int) -> int:
    """Cache slot of the keys/values of timestep ``position``
    (*全面解析* section 1.2.2: position i mod W)."""
    if W <= 0 or position < 0:
        raise ValueError("W must be positive and the position non-negative")
    return position % W


def window_keys(position: int, W: int) -> range:
    """Positions a token at ``position`` attends to: the W most recent
    tokens, itself included (*全面解析* sections 1.1 and 1.2.1)."""
    if W <= 0 or position < 0:
        raise ValueError("W must be positive and the position non-negative")
    return range(max(0, position - W + 1), position + 1)


def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    """Key/value head shared by query head h (grouped-query attention,
    *全面解析* section 1.1; consecutive groups is the reading)."""
    if n_heads % n_kv_heads != 0:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    return h // (n_heads // n_kv_heads)


def _attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """softmax(keys . q / sqrt(hd)) . values for one query vector."""
    s = keys @ q / math.sqrt(q.shape[0])
    s = s - s.max()
    p = np.exp(s)
    return (p / p.sum()) @ values


def swa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, W: int) -> np.ndarray:
    """Sliding-window grouped-query attention over one whole sequence.

    q [T, H, hd], k and v [T, KVH, hd] (any float dtype; computed in float64).
    Returns o [T, H, hd] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, hd = q.shape
    KVH = k.shape[1]
    out = np.zeros((T, H, hd))
    for i in range(T):
        js = list(window_keys(i, W))
        for h in range(H):
            g = kv_head_of(h, H, KVH)
            out[i, h] = _attend(q[i, h], k[js, g], v[js, g])
    return out


def swa_chunk_attention(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                        k_cache: np.ndarray, v_cache: np.ndarray, pos0: int,
                        W: int, rows=None) -> np.ndarray:
    """One chunk of T <= W tokens at positions pos0 .. pos0+T-1 of one
    sequence, given the rolling cache as it stands before the chunk
    (*全面解析* section 1.2.3): a key at position p < pos0 is read from cache
    slot p mod W, a key at p >= pos0 from the chunk row p - pos0.

    q [T, H, hd]; k_new, v_new [T, KVH, hd]; k_cache, v_cache [W, KVH, hd].
    ``rows`` picks the chunk tokens to compute (default: all).
    Returns o [len(rows), H, hd] float64."""
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    T, H, hd = q.shape
    KVH = k_new.shape[1]
    if T > W:
        raise ValueError("a chunk is at most W tokens long")
    rows = range(T) if rows is None else list(rows)
    out = np.zeros((len(rows), H, hd))
    for n, t in enumerate(rows):
        p = pos0 + t
        pos = list(window_keys(p, W))
        keys = np.stack([k_cache[rolling_slot(j, W)] if j < pos0 else k_new[j - pos0]
                         for j in pos])
        vals = np.stack([v_cache[rolling_slot(j, W)] if j < pos0 else v_new[j - pos0]
                         for j in pos])
        for h in range(H):
            g = kv_head_of(h, H, KVH)
            out[n, h] = _attend(q[t, h], keys[:, g], vals[:, g])
    return out


def rolling_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, W: int, chunk: int):
    """The pages' prefill procedure (*全面解析* sections 1.2.2 and 1.2.3):
    split the sequence into chunks of at most W tokens; each chunk attends
    through ``swa_chunk_attention`` to the cache as it stands, then writes its
    keys and values into slots position mod W.

    Returns (o [T, H, hd], k_cache [W, KVH, hd], v_cache [W, KVH, hd],
    filled [W] bool)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, hd = q.shape
    KVH = k.shape[1]
    if not 0 < chunk <= W:
        raise ValueError("chunk must be in 1 .. W")
    k_cache = np.zeros((W, KVH, hd))
    v_cache = np.zeros((W, KVH, hd))
    filled = np.zeros(W, dtype=bool)
    out = np.zeros((T, H, hd))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        out[c0:c1] = swa_chunk_attention(q[c0:c1], k[c0:c1], v[c0:c1], k_cache, v_cache, c0, W)
        for p in range(c0, c1):
            s = rolling_slot(p, W)
            k_cache[s] = k[p]
            v_cache[s] = v[p]
            filled[s] = True
    return out, k_cache, v_cache, filled
