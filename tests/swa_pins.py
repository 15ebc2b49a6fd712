"""Checks that pin the attention oracle (``oracle/swa_oracle.py``) to facts
outside itself.  Each ``check_*`` raises AssertionError on failure; they run
as tests in ``test_swa_oracle.py`` and against planted mistakes there.

Sources (page title, section): "从Mistral 7B到MoE模型Mixtral 8x7B的全面解析"
(aiqianji.com blog, *全面解析*), section 1.1 (GQA head counts, window 4096,
the 5000th token attends to tokens 905..5000), section 1.2.1 (a token sees
at most W tokens, itself included; the W = 3 sentence), section 1.2.2 (slot
i mod W; the W = 3 "The cat sat on the mat" slots), section 1.2.3 (chunks
attend to the cache and causally to themselves).
"""

from __future__ import annotations

import math

import numpy as np

from oracle import swa_oracle as A


def _qkv(seed, T, H, KVH, hd, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, H, hd)) * scale, r.standard_normal((T, KVH, hd)),
            r.standard_normal((T, KVH, hd)))


def _dense_band_attention(q, k, v, W):
    """Independent formulation: the full score matrix of every head at once,
    keys expanded to query heads by np.repeat, a band mask 0 <= i - j < W, a
    masked softmax over the key axis."""
    T, H, hd = q.shape
    KVH = k.shape[1]
    kk = np.repeat(k, H // KVH, axis=1)          # [T, H, hd]
    vv = np.repeat(v, H // KVH, axis=1)
    s = np.einsum("ihd,jhd->hij", q, kk) / math.sqrt(hd)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = (i - j >= 0) & (i - j < W)
    s = np.where(mask[None], s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=2, keepdims=True)
    return np.einsum("hij,jhd->ihd", p, vv)


def check_slots_page_example():
    # "The cat sat on the mat" with W = 3: slots 0, 1, 2, 0, 1, 2
    assert [A.rolling_slot(i, 3) for i in range(6)] == [0, 1, 2, 0, 1, 2]


def check_window_page_examples():
    # the 5000th token (index 4999) attends to the 905th .. 5000th tokens
    r = A.window_keys(4999, 4096)
    assert (r.start, r.stop - 1, len(r)) == (904, 4999, 4096)
    r = A.window_keys(5000, 4096)
    assert (r.start, r.stop - 1) == (905, 5000)
    # W = 3: the last "the" of "The cat sat on the" sees "sat on the"
    assert list(A.window_keys(4, 3)) == [2, 3, 4]
    # the first tokens see everything before them
    assert list(A.window_keys(1, 3)) == [0, 1]


def check_gqa_grouping():
    # 32 query heads over 8 key/value heads: 4 consecutive query heads each
    assert [A.kv_head_of(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert all(A.kv_head_of(h, 8, 8) == h for h in range(8))


def check_dense_band_reference():
    for W, T in [(3, 9), (5, 5), (16, 12), (1, 4)]:
        q, k, v = _qkv(W * 100 + T, T, 8, 2, 16)
        got = A.swa_attention(q, k, v, W)
        ref = _dense_band_attention(q, k, v, W)
        assert np.max(np.abs(got - ref)) < 1e-12, (W, T)


def check_single_key_is_its_value():
    q, k, v = _qkv(3, 4, 4, 2, 8)
    o = A.swa_attention(q, k, v, 1)              # W = 1: each token sees itself
    for h in range(4):
        assert np.array_equal(o[:, h], v[:, A.kv_head_of(h, 4, 2)])
    o = A.swa_attention(q, k, v, 4)
    assert np.array_equal(o[0], v[0][[0, 0, 1, 1]])


def check_uniform_keys_average_values():
    T, W = 10, 4
    q, k, v = _qkv(4, T, 4, 2, 8)
    k[:] = k[0:1]                                 # one key everywhere: equal scores
    o = A.swa_attention(q, k, v, W)
    for i in range(T):
        lo = max(0, i - W + 1)
        mean = v[lo:i + 1].mean(axis=0)           # [KVH, hd]
        assert np.allclose(o[i], mean[[0, 0, 1, 1]], atol=1e-12)


def check_dominant_key():
    # a key aligned with the query and scaled up takes (almost) all the weight
    T, W, hd = 6, 6, 16
    q, k, v = _qkv(5, T, 2, 1, hd)
    k[2, 0] = q[5, 0] * 50.0
    o = A.swa_attention(q, k, v, W)
    assert np.allclose(o[5, 0], v[2, 0], atol=1e-9)


def check_gqa_equals_replicated_heads():
    T, W = 7, 3
    q, k, v = _qkv(6, T, 8, 2, 8)
    o = A.swa_attention(q, k, v, W)
    o_mha = A.swa_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), W)
    assert np.max(np.abs(o - o_mha)) < 1e-14


def check_chunked_prefill_equals_full():
    # the pages' chunked prefill through the rolling cache reproduces the
    # sliding-window attention of the whole sequence, wrap-around included
    T, W = 23, 5
    q, k, v = _qkv(7, T, 4, 2, 8)
    full = A.swa_attention(q, k, v, W)
    for chunk in (1, 2, 3, 5):
        o, _, _, _ = A.rolling_prefill(q, k, v, W, chunk)
        assert np.max(np.abs(o - full)) < 1e-12, chunk


def check_final_cache_holds_last_window():
    T, W = 13, 4
    q, k, v = _qkv(8, T, 2, 1, 4)
    _, kc, vc, filled = A.rolling_prefill(q, k, v, W, 3)
    assert filled.all()
    for p in range(T - W, T):
        assert np.array_equal(kc[p % W], k[p]) and np.array_equal(vc[p % W], v[p])


def check_chunk_attention_contract():
    # one chunk after a wrapped cache: positions 9 .. 12 with W = 5 read
    # positions 5 .. 8 from slots p mod 5 and the rest from the chunk
    T, W = 13, 5
    q, k, v = _qkv(9, T, 4, 2, 8)
    kc = np.full((W, 2, 8), np.nan)
    vc = np.full((W, 2, 8), np.nan)
    for p in range(4, 9):                         # cache after positions 0 .. 8
        kc[p % W], vc[p % W] = k[p], v[p]
    o = A.swa_chunk_attention(q[9:], k[9:], v[9:], kc, vc, 9, W)
    assert np.max(np.abs(o - A.swa_attention(q, k, v, W)[9:])) < 1e-12


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_") and callable(v)]
