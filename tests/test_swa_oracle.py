"""The attention oracle against the pages' examples, an independent dense
formulation, closed forms and special cases; and planted mistakes that the
pins must catch (``swa_pins.py`` names the sources)."""
import math

import numpy as np
import pytest

from oracle import swa_oracle as A
from tests import swa_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def _window_one_too_wide(position, W):
    return range(max(0, position - W), position + 1)


def _slot_wrong_modulus(position, W):
    return position % max(1, W - 1)


def _kv_head_interleaved(h, n_heads, n_kv_heads):
    return h % n_kv_heads


def _attend_unscaled(q, keys, values):
    s = keys @ q
    s = s - s.max()
    p = np.exp(s)
    return (p / p.sum()) @ values


def _attend_no_max_shift_sum_to_one_missing(q, keys, values):
    s = keys @ q / math.sqrt(q.shape[0])
    return np.exp(s - s.max()) @ values          # weights not normalised


_orig_chunk = A.swa_chunk_attention


def _prefill_writes_before_attending(q, k, v, W, chunk):
    # cache updated with the chunk first, then the chunk attends to it
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, hd = q.shape
    kc = np.zeros((W, k.shape[1], hd))
    vc = np.zeros((W, k.shape[1], hd))
    out = np.zeros((T, H, hd))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        for p in range(c0, c1):
            kc[p % W], vc[p % W] = k[p], v[p]
        pos = [p for p in range(c0, c1)]
        out[c0:c1] = _orig_chunk(q[c0:c1], kc[[p % W for p in pos]], vc[[p % W for p in pos]],
                                 kc, vc, c0, W)
    return out, kc, vc, np.ones(W, dtype=bool)


MUTATIONS = {
    "window_one_too_wide": ("window_keys", _window_one_too_wide),
    "slot_wrong_modulus": ("rolling_slot", _slot_wrong_modulus),
    "gqa_heads_interleaved": ("kv_head_of", _kv_head_interleaved),
    "scores_not_scaled": ("_attend", _attend_unscaled),
    "weights_not_normalised": ("_attend", _attend_no_max_shift_sum_to_one_missing),
    "cache_written_before_chunk_attends": ("rolling_prefill", _prefill_writes_before_attending),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(A, attr, fake)
    failed = []
    for check in P.ALL_CHECKS:
        try:
            check()
        except Exception:
            failed.append(check.__name__)
    assert failed, "planted mistake %s went unnoticed" % name
