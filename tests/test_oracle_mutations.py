"""Plant plausible mistakes in the CPU oracle (on the CPU, in this process
only) and require that the pins catch every one of them."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import oracle_pins as P


def _softmax_all_no_renorm(logits, idx):
    l = np.asarray(logits, dtype=np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, idx, axis=1)


def _topk_upper_tiebreak(logits, K):
    l = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-l[:, ::-1], axis=1, kind="stable")
    return (l.shape[1] - 1 - order)[:, :K]


def _swiglu_swapped(x_rows, W1, W3, W2, faithful=False):
    return _orig_swiglu(x_rows, W3, W1, W2, faithful)


def _swiglu_relu(x_rows, W1, W3, W2, faithful=False):
    x_rows = np.asarray(x_rows, dtype=np.float64)
    a = x_rows @ W1
    return (np.maximum(a, 0) * (x_rows @ W3)) @ W2


def _silu_wrong_sign(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(z))


def _route_unstable(idx, E):
    counts, offsets, st, sr, pos = _orig_route(idx, E)
    st = st.copy()
    for e in range(E):                       # reverse each segment
        st[offsets[e]:offsets[e + 1]] = st[offsets[e]:offsets[e + 1]][::-1].copy()
    return counts, offsets, st, sr, pos


def _gate_weights_rank_swap(logits, idx):
    return _orig_gate_weights(logits, idx)[:, ::-1]


def _bf16_truncate(a):
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.trunc(m * 256) / 256, e)


def _router_transposed(x, W_g):
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W_g, dtype=np.float64)
    if W.shape[0] == W.shape[1]:
        return x @ W.T
    return x @ W[::-1]


def _swiglu_rounds_output(x_rows, W1, W3, W2, faithful=False):
    x_rows = np.asarray(x_rows, dtype=np.float64)
    a = x_rows @ np.asarray(W1, dtype=np.float64)
    h = O.silu(a) * (x_rows @ np.asarray(W3, dtype=np.float64))
    out = h @ np.asarray(W2, dtype=np.float64)
    return O.bf16_round(out) if faithful else out


def _stack_moe_reads_h(h0, blocks, K, eps=1e-5, faithful=False):
    h = np.asarray(h0, dtype=np.float64)
    margins = []
    for (W_g, W1s, W3s, W2s) in blocks:
        y, aux = O.moe_forward(h, W_g, W1s, W3s, W2s, K, faithful)
        margins.append(O.routing_margins(aux["logits"], K))
        h = h + y
        if faithful:
            h = O.bf16_round(h)
    return h, margins


def _stack_post_norm(h0, blocks, K, eps=1e-5, faithful=False):
    h = np.asarray(h0, dtype=np.float64)
    margins = []
    for (W_g, W1s, W3s, W2s) in blocks:
        y, aux = O.moe_forward(h, W_g, W1s, W3s, W2s, K, faithful)
        margins.append(O.routing_margins(aux["logits"], K))
        h = O.rmsnorm(h + y, eps, faithful)
    return h, margins


def _stack_blocks_read_h0(h0, blocks, K, eps=1e-5, faithful=False):
    h0 = np.asarray(h0, dtype=np.float64)
    xn = O.rmsnorm(h0, eps, faithful)
    h = h0.copy()
    margins = []
    for (W_g, W1s, W3s, W2s) in blocks:
        y, aux = O.moe_forward(xn, W_g, W1s, W3s, W2s, K, faithful)
        margins.append(O.routing_margins(aux["logits"], K))
        h = h + y
        if faithful:
            h = O.bf16_round(h)
    return h, margins


def _stack_no_residual_rounding(h0, blocks, K, eps=1e-5, faithful=False):
    h = np.asarray(h0, dtype=np.float64)
    margins = []
    for (W_g, W1s, W3s, W2s) in blocks:
        y, aux = O.moe_forward(O.rmsnorm(h, eps, faithful), W_g, W1s, W3s, W2s, K, faithful)
        margins.append(O.routing_margins(aux["logits"], K))
        h = h + y
    return h, margins


def _stats_second_choice(idx, E):
    idx = np.asarray(idx)
    counts = np.bincount(idx[(idx >= 0) & (idx < E)].reshape(-1), minlength=E)
    col = idx[:, -1]
    return counts, int(np.sum((col[1:] == col[:-1]) & (col[1:] >= 0) & (col[1:] < E)))


def _stats_first_choice_load(idx, E):
    idx = np.asarray(idx)
    first = idx[:, 0]
    counts = np.bincount(first[(first >= 0) & (first < E)], minlength=E)
    return counts, int(np.sum((first[1:] == first[:-1]) & (first[1:] >= 0) & (first[1:] < E)))


def _stats_stride_two(idx, E):
    idx = np.asarray(idx)
    counts = np.bincount(idx[(idx >= 0) & (idx < E)].reshape(-1), minlength=E)
    first = idx[:, 0]
    return counts, int(np.sum((first[2:] == first[:-2]) & (first[2:] >= 0) & (first[2:] < E)))


_orig_swiglu = O.swiglu_expert
_orig_route = O.route_tables
_orig_gate_weights = O.gate_weights

MUTATIONS = {
    "gate_no_renormalise": ("gate_weights", _softmax_all_no_renorm),
    "topk_upper_index_wins": ("topk_select", _topk_upper_tiebreak),
    "swiglu_branches_swapped": ("swiglu_expert", _swiglu_swapped),
    "swiglu_relu_activation": ("swiglu_expert", _swiglu_relu),
    "silu_sign_flip": ("silu", _silu_wrong_sign),
    "dispatch_not_stable": ("route_tables", _route_unstable),
    "gate_ranks_swapped": ("gate_weights", _gate_weights_rank_swap),
    "bf16_truncates": ("bf16_round", _bf16_truncate),
    "router_operand_flipped": ("router_logits", _router_transposed),
    "faithful_rounds_expert_output": ("swiglu_expert", _swiglu_rounds_output),
    "stack_moe_reads_unnormalised_h": ("stack_forward", _stack_moe_reads_h),
    "stack_post_norm": ("stack_forward", _stack_post_norm),
    "stack_every_block_reads_h0": ("stack_forward", _stack_blocks_read_h0),
    "stack_faithful_skips_residual_rounding": ("stack_forward", _stack_no_residual_rounding),
    "stats_repeat_on_second_choice": ("routing_stats", _stats_second_choice),
    "stats_load_counts_first_choice_only": ("routing_stats", _stats_first_choice_load),
    "stats_compares_tokens_two_apart": ("routing_stats", _stats_stride_two),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fake)
    failed = []
    for check in P.ALL_CHECKS:
        try:
            check()
        except Exception:
            failed.append(check.__name__)
    assert failed, "planted mistake %s went unnoticed" % name
