"""Seeded input recipes: determinism, shapes, and the routing structure the
prefill recipe is built to have (measured with the CPU oracle's router)."""
import numpy as np
import torch

import workloads as W
from oracle import moe_oracle as O
from tests import oracle_pins as P


def test_deterministic_bytes():
    w = W.scaled(W.WORKLOADS["decode_bf16_T8"], d=256, d_ff=512, T=16)
    a = W.layer_inputs(w)
    b = W.layer_inputs(w)
    ta = [a["x"], a["W_g"], *a["W1"], *a["W3"], *a["W2"]]
    tb = [b["x"], b["W_g"], *b["W1"], *b["W3"], *b["W2"]]
    assert W.sha256_of(ta) == W.sha256_of(tb)
    assert a["x"].dtype == torch.bfloat16 and a["W1"][0].shape == (256, 512)
    assert a["W2"][0].shape == (512, 256) and a["W_g"].shape == (256, 8)
    # different tensors get different streams
    assert not torch.equal(a["W1"][0], a["W3"][0])


def test_mixtral_shapes_match_published_counts():
    w = W.WORKLOADS["decode_bf16_T8"]
    P.check_shapes_closed_form(w.d, w.d_ff, w.E, w.K)
    for name in ("mid_bf16_T512", "prefill_bf16_T4096_zipf", "stack32_bf16_T4096"):
        v = W.WORKLOADS[name]
        assert (v.d, v.d_ff, v.E, v.K) == (w.d, w.d_ff, w.E, w.K)


def test_unit_rms_rows():
    w = W.scaled(W.WORKLOADS["mid_bf16_T512"], T=64)
    x = W.make_x(w, W.expert_weights(W.scaled(w, E=1), experts=[])[0]).double()
    rms = x.pow(2).mean(dim=1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=5e-3)


def test_prefill_recipe_routing_structure():
    w = W.WORKLOADS["prefill_bf16_T4096_zipf"]
    W_g, _, _, _ = W.expert_weights(w, experts=[])
    x = W.make_x(w, W_g)
    logits = O.router_logits(x.float().numpy(), W_g.float().numpy())
    idx = O.topk_select(logits, w.K)
    shares = np.bincount(idx.reshape(-1), minlength=w.E) / idx.size
    target = 1.0 / np.arange(1, 9) ** 1.2
    target /= target.sum()
    assert np.all(np.abs(shares - target) < 0.01), (shares, target)
    first = idx[:, 0]
    repeat = np.mean(first[1:] == first[:-1])
    assert repeat > 0.5            # runs of shared base vectors


def test_uniform_recipe_first_choice_repeat_rate():
    """The 512-token workload routes near-uniformly: its consecutive tokens
    repeat their first choice at about random routing's 1/E = 12.5 %
    ("Mixtral of Experts" (xyznot.com), limitations), within three binomial
    standard deviations (routing by the oracle's float64 router)."""
    w = W.WORKLOADS["mid_bf16_T512"]
    W_g, _, _, _ = W.expert_weights(w, experts=[])
    x = W.make_x(w, W_g)
    idx = O.topk_select(O.router_logits(x.float().numpy(), W_g.float().numpy()), w.K)
    _, repeats = O.routing_stats(idx, w.E)
    rate = repeats / (w.T - 1)
    sigma = np.sqrt(0.125 * 0.875 / (w.T - 1))
    assert abs(rate - 0.125) < 3 * sigma, rate
