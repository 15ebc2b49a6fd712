"""Calibrate the per-expert router bias behind the skewed-load prefill workload.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

The prefill workload (T = 4096, Mixtral shape) wants expert popularity to
follow Zipf(s = 1.2): the share of the T*K (token, expert) pairs that go to the
expert of popularity rank j is proportional to 1 / j**1.2.  A bias b_e is added
to logit e, folded into the token rows by the generator (``workloads``).

Two stages, both with the oracle's float64 router and top-K:
1. a start on seeded standard-normal logits (each logit of a unit-RMS row with
   W_g ~ N(0, 1/d) is close to a standard normal), by the fixed-point
   iteration  b_e += 0.5 * (log p_e - log share_e(b));
2. the same iteration on the workload instance itself (its runs of shared
   base vectors make the realised shares of 4096 tokens differ from the
   i.i.d. ones by more than a per cent): the rows are rebuilt with the
   candidate bias, rounded to bf16 exactly as the generator stores them, and
   routed, until every realised share is within 0.5 % (absolute) of the target.
Run it as ``python -m oracle.calibrate_zipf_bias``; it prints the vector
stored as ``ZIPF_BIAS`` in ``workloads/__init__.py``.
"""

from __future__ import annotations

import numpy as np

from oracle.moe_oracle import router_logits, topk_select


def zipf_shares(E: int, s: float) -> np.ndarray:
    p = 1.0 / np.arange(1, E + 1) ** s
    return p / p.sum()


def pair_shares(logits: np.ndarray, K: int) -> np.ndarray:
    idx = topk_select(logits, K)
    E = logits.shape[1]
    return np.bincount(idx.reshape(-1), minlength=E) / idx.size


def calibrate(E: int = 8, K: int = 2, s: float = 1.2, n: int = 400_000,
              iters: int = 60, seed: int = 20240112) -> np.ndarray:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, E))
    target = zipf_shares(E, s)
    b = np.log(target) - np.log(target).mean()
    for _ in range(iters):
        got = pair_shares(z + b, K)
        b = b + 0.5 * (np.log(target) - np.log(got))
        b = b - b.mean()
    return b


def instance_shares(b, t, W_g, K):
    import torch
    import workloads as W
    x = W.biased_rows(t, W_g, b, torch.bfloat16)
    return pair_shares(router_logits(x.float().numpy(), W_g.float().numpy()), K)


def calibrate_instance(b0, name: str = "prefill_bf16_T4096_zipf", s: float = 1.2,
                       tol: float = 0.005, iters: int = 40):
    import workloads as W
    w = W.WORKLOADS[name]
    W_g = W.expert_weights(w, "cpu", experts=[])[0]
    t = W.zipf_rows(w)
    target = zipf_shares(w.E, s)
    b = np.asarray(b0, dtype=np.float64)
    for _ in range(iters):
        got = instance_shares(b, t, W_g, w.K)
        if np.abs(got - target).max() < tol:
            break
        b = b + 0.5 * (np.log(target) - np.log(got))
        b = b - b.mean()
    return b, got, target


if __name__ == "__main__":
    b = calibrate()
    b, got, target = calibrate_instance(b)
    print("bias:", np.array2string(b, precision=6, separator=", "))
    print("target:", np.round(target, 4))
    print("realised on the prefill instance:", np.round(got, 4),
          "max |diff| %.4f" % np.abs(got - target).max())
