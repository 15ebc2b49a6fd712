"""Calibrate the per-expert router bias behind the skewed-load prefill workload.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

The prefill workload (T = 4096, Mixtral shape) wants expert popularity to
follow Zipf(s = 1.2): the share of the T*K (token, expert) pairs that go to the
expert of popularity rank j is proportional to 1 / j**1.2.  Its router logits
are x . W_g with unit-RMS rows x and W_g ~ N(0, 1/d), so each logit is close to
a standard normal; a bias b_e is added to logit e (folded into x by the
generator).  This script finds b by the fixed-point iteration
    b_e += 0.5 * (log p_e - log share_e(b))
on seeded standard-normal logits, measuring the shares with the oracle's own
top-K selection.  Run it as ``python -m oracle.calibrate_zipf_bias``; it prints
the vector stored as ``ZIPF_BIAS`` in ``workloads/__init__.py``.
"""

from __future__ import annotations

import numpy as np

from oracle.moe_oracle import topk_select


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


if __name__ == "__main__":
    b = calibrate()
    z = np.random.default_rng(7).standard_normal((200_000, 8))
    print("bias:", np.array2string(b, precision=6, separator=", "))
    print("target:", np.round(zipf_shares(8, 1.2), 4))
    print("check :", np.round(pair_shares(z + b, 2), 4))
