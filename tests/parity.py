"""Comparison rules between the HIP path and the CPU oracle.

Tolerances (the spec parity bar of this layer):
* expert indices and the expert-sorted permutation: bit-exact for every token
  whose routing is decided, i.e. whose oracle (float64) gap between the K-th
  and (K+1)-th logit exceeds 1e-3 (the rank order is compared where the gaps
  inside the selection exceed 1e-3 as well);
* gate weights: within 1e-5 absolute;
* outputs: max|y - y_ref| / rms(y_ref) <= 1e-4 for the float32 layer and
  <= 1e-2 for the bfloat16 layer, over decided tokens.  The bf16 layer is
  compared through its float32 pre-rounding output against the oracle in
  "faithful" mode (H rounded to bf16 like the kernels store it), and the bf16
  store must then equal round-to-nearest-even of that float32 output bit for
  bit.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O

DECIDED_GAP = 1e-3
TOL_F32 = 1e-4
TOL_BF16 = 1e-2
TOL_GATE = 1e-5


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def decided(logits64: np.ndarray, K: int):
    m_rank, m_cut = O.routing_margins(logits64, K)
    set_ok = m_cut > DECIDED_GAP
    rank_ok = set_ok & (m_rank > DECIDED_GAP)
    return set_ok, rank_ok


def check_routing(gpu_idx, gpu_w, ref_idx, ref_w, logits64, K, tokens=None):
    """gpu_* and ref_* are [n, K] arrays for the same tokens."""
    gpu_idx = np.asarray(gpu_idx)
    gpu_w = np.asarray(gpu_w, dtype=np.float64)
    set_ok, rank_ok = decided(logits64, K)
    for t in np.nonzero(set_ok)[0]:
        assert sorted(gpu_idx[t]) == sorted(ref_idx[t]), (t, gpu_idx[t], ref_idx[t])
        gw = dict(zip(gpu_idx[t].tolist(), gpu_w[t].tolist()))
        rw = dict(zip(ref_idx[t].tolist(), ref_w[t].tolist()))
        for e in rw:
            assert abs(gw[e] - rw[e]) <= TOL_GATE, (t, e, gw[e], rw[e])
    assert np.array_equal(gpu_idx[rank_ok], ref_idx[rank_ok])
    return set_ok


def check_permutation(gpu_offsets, gpu_sorted_token, ref_idx, E, K, keep_token):
    """Per-expert token lists equal after deleting tokens that are not kept."""
    _, ref_off, ref_st, _, _ = O.route_tables(ref_idx, E)
    gpu_offsets = np.asarray(gpu_offsets)
    gpu_st = np.asarray(gpu_sorted_token)
    assert gpu_offsets[0] == 0 and gpu_offsets[-1] == ref_idx.size
    for e in range(E):
        g = gpu_st[gpu_offsets[e]:gpu_offsets[e + 1]]
        r = ref_st[ref_off[e]:ref_off[e + 1]]
        assert np.all(np.diff(g) > 0)
        assert g[keep_token[g]].tolist() == r[keep_token[r]].tolist(), e


def rel_err(y, y_ref, rows=None) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if rows is not None:
        y, y_ref = y[rows], y_ref[rows]
    if y_ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(y_ref ** 2))
    return float(np.abs(y - y_ref).max() / rms)


def bf16_rne_of(y32: torch.Tensor) -> torch.Tensor:
    return y32.to(torch.bfloat16)
