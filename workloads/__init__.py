"""Seeded synthetic inputs for the Mixtral sparse-MoE layer forward.

Both the HIP path (through its Python binding) and the CPU oracle consume the
tensors made here; this module holds none of the layer's arithmetic (no
routing, gating or expert math), only the recipes that draw inputs.

Shapes follow "Mixtral of Experts" (xyznot.com paper page), section "Method
with key equations": hidden size 4096, 8 experts, SwiGLU width 14336, two
experts per token.  The consecutive-token locality of the prefill recipe
follows the routing analysis reported in "杀疯了的开源专家模型 Mixtral 8x7B
论文公开啦！" (redian.news), section "实验" (consecutive tokens often share an
expert).  Every tensor has its own seed, derived from the workload seed and the
tensor's name, so any one matrix can be regenerated alone.  Values are drawn in
float32 with torch's seeded generators and rounded to bfloat16 by torch's
round-to-nearest-even conversion.  The routing inputs (token rows and router
weights) are drawn on the host and copied, so a workload routes the same way
on every device; the expert matrices are drawn on the device that holds them.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

# Per-expert router bias of the skewed prefill workload: makes the share of
# (token, expert) pairs of expert e follow Zipf(1.2) over 8 experts, within
# 0.5 % on the 4096-token instance.  Written by
# ``python -m oracle.calibrate_zipf_bias`` (fixed-point iteration, first on
# standard-normal logits, then on the instance's own rows).
ZIPF_BIAS = (1.750051, 0.431113, 0.098852, -0.128279,
             -0.280979, -0.506476, -0.630174, -0.734108)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    d_ff: int
    E: int
    K: int
    dtype: str            # "f32" or "bf16": storage and MFMA input type
    x_recipe: str         # "normal", "unit_rms", "zipf_runs"
    seed: int
    layers: int = 1
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_T64", 64, 128, 256, 8, 2, "f32", "normal", 20240108,
                 description="tiny fp32 layer, x ~ N(0,1), weights N(0,1/fan_in)"),
        Workload("decode_bf16_T8", 8, 4096, 14336, 8, 2, "bf16", "unit_rms", 20240109,
                 description="Mixtral-shape decode, 8 tokens, unit-RMS N(0,1) rows"),
        Workload("mid_bf16_T512", 512, 4096, 14336, 8, 2, "bf16", "unit_rms", 20240110,
                 description="Mixtral-shape 512 tokens, near-uniform routing"),
        Workload("prefill_bf16_T4096_zipf", 4096, 4096, 14336, 8, 2, "bf16", "zipf_runs",
                 20240111,
                 description="Mixtral-shape prefill, 4096 tokens, Zipf(1.2) expert load, "
                             "runs of Geom(0.3) length sharing a base vector"),
        Workload("stack32_bf16_T4096", 4096, 4096, 14336, 8, 2, "bf16", "normal", 20240112,
                 layers=32,
                 description="32 MoE blocks joined by RMSNorm and residual add"),
    ]
}


def _seed(base: int, *names) -> int:
    h = hashlib.sha256(("%d/" % base + "/".join(str(n) for n in names)).encode()).digest()
    return int.from_bytes(h[:8], "little") & 0x7FFF_FFFF_FFFF_FFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, device, seed, out_dtype):
    g = _gen(device, seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(out_dtype)


def _unit_rms_rows(t: torch.Tensor) -> torch.Tensor:
    """Scale every row of a float32 matrix to root-mean-square 1 (input recipe
    of the Mixtral-shape workloads; float64 row norms)."""
    r = t.double().pow(2).mean(dim=1, keepdim=True).sqrt()
    return (t.double() / r).float()


def expert_weights(w: Workload, device="cpu", block: int = 0, experts=None):
    """(W_g, W1s, W3s, W2s) of one block.  W_g [d, E], W1/W3 [d, d_ff],
    W2 [d_ff, d]; every entry N(0, 1/fan_in).  W_g is drawn on the host and
    copied to ``device`` (the routing inputs are the same bytes whatever the
    device); the expert matrices are drawn on ``device``."""
    dt = w.torch_dtype
    experts = range(w.E) if experts is None else experts
    W_g = _normal((w.d, w.E), w.d ** -0.5, "cpu", _seed(w.seed, block, "W_g"), dt).to(device)
    W1s, W3s, W2s = [], [], []
    for e in experts:
        W1s.append(_normal((w.d, w.d_ff), w.d ** -0.5, device, _seed(w.seed, block, "W1", e), dt))
        W3s.append(_normal((w.d, w.d_ff), w.d ** -0.5, device, _seed(w.seed, block, "W3", e), dt))
        W2s.append(_normal((w.d_ff, w.d), w.d_ff ** -0.5, device, _seed(w.seed, block, "W2", e), dt))
    return W_g, W1s, W3s, W2s


def run_lengths(T: int, p: float, seed: int) -> np.ndarray:
    """Split T tokens into runs of Geom(p) length on {1, 2, ...}; returns the
    run id of every token."""
    rng = np.random.default_rng(seed)
    ids, run = [], 0
    while len(ids) < T:
        L = int(rng.geometric(p))
        ids.extend([run] * L)
        run += 1
    return np.asarray(ids[:T], dtype=np.int64)


def fold_bias(W_g: torch.Tensor, b) -> torch.Tensor:
    """u = W_g (W_g^T W_g)^-1 b, so that (x + u) . W_g = x . W_g + b exactly in
    real arithmetic; float64 solve on the host from W_g's stored values."""
    Wg = W_g.detach().to("cpu", torch.float64).numpy()
    u = Wg @ np.linalg.solve(Wg.T @ Wg, np.asarray(b, dtype=np.float64))
    return torch.from_numpy(u)


def zipf_rows(w: Workload, block: int = 0, T: int | None = None) -> torch.Tensor:
    """The skewed recipe's rows before the router bias, float32 on the host:
    runs of Geom(0.3) length share a base vector v ~ N(0, I), each token is
    v + 0.1 N(0, I), every row scaled to unit RMS."""
    T = w.T if T is None else T
    run = torch.from_numpy(run_lengths(T, 0.3, _seed(w.seed, block, "runs")))
    n_runs = int(run.max().item()) + 1
    base = _normal((n_runs, w.d), 1.0, "cpu", _seed(w.seed, block, "base"), torch.float32)
    noise = _normal((T, w.d), 1.0, "cpu", _seed(w.seed, block, "noise"), torch.float32)
    return _unit_rms_rows(base[run] + 0.1 * noise)


def biased_rows(t: torch.Tensor, W_g: torch.Tensor, b, dt) -> torch.Tensor:
    """Rows t moved by the folded bias u of ``fold_bias`` (float64 add on the
    host), rounded to dt."""
    u = fold_bias(W_g, b)
    return (t.double() + u[None, :]).float().to(dt)


def make_x(w: Workload, W_g: torch.Tensor, device="cpu", block: int = 0,
           T: int | None = None) -> torch.Tensor:
    """Token rows [T, d] in the workload's dtype, drawn on the host (so the
    routing of a workload does not depend on the device) and copied to
    ``device``."""
    T = w.T if T is None else T
    dt = w.torch_dtype
    if w.x_recipe == "normal":
        x = _normal((T, w.d), 1.0, "cpu", _seed(w.seed, block, "x"), dt)
    elif w.x_recipe == "unit_rms":
        t = _normal((T, w.d), 1.0, "cpu", _seed(w.seed, block, "x"), torch.float32)
        x = _unit_rms_rows(t).to(dt)
    elif w.x_recipe == "zipf_runs":
        t = zipf_rows(w, block, T)
        x = biased_rows(t, W_g, ZIPF_BIAS, dt) if w.E == len(ZIPF_BIAS) else t.to(dt)
    else:
        raise ValueError("unknown x recipe " + w.x_recipe)
    return x.to(device)


def layer_inputs(w, device="cpu", block: int = 0, T: int | None = None):
    """Everything one layer forward needs: dict with x, W_g, W1, W3, W2."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    W_g, W1s, W3s, W2s = expert_weights(w, device, block)
    x = make_x(w, W_g, device, block, T)
    return dict(x=x, W_g=W_g, W1=W1s, W3=W3s, W2=W2s, workload=w)


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (for small test sizes)."""
    d = dict(w.__dict__)
    d.update(changes)
    return Workload(**d)


def sha256_of(tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# Attention sub-block (sliding-window grouped-query attention with a rolling
# cache): seeded synthetic chunks.  q, k, v ~ N(0, 1) rounded to bf16, so the
# scaled scores q.k / sqrt(128) are ~N(0, 1); the cache is filled with N(0, 1)
# rows (any slot content is a possible history: only the slots of the last
# W - 1 positions before pos0 are ever read).

@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    T: int
    W: int
    H: int
    KVH: int
    pos0: tuple
    seed: int
    hd: int = 128


ATTN_WORKLOADS = {
    # decode: 8 sequences, one new token each, cache wrapped (position 8191 > W)
    "attn_decode_bf16_B8": AttnWorkload("attn_decode_bf16_B8", 8, 1, 4096, 32, 8, (8191,) * 8,
                                        20240201),
    # prefill of a second 4096-token chunk: attends to the previous chunk in
    # the cache through the window and causally to itself (the pages' chunking)
    "attn_prefill_bf16_T4096": AttnWorkload("attn_prefill_bf16_T4096", 1, 4096, 4096, 32, 8,
                                            (4096,), 20240202),
}


def attn_inputs(w: AttnWorkload, device="cpu") -> dict:
    """q [B,T,H,hd], k_new/v_new [B,T,KVH,hd], k_cache/v_cache [B,W,KVH,hd]
    (bf16) and pos0 [B] (int32) of an attention workload."""
    bf = torch.bfloat16
    return dict(
        q=_normal((w.B, w.T, w.H, w.hd), 1.0, device, _seed(w.seed, 0, "q"), bf),
        k_new=_normal((w.B, w.T, w.KVH, w.hd), 1.0, device, _seed(w.seed, 0, "k_new"), bf),
        v_new=_normal((w.B, w.T, w.KVH, w.hd), 1.0, device, _seed(w.seed, 0, "v_new"), bf),
        k_cache=_normal((w.B, w.W, w.KVH, w.hd), 1.0, device, _seed(w.seed, 0, "k_cache"), bf),
        v_cache=_normal((w.B, w.W, w.KVH, w.hd), 1.0, device, _seed(w.seed, 0, "v_cache"), bf),
        pos0=torch.tensor(list(w.pos0), dtype=torch.int32, device=device),
    )
