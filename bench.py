"""Throughput of the Mixtral sparse-MoE layer forward on one MI355X.

One step = one forward of the layer (router + top-2 + softmax, dispatch
tables, W1/W3 SwiGLU grouped GEMM, W2 grouped GEMM, combine) over one batch
of seeded synthetic Mixtral-shape tokens, inputs resident in HBM.  The step is
issued as the five C-ABI stage calls (the same kernels and launch shapes that
moe_forward enqueues) so that HIP events on the launch stream can time each
kernel inside the timed region.

Prints ONE JSON line: the headline workload is 8-token decode (d=4096,
d_ff=14336, E=8, K=2, bf16); the 512- and 4096-token layers are timed the
same way and reported under "sweep".  A CPU leg times the float64 oracle on a
bounded sample (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_mixture_experts_32_amd as M  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
NOMINAL_SCLK_GHZ = 2.4          # the clock behind the 2.5 PFLOP/s figure
HEADLINE = "decode_bf16_T8"
SWEEP = ("mid_bf16_T512", "prefill_bf16_T4096_zipf")
DECODE_SWEEP_T = (1, 2, 4, 16, 32, 64)
STACK = "stack32_bf16_T4096"
DECODE_STACK_T = 8
SWEEP_MIN_STEPS = {"mid_bf16_T512": 50, "prefill_bf16_T4096_zipf": 20}
CPU_SAMPLE_TOKENS = 64          # tokens of a sweep workload the oracle runs for its baseline
STACK_STEPS = {4096: 5, 8: 20}  # timed steps of the 32-block stacks
STAGES = ("router_topk", "route_permute", "expert_swiglu", "swiglu_finish", "expert_down",
          "combine")


class Layer:
    """Device buffers of one workload and the staged step."""

    def __init__(self, w: W.Workload, dev):
        self.w = w
        inp = W.layer_inputs(w, dev)
        self.x, self.W_g = inp["x"], inp["W_g"]
        self.W1, self.W3, self.W2 = inp["W1"], inp["W3"], inp["W2"]
        T, d, d_ff, E, K = w.T, w.d, w.d_ff, w.E, w.K
        P = T * K
        i32 = dict(dtype=torch.int32, device=dev)
        self.topk_idx = torch.empty((T, K), **i32)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_token = torch.empty(P, **i32)
        self.pos = torch.empty((T, K), **i32)
        self.plan = M.plan_for(T, d, d_ff, E, K, M.BF16)
        self.H = torch.empty((P, d_ff), dtype=torch.bfloat16, device=dev)
        self.O = torch.empty((self.plan["down_splits"], P, d), dtype=torch.float32, device=dev)
        # one scratch for the W1/W3 partial sums and the W2 tail pieces (used in turn)
        self.scratch = torch.empty(max(self.plan["swiglu_scratch_bytes"],
                                       self.plan["down_scratch_bytes"], 16),
                                   dtype=torch.uint8, device=dev)
        self.y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(M.workspace_size(T, d, d_ff, E, K, M.BF16), dtype=torch.uint8,
                              device=dev)

    def step(self, events=None):
        w = self.w
        ev = events or [None] * (len(STAGES) + 1)
        s = torch.cuda.current_stream()

        def mark(i):
            if ev[i] is not None:
                ev[i].record(s)

        mark(0)
        M.moe_router_topk(self.x, self.W_g, w.K, self.topk_idx, self.topk_w)
        mark(1)
        M.moe_route_permute(self.topk_idx, w.E, self.offsets, self.sorted_token, self.pos)
        mark(2)
        M.moe_expert_swiglu(self.x, self.W1, self.W3, w.K, self.offsets, self.sorted_token, self.H,
                            self.scratch, finish=False)
        mark(3)
        M.moe_swiglu_finish(self.scratch, w.T, w.d, w.d_ff, w.E, w.K, M.BF16, self.offsets,
                            self.H)
        mark(4)
        M.moe_expert_down(self.H, self.W2, w.T, w.K, self.offsets, self.O, scratch=self.scratch)
        mark(5)
        M.moe_combine(self.O, self.topk_w, self.pos, self.y)
        mark(6)

    def forward_call(self):
        w = self.w
        M.moe_forward(self.x, self.W_g, self.W1, self.W3, self.W2, w.K, y=self.y,
                      workspace=self.ws)

    def counts(self):
        off = self.offsets.cpu().numpy()
        return np.diff(off)

    def routing_stats(self):
        """Expert load and the share of consecutive tokens whose first-choice
        expert repeats (uniform independent routing gives about 1/E), from
        the routing-statistics kernel on the layer's routing table."""
        counts, repeats = M.moe_routing_stats(self.topk_idx, self.w.E)
        T = self.w.T
        rep = int(repeats.item()) / (T - 1) if T > 1 else None
        return dict(expert_counts=counts.cpu().numpy().tolist(),
                    first_choice_repeat_rate=None if rep is None else round(rep, 4))


def algorithmic(w: W.Workload, counts):
    """Algorithmic bytes and flops of the layer and of its two GEMM kernels.
    Bytes count each needed operand once: x, W_g, the weights of experts that
    received tokens, y; H/O round trips are implementation traffic."""
    n_act = int(np.sum(np.asarray(counts) > 0))
    P = w.T * w.K
    wbytes = w.d * w.d_ff * 2
    layer_bytes = 2 * w.T * w.d + 2 * w.d * w.E + n_act * 3 * wbytes + 2 * w.T * w.d
    layer_flops = P * 6 * w.d * w.d_ff + 2 * w.T * w.d * w.E
    g1_bytes = n_act * 2 * wbytes + 2 * w.T * w.d + P * w.d_ff * 2
    g1_flops = P * 4 * w.d * w.d_ff
    g2_bytes = n_act * wbytes + P * w.d_ff * 2 + P * w.d * 4
    g2_flops = P * 2 * w.d * w.d_ff
    return dict(n_active=n_act, layer_bytes=layer_bytes, layer_flops=layer_flops,
                swiglu_bytes=g1_bytes, swiglu_flops=g1_flops, down_bytes=g2_bytes,
                down_flops=g2_flops)


def time_layer(layer: Layer, steps: int, warmup: int):
    """The timed step is one moe_forward call (all kernels of the layer on the
    current stream, no host synchronisation inside): `steps` of them between
    two synchronisations.  A second pass runs the same kernels through the
    stage entry points with HIP events between them, for per-kernel times.
    Returns (wall seconds of the moe_forward steps, per-stage median ms, wall
    seconds of the staged steps).  Medians: an event pair also times any
    idle gap while the host is late with the next launch, and one such
    stall would dominate a mean."""
    for _ in range(warmup):
        layer.forward_call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward_call()
    torch.cuda.synchronize()
    wall_fwd = time.perf_counter() - t0
    # staged pass: the same kernels, HIP events between the stages
    for _ in range(max(1, warmup // 2)):
        layer.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        layer.step(evs[i])
    torch.cuda.synchronize()
    wall_staged = time.perf_counter() - t1
    per_stage = {name: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs]))
                 for j, name in enumerate(STAGES)}
    return wall_fwd, per_stage, wall_staged


FLUSH_BYTES = 1 << 30


def time_cold(layer: Layer, steps: int):
    """Each step timed alone with HIP events after writing a 1 GiB buffer, so
    neither L2 nor the 256 MB Infinity Cache holds a tail of the weights from
    the previous step: moe_forward steps (percentiles of the whole call), then
    staged steps (per-stage medians, for the kernel roofline)."""
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=layer.x.device)
    tot = []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.forward_call()
        e1.record()
        torch.cuda.synchronize()
        tot.append(e0.elapsed_time(e1))
    per = []
    for i in range(steps):
        flush.fill_((i + 7) & 0xFF)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
        layer.step(evs)
        torch.cuda.synchronize()
        per.append([evs[j].elapsed_time(evs[j + 1]) for j in range(len(STAGES))])
    del flush
    per = np.asarray(per)
    tot = np.asarray(tot)
    return dict(steps=steps, ms_median=round(float(np.median(tot)), 4),
                ms_p10=round(float(np.percentile(tot, 10)), 4),
                ms_p90=round(float(np.percentile(tot, 90)), 4),
                staged_ms_median=round(float(np.median(per.sum(axis=1))), 4),
                stage_ms={name: round(float(np.median(per[:, j])), 4) for j, name in enumerate(STAGES)})


# The W1/W3 stage is one launch of the kernel below (the split finish is a
# separate stage); its measured HBM traffic sits in the committed counter
# summary, keyed by kernel, workload and the sha256 of the kernel's source.
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_32_amd", "csrc")


def swiglu_kernel(plan):
    """(kernel name as the profiler prints it, source file) of the W1/W3
    stage: the streaming kernel in its fused form, the per-matrix streaming
    kernel over a persistent grid, the tiled kernel with a tile shape per
    expert, or the tiled kernel with 256 x 256 tiles."""
    if plan["streaming"]:
        if plan["swiglu_splits"] == 0:
            return "stream_gemm_kernel<1, 1>", "expert_stream_bf16.hip"
        return "stream_sk_kernel", "expert_stream_bf16.hip"
    if plan.get("swiglu_mixed"):
        return "tiled_mixed_kernel", "expert_tiled_bf16.hip"
    nt = "true" if plan.get("weights_nt") else "false"
    return "tiled_gemm_kernel<256, true, 256, %s>" % nt, "expert_tiled_bf16.hip"


def measured_traffic(workload, plan):
    """Calibrated FETCH+WRITE bytes per dispatch of the W1/W3 kernel, or None
    when no row matches this workload or the kernel source changed since the
    counters were taken."""
    kernel, src = swiglu_kernel(plan)
    try:
        import hashlib
        sha = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
        rows = [ln.split("|") for ln in open(COUNTERS) if not ln.startswith("#") and "|" in ln]
    except OSError:
        return None
    for r in rows:
        r = [c.strip() for c in r]
        if len(r) == 8 and r[0] == kernel and r[1] == workload and r[2] == sha:
            return int(r[7])
    return None


def traced_avg_ms(workload, plan):
    """Average duration (ms) of the W1/W3 kernel in the committed rocprofv3
    kernel-trace summary of this workload, or None when there is none or the
    kernel's source changed since the trace was taken."""
    kernel, src = swiglu_kernel(plan)
    path = os.path.join(ROOT, "profiles", "%s_kernel_trace.txt" % workload)
    try:
        import hashlib
        sha = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
        text = open(path).read()
    except OSError:
        return None
    if ("%s: %s" % (src, sha)) not in text:
        return None
    for ln in text.splitlines():
        r = [c.strip() for c in ln.split("|")]
        if not ln.startswith("#") and len(r) >= 3 and r[0] == kernel:
            return float(r[2]) / 1e3
    return None


TILED_COUNTERS = os.path.join(ROOT, "profiles", "prefill_bf16_T4096_zipf_tiled_counters.txt")


def measured_sclk(kernel, src):
    """Clock (GHz) the kernel ran at in the committed core-counter summary
    (GRBM_GUI_ACTIVE per XCD over the traced duration), or None when it has no
    row for the kernel or the kernel's source changed since."""
    try:
        import hashlib
        sha = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
        text = open(TILED_COUNTERS).read()
    except OSError:
        return None
    if ("%s: %s" % (src, sha)) not in text:
        return None
    for ln in text.splitlines():
        r = [c.strip() for c in ln.split("|")]
        if not ln.startswith("#") and len(r) >= 3 and r[0] == kernel:
            return float(r[2])
    return None


def roofline_for(w, alg, per_stage_ms, plan):
    """Roofline object of the W1/W3 kernel: `frac` from its HIP-event time in
    this run, `frac_trace` from the average duration in the committed kernel
    trace (null when that trace is of another source)."""
    g1_ms = per_stage_ms["expert_swiglu"]
    intensity = alg["swiglu_flops"] / alg["swiglu_bytes"]
    kernel = swiglu_kernel(plan)[0]
    traffic = measured_traffic(w.name, plan)
    tr_ms = traced_avg_ms(w.name, plan)
    if intensity < 312:
        work, scale, peak, bound, unit = alg["swiglu_bytes"], 1e9, HBM_PEAK_GBS, "hbm", "GB/s"
    else:
        work, scale, peak, bound, unit = (alg["swiglu_flops"], 1e12, MFMA_BF16_PEAK_TFLOPS,
                                          "mfma", "TFLOP/s")
    achieved = work / (g1_ms * 1e-3) / scale
    out = dict(kernel=kernel, bound=bound, achieved=round(achieved, 1), peak=peak, unit=unit,
               frac=round(achieved / peak, 4), traffic=traffic, avg_ms=round(g1_ms, 4),
               trace_avg_ms=None if tr_ms is None else round(tr_ms, 4),
               frac_trace=None if tr_ms is None else round(work / (tr_ms * 1e-3) / scale / peak,
                                                           4))
    if bound == "mfma":
        # the matrix peak at the clock the part held under this kernel
        sclk = measured_sclk(kernel, swiglu_kernel(plan)[1])
        if sclk is not None:
            at = peak * sclk / NOMINAL_SCLK_GHZ
            out.update(sclk_ghz=sclk, peak_at_sclk=round(at, 1), frac_at_sclk=round(achieved / at, 4))
    return out


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(layer: Layer, max_tokens: int = 8, min_s: float = 10.0):
    """Float64 oracle on the first `max_tokens` tokens of the workload (all 8
    for decode), weights copied to host outside the timed region, repeated
    until about `min_s` seconds of CPU work (at least 3 runs, or 1 when a run
    takes longer than min_s)."""
    from oracle import moe_oracle as O
    threads = blas_threads()
    w = layer.w
    n = min(max_tokens, w.T)
    x = layer.x[:n].float().cpu().numpy()
    Wg = layer.W_g.float().cpu().numpy()
    W1 = [t.float().cpu().numpy() for t in layer.W1]
    W3 = [t.float().cpu().numpy() for t in layer.W3]
    W2 = [t.float().cpu().numpy() for t in layer.W2]
    reps, t0 = 0, time.perf_counter()
    while True:
        y_ref, aux = O.moe_forward(x, Wg, W1, W3, W2, w.K, faithful=True)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s and (reps >= 3 or el / reps >= min_s / 3):
            break
    dt = (time.perf_counter() - t0) / reps
    del W1, W3, W2
    base = dict(value=round(n / dt, 3), unit="tokens/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(),
                sample="first %d of %d tokens of %s, float64 oracle in faithful mode, "
                       "%.2f s per run, mean of %d runs" % (n, w.T, w.name, dt, reps))
    return base, parity_against(layer, n, y_ref, aux)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parity_against(layer: Layer, n, y_ref, aux):
    """The layer's GPU outputs for its first n tokens against the oracle
    output the CPU leg computed: routing of decided tokens (fp64 margin
    between the K-th and (K+1)-th logit above 1e-3), gate weights, the fp32
    output's max error over rms, and the bf16 store = RNE(fp32 output)."""
    w = layer.w
    K = w.K
    ws = torch.empty(M.workspace_size(w.T, w.d, w.d_ff, w.E, K, M.BF16), dtype=torch.uint8,
                     device=layer.x.device)
    y32 = M.moe_forward(layer.x, layer.W_g, layer.W1, layer.W3, layer.W2, K,
                        y_dtype=torch.float32, workspace=ws)
    views = M.workspace_views(ws, w.T, w.d, w.d_ff, w.E, K, M.BF16)
    yb = M.moe_forward(layer.x, layer.W_g, layer.W1, layer.W3, layer.W2, K)
    torch.cuda.synchronize()
    gi = views["topk_idx"][:n].cpu().numpy()
    gw = views["topk_w"][:n].cpu().numpy()
    srt = -np.sort(-aux["logits"], axis=1)
    decided = srt[:, K - 1] - srt[:, K] > 1e-3 if K < w.E else np.ones(n, dtype=bool)
    ordered = decided & np.all(srt[:, :K - 1] - srt[:, 1:K] > 1e-3, axis=1)
    set_ok = np.array([sorted(gi[t]) == sorted(aux["idx"][t]) for t in range(n)])
    rank_ok = np.all(gi == aux["idx"], axis=1)
    y = y32[:n].double().cpu().numpy()
    rows = decided & set_ok
    err = (float(np.abs(y[rows] - y_ref[rows]).max() / np.sqrt(np.mean(y_ref[rows] ** 2)))
           if rows.any() else None)
    return dict(tokens=int(n), decided=int(decided.sum()),
                expert_set_mismatches=int(np.sum(decided & ~set_ok)),
                rank_order_mismatches=int(np.sum(ordered & ~rank_ok)),
                max_gate_weight_err=float(np.abs(gw - aux["w"])[ordered & rank_ok].max())
                if np.any(ordered & rank_ok) else None,
                rel_err_faithful=err, tol=1e-2,
                bf16_store_is_rne_of_fp32=bool(torch.equal(yb, y32.to(torch.bfloat16))))


def input_record(w, layer):
    """The workload's seed and the SHA-256 of the token and router bytes the
    GPU consumed (the expert weights come from per-tensor seeds derived from
    the same seed)."""
    import hashlib

    def sha(t):
        return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()
    return dict(seed=w.seed, x_sha256=sha(layer.x), W_g_sha256=sha(layer.W_g))


def run_workload(name, dev, steps, warmup):
    w = W.WORKLOADS[name]
    layer = Layer(w, dev)
    layer.step()
    torch.cuda.synchronize()
    counts = layer.counts()
    wall, per_stage, wall_staged = time_layer(layer, steps, warmup)
    alg = algorithmic(w, counts)
    ms = wall / steps * 1e3
    res = dict(workload=name, T=w.T, steps=steps, ms_per_step=round(ms, 4),
               inputs=input_record(w, layer),
               tokens_per_s=round(w.T * steps / wall, 1),
               ms_per_step_staged=round(wall_staged / steps * 1e3, 4),
               stage_ms={k: round(v, 4) for k, v in per_stage.items()},
               n_active_experts=alg["n_active"], expert_counts=counts.tolist(),
               plan=layer.plan, routing=layer.routing_stats(), warmup=warmup,
               layer_roofline_frac=round(max(alg["layer_bytes"] / (HBM_PEAK_GBS * 1e9),
                                             alg["layer_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                                         / (ms * 1e-3), 4),
               roofline=roofline_for(w, alg, per_stage, layer.plan))
    cold = time_cold(layer, steps)
    cold["roofline"] = roofline_for(w, alg, cold["stage_ms"], layer.plan)
    res["cold_cache"] = cold
    return res, layer


# the attention kernel each workload runs: chunks of 64 tokens or more take
# two 16-token tiles per wave, shorter ones one tile
ATTN_KERNEL = {True: "swa_attn_kernel<2>", False: "swa_attn_kernel<1>"}
ATTN_COUNTERS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                             "attn_counters.txt")


def attn_sclk(kernel, workload):
    """Clock (GHz) the attention kernel ran at in the committed counters, or
    None (no clock for short dispatches, or swa_attention.hip changed)."""
    try:
        import hashlib
        sha = hashlib.sha256(open(os.path.join(CSRC, "swa_attention.hip"), "rb").read()).hexdigest()
        text = open(ATTN_COUNTERS).read()
    except OSError:
        return None
    if ("swa_attention.hip: " + sha) not in text:
        return None
    for ln in text.splitlines():
        r = [c.strip() for c in ln.split("|")]
        if not ln.startswith("#") and len(r) >= 7 and r[0] == kernel and r[1] == workload:
            try:
                return float(r[6])
            except ValueError:
                return None
    return None


def attn_traffic(kernel, workload):
    """Calibrated FETCH+WRITE bytes per dispatch of the attention kernel, or
    None when no row matches or swa_attention.hip changed since the counters
    were taken."""
    try:
        import hashlib
        sha = hashlib.sha256(open(os.path.join(CSRC, "swa_attention.hip"), "rb").read()).hexdigest()
        text = open(ATTN_COUNTERS).read()
    except OSError:
        return None
    if ("swa_attention.hip: " + sha) not in text:
        return None
    for ln in text.splitlines():
        r = [c.strip() for c in ln.split("|")]
        if not ln.startswith("#") and len(r) >= 6 and r[0] == kernel and r[1] == workload:
            return int(r[5])
    return None


def run_attention(dev, steps, warmup, cpu=True):
    """The attention sub-block (sliding-window GQA with the rolling cache):
    decode (8 sequences, one token each, full wrapped cache) and the prefill
    of a 4096-token chunk after a previous chunk.  Each entry times
    swa_attention (and the cache append) with HIP events, inputs resident."""
    out = []
    for name, w in W.ATTN_WORKLOADS.items():
        inp = W.attn_inputs(w, dev)
        ws = torch.empty(max(M.swa_workspace_size(w.B, w.T, w.W, w.H, w.KVH), 16),
                         dtype=torch.uint8, device=dev)
        o = torch.empty((w.B, w.T, w.H, w.hd), dtype=torch.bfloat16, device=dev)
        kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()

        def attn():
            M.swa_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"],
                            inp["v_cache"], inp["pos0"], w.W, out=o, workspace=ws)

        def append():
            M.swa_cache_append(inp["k_new"], inp["v_new"], inp["pos0"], kc, vc)

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        ms = timed(attn)
        ms_append = timed(append)
        # keys each query attends to: the window, capped by the positions that exist
        keys = sum(min(w.W, p + t + 1) for p in w.pos0 for t in range(w.T))
        flops = 4.0 * keys * w.H * w.hd                      # q.k and p.v, 2 flops per MAC
        cache_rows = sum(min(w.W - 1, p) for p in w.pos0)    # cache positions read
        kv_bytes = 2 * 2 * w.KVH * w.hd * (cache_rows + w.B * w.T)
        io_bytes = 2 * w.B * w.T * w.H * w.hd * 2            # q read, out written
        alg_bytes = kv_bytes + io_bytes
        t_roof = max(alg_bytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
        bound = "hbm" if alg_bytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) \
            else "mfma"
        achieved = (alg_bytes / (ms * 1e-3) / 1e9 if bound == "hbm"
                    else flops / (ms * 1e-3) / 1e12)
        peak = HBM_PEAK_GBS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS
        kernel = ATTN_KERNEL[w.T >= 64]
        res = dict(workload=name, B=w.B, T=w.T, W=w.W, heads=w.H, kv_heads=w.KVH,
                   pos0=list(w.pos0), ms_per_call=round(ms, 4),
                   tokens_per_s=round(w.B * w.T / (ms * 1e-3), 1),
                   ms_cache_append=round(ms_append, 4), bound=bound,
                   algorithmic_bytes=int(alg_bytes), algorithmic_flops=flops,
                   achieved=round(achieved, 1),
                   unit="GB/s" if bound == "hbm" else "TFLOP/s",
                   roofline_frac=round(t_roof / (ms * 1e-3), 4),
                   key_splits=M.swa_workspace_size(w.B, w.T, w.W, w.H, w.KVH) > 0,
                   roofline=dict(kernel=kernel, bound=bound, achieved=round(achieved, 1),
                                 peak=peak, unit="GB/s" if bound == "hbm" else "TFLOP/s",
                                 frac=round(achieved / peak, 4),
                                 traffic=attn_traffic(kernel, name)))
        sclk = attn_sclk(kernel, name) if bound == "mfma" else None
        if sclk is not None:
            at = peak * sclk / NOMINAL_SCLK_GHZ
            res["roofline"].update(sclk_ghz=sclk, peak_at_sclk=round(at, 1),
                                   frac_at_sclk=round(achieved / at, 4))
        if cpu and w.T == 1:
            from oracle import swa_oracle as A
            t0 = time.perf_counter()
            npi = {k: v.detach().double().cpu().numpy() for k, v in inp.items() if k != "pos0"}
            t0 = time.perf_counter()
            for b in range(w.B):
                A.swa_chunk_attention(npi["q"][b], npi["k_new"][b], npi["v_new"][b],
                                      npi["k_cache"][b], npi["v_cache"][b], w.pos0[b], w.W)
            res["oracle_s"] = round(time.perf_counter() - t0, 3)
        out.append(res)
        del inp, ws, o, kc, vc
        torch.cuda.empty_cache()
    return out


def run_decode_sweep(dev, steps, warmup):
    """Small batches through the decode-shape layer (T = 1 .. 64)."""
    out = []
    for T in DECODE_SWEEP_T:
        w = W.scaled(W.WORKLOADS[HEADLINE], name="decode_bf16_T%d" % T, T=T)
        layer = Layer(w, dev)
        layer.step()
        torch.cuda.synchronize()
        wall, per_stage, _ = time_layer(layer, steps, warmup)
        out.append(dict(T=T, ms_per_step=round(wall / steps * 1e3, 4),
                        tokens_per_s=round(T * steps / wall, 1),
                        n_active_experts=int(np.sum(layer.counts() > 0)), plan=layer.plan))
        del layer
        torch.cuda.empty_cache()
    return out


def _time_stack(h, h0, run, steps, warmup):
    for _ in range(warmup):
        h.copy_(h0)
        run()
    torch.cuda.synchronize()
    t = 0.0
    for _ in range(steps):
        h.copy_(h0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        t += time.perf_counter() - t0
    return t


def run_dense_reference(dev, steps=10, warmup=3):
    """Context, not the product: hipBLASLt through torch on dense stand-ins
    for the products, bf16 with fp32 accumulation, contiguous row-major
    operands, timed with HIP events.  Prefill: all 8192 (token, expert) rows
    against one [4096, 28672] W1|W3 matrix and one [14336, 4096] W2 matrix
    (torch.matmul).  T = 512: eight equal groups of 128 rows, one per
    expert, each against its own weights (torch.bmm over [8, ...] stacks:
    the same 1.88 GB and 0.94 GB of weights as the layer reads), reported
    also as weight bytes per second.  And a square 8192^3 product: the
    library's own rate on a shape it is best at, a practical ceiling for
    bf16 matrix-core work on the part."""
    g = torch.Generator(device=dev).manual_seed(7)
    out = []
    for name, bsz, m, k, n in [("w1w3_dense", 1, 8192, 4096, 2 * 14336),
                               ("w2_dense", 1, 8192, 14336, 4096),
                               ("w1w3_8x128_batched", 8, 128, 4096, 2 * 14336),
                               ("w2_8x128_batched", 8, 128, 14336, 4096),
                               ("square_8192", 1, 8192, 8192, 8192)]:
        shape_a = (m, k) if bsz == 1 else (bsz, m, k)
        shape_b = (k, n) if bsz == 1 else (bsz, k, n)
        a = torch.randn(shape_a, generator=g, device=dev).to(torch.bfloat16)
        b = (torch.randn(shape_b, generator=g, device=dev) / k ** 0.5).to(torch.bfloat16).contiguous()
        prod = torch.matmul if bsz == 1 else torch.bmm
        for _ in range(warmup):
            prod(a, b)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            prod(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tflops = 2.0 * bsz * m * k * n / (ms * 1e-3) / 1e12
        res = dict(product=name, shape=[bsz, m, k, n] if bsz > 1 else [m, k, n], ms=round(ms, 4),
                   tflops=round(tflops, 1), mfma_frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4))
        if bsz > 1:
            res["weight_gbps"] = round(bsz * k * n * 2 / (ms * 1e-3) / 1e9, 1)
        out.append(res)
        del a, b
        torch.cuda.empty_cache()
    return out


def stack_cpu_baseline(blocks, h0, K, n_tokens=16, n_blocks=2):
    """The float64 oracle's pre-norm stack on a bounded sample: the first
    n_tokens rows through the first n_blocks blocks (weights copied to host
    outside the timed region).  Rows and blocks cost the same everywhere in
    the stack, so the rate through all L blocks is n_tokens / (L x time per
    block)."""
    from oracle import moe_oracle as O
    L = len(blocks)
    h = h0[:n_tokens].float().cpu().numpy()
    host = [(Wg.float().cpu().numpy(), [t.float().cpu().numpy() for t in W1],
             [t.float().cpu().numpy() for t in W3], [t.float().cpu().numpy() for t in W2])
            for Wg, W1, W3, W2 in blocks[:n_blocks]]
    t0 = time.perf_counter()
    O.stack_forward(h, host, K, faithful=True)
    per_block = (time.perf_counter() - t0) / n_blocks
    del host
    return dict(value=round(n_tokens / (L * per_block), 4), unit="tokens/s (through all %d "
                "blocks)" % L, cores=blas_threads(), kind="oracle", cpu_model=cpu_model(),
                sample="first %d tokens through blocks 0-%d of %d, float64 oracle in faithful "
                       "mode, %.2f s per block" % (n_tokens, n_blocks - 1, L, per_block))


def run_stacks(dev, cpu=True):
    """The 32-block stack (RMSNorm + MoE + residual per block, 90 GB of
    expert weights resident), one moe_stack_forward call per step: T = 4096
    tokens per step, and the same blocks at T = 8 (decode through all 32
    blocks, eager and replayed from a HIP graph that holds the whole step)."""
    w = W.WORKLOADS[STACK]
    blocks = [W.expert_weights(w, dev, block=b) for b in range(w.layers)]
    weights_gb = w.layers * w.E * 3 * w.d * w.d_ff * 2 / 1e9
    warmup = 1
    out = []
    for T in (w.T, DECODE_STACK_T):
        decode_steps = steps = STACK_STEPS[T]
        h0 = W.make_x(w, blocks[0][0], dev, T=T)
        h = h0.clone()
        ws = torch.empty(M.stack_workspace_size(T, w.d, w.d_ff, w.E, w.K, M.BF16),
                         dtype=torch.uint8, device=dev)

        def run():
            M.moe_stack_forward(h, blocks, w.K, workspace=ws)

        t = _time_stack(h, h0, run, steps, warmup)
        n = steps
        ms = t / n * 1e3
        res = dict(workload="stack32_bf16_T%d" % T, T=T, layers=w.layers, steps=n,
                   ms_per_step=round(ms, 3), tokens_per_s=round(T / (ms * 1e-3), 1),
                   weights_gb=round(weights_gb, 1))
        # routing statistics of every block (untimed pass): expert loads and
        # the first-choice repeat rate of consecutive tokens, from the kernels
        stats = torch.empty((w.layers, w.E + 1), dtype=torch.int32, device=dev)
        h.copy_(h0)
        M.moe_stack_forward(h, blocks, w.K, workspace=ws, stats=stats)
        st = stats.cpu().numpy()
        n_active = [int(np.sum(row[:w.E] > 0)) for row in st]
        res["layer_expert_counts"] = st[:, :w.E].tolist()
        res["layer_first_choice_repeat_rate"] = [round(float(r) / max(T - 1, 1), 4)
                                                 for r in st[:, w.E]]
        if T == w.T:
            flops = w.layers * (T * w.K * 6 * w.d * w.d_ff)
            res["achieved_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
            res["mfma_frac"] = round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        else:
            alg = sum(n_active) * 3 * w.d * w.d_ff * 2 + w.layers * (
                w.d * w.E * 2 + 3 * T * w.d * 2)
            res["n_active_per_block"] = n_active
            res["algorithmic_bytes"] = alg
            res["hbm_frac"] = round(alg / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3), 4)
            # the whole step captured once and replayed
            g = torch.cuda.CUDAGraph()
            h.copy_(h0)
            run()                      # warm (first-use attributes set outside the capture)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                run()
            tg = _time_stack(h, h0, g.replay, decode_steps, warmup)
            msg = tg / decode_steps * 1e3
            res["graph_ms_per_step"] = round(msg, 3)
            res["graph_tokens_per_s"] = round(T / (msg * 1e-3), 1)
            res["graph_hbm_frac"] = round(alg / (HBM_PEAK_GBS * 1e9) / (msg * 1e-3), 4)
            del g
        if cpu and T == w.T:
            res["cpu_baseline"] = stack_cpu_baseline(blocks, h0, w.K)
        out.append(res)
        del h, h0, ws
    del blocks
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None, help="time just this workload (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU only (the MoE layer is not sharded "
              "across GPUs); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    M.load_library()
    dev = torch.device("cuda:0")

    if args.only == "copy_calibration":
        # a plain device copy of known size: what HBM counters read for it
        # calibrates the counters of the MoE kernels
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes_read=n, copy_bytes_written=n, calls=args.steps)))
        return
    if args.only == "stack":
        print(json.dumps(run_stacks(dev, cpu=not args.no_cpu)), flush=True)
        return
    if args.only == "attention":
        print(json.dumps(run_attention(dev, args.steps, args.warmup, cpu=False)), flush=True)
        return
    if args.only:
        res, _ = run_workload(args.only, dev, args.steps, args.warmup)
        print(json.dumps(res), flush=True)
        return

    head, layer = run_workload(HEADLINE, dev, args.steps, args.warmup)
    print("# %s done: %.3f ms/step" % (HEADLINE, head["ms_per_step"]), file=sys.stderr,
          flush=True)
    cpu, parity = (None, None) if args.no_cpu else cpu_baseline(layer)
    del layer
    torch.cuda.empty_cache()
    sweep = []
    if not args.no_sweep:
        for name in SWEEP:
            # at least 50 timed steps at T = 512 and 20 at T = 4096, 10 warm-up
            r, lay = run_workload(name, dev, max(SWEEP_MIN_STEPS[name], args.steps),
                                  max(10, args.warmup))
            print("# %s done: %.3f ms/step" % (name, r["ms_per_step"]), file=sys.stderr,
                  flush=True)
            if not args.no_cpu:
                r["cpu_baseline"], r["parity"] = cpu_baseline(lay, max_tokens=CPU_SAMPLE_TOKENS,
                                                              min_s=6.0)
            sweep.append(r)
            del lay
            torch.cuda.empty_cache()
    decode_sweep = [] if args.no_sweep else run_decode_sweep(dev, max(20, args.steps), 5)
    attention = [] if args.no_sweep else run_attention(dev, max(10, args.steps // 2), 3,
                                                       cpu=not args.no_cpu)
    for r in attention:
        print("# %s done: %.4f ms/call" % (r["workload"], r["ms_per_call"]), file=sys.stderr,
              flush=True)
    stack = None if (args.no_sweep or args.no_stack) else run_stacks(dev, cpu=not args.no_cpu)
    dense = None if args.no_sweep else run_dense_reference(dev)
    for r in dense or []:
        print("# dense %s (hipBLASLt) done: %.3f ms" % (r["product"], r["ms"]), file=sys.stderr,
              flush=True)
    for r in stack or []:
        print("# %s done: %.1f ms/step" % (r["workload"], r["ms_per_step"]), file=sys.stderr,
              flush=True)
    w = W.WORKLOADS[HEADLINE]
    out = {
        "metric": "MoE-layer tokens/s at Mixtral shape (T=8/512/4096); % HBM or MFMA peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) unit-RMS tokens, N(0,1/fan_in) weights)",
        "config": {"workload": HEADLINE, "T": w.T, "d_model": w.d, "d_ff": w.d_ff,
                   "experts": w.E, "top_k": w.K, "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "parity": parity,
        "detail": {k: v for k, v in head.items() if k not in ("roofline",)},
        "sweep": sweep,
        "decode_sweep": decode_sweep,
        "stack": stack,
        "dense_reference": dense,
        "attention": attention,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
