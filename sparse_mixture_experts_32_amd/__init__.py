"""Mixtral sparse-MoE layer forward on AMD MI355X (gfx950).

A thin ctypes binding over ``libmoe_mi355x.so`` (C ABI in
``include/moe_mi355x.h``).  Every function here only marshals torch tensors
into pointers, sizes and the current HIP stream; all arithmetic runs in the
library's HIP kernels.  If the library is missing the functions raise
``MoeLibraryMissing`` -- there is no fallback path.

The layer ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析", aiqianji.com, section
2.1.1): y = sum over the top-K experts of Softmax(TopK(x W_g))_i *
SwiGLU_i(x), SwiGLU_i(x) = (SiLU(x W1_i) * (x W3_i)) W2_i.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import library_path

__all__ = [
    "MoeError", "MoeLibraryMissing", "F32", "BF16", "WS_ITEMS",
    "load_library", "plan_for", "workspace_size", "workspace_layout", "moe_forward",
    "moe_router_topk", "moe_route_permute", "moe_expert_swiglu", "moe_swiglu_finish",
    "moe_expert_down",
    "moe_combine", "moe_rmsnorm", "moe_stack_forward", "EXPORTED_SYMBOLS",
    "moe_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_routing_stats",
    "stack_workspace_size", "ABI_VERSION",
    "swa_workspace_size", "swa_attention", "swa_cache_append",
]

F32 = 0
BF16 = 1
WS_ITEMS = ("topk_idx", "topk_w", "offsets", "sorted_token", "pos", "H", "O", "scratch")

EXPORTED_SYMBOLS = (
    "moe_status_str", "moe_last_error", "moe_abi_version", "moe_plan_for", "moe_workspace_size",
    "moe_workspace_layout", "moe_forward", "moe_router_topk", "moe_route_permute",
    "moe_expert_swiglu", "moe_swiglu_finish", "moe_expert_down", "moe_combine", "moe_rmsnorm",
    "swa_workspace_size", "swa_attention", "swa_cache_append", "moe_forward_noalloc",
    "moe_routing_stats", "moe_stack_workspace_size", "moe_stack_forward",
)

# Size of the library's static scratch behind moe_forward_noalloc
# (MOE_NOALLOC_SCRATCH_BYTES in the header).
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__("%s: %s" % (name, detail))
        self.status = status
        self.name = name


_lib = None
_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_p = ctypes.c_void_p
_c_sz = ctypes.c_size_t


ABI_VERSION = 5   # MOE_ABI_VERSION of include/moe_mi355x.h that this binding speaks


class _Plan(ctypes.Structure):
    _fields_ = [("swiglu_splits", ctypes.c_int32), ("down_splits", ctypes.c_int32),
                ("swiglu_scratch_bytes", ctypes.c_size_t), ("streaming", ctypes.c_int32),
                ("down_scratch_bytes", ctypes.c_size_t), ("swiglu_mixed", ctypes.c_int32),
                ("weights_nt", ctypes.c_int32)]


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle of libmoe_mi355x.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise MoeLibraryMissing(
            "libmoe_mi355x.so not built (expected at %s); run "
            "`python -m sparse_mixture_experts_32_amd.build`" % path)
    lib = ctypes.CDLL(path)
    sig = {
        "moe_status_str": (ctypes.c_char_p, [_c_i32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (_c_i32, []),
        "moe_plan_for": (_c_i32, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                  ctypes.POINTER(_Plan)]),
        "moe_workspace_size": (_c_i32, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                        ctypes.POINTER(_c_sz)]),
        "moe_workspace_layout": (_c_i32, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                          ctypes.POINTER(_c_sz)]),
        "moe_forward": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32,
                                 _c_i32, _c_i32, _c_p, _c_i32, _c_i32, _c_p, _c_sz, _c_p]),
        "moe_forward_noalloc": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                         _c_i32, _c_i32, _c_i32, _c_p, _c_i32, _c_i32, _c_p]),
        "moe_router_topk": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_p,
                                     _c_p, _c_p, _c_p]),
        "moe_route_permute": (_c_i32, [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p]),
        "moe_routing_stats": (_c_i32, [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
        "moe_expert_swiglu": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                                       _c_i32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
        "moe_swiglu_finish": (_c_i32, [_c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_p,
                                       _c_p, _c_p]),
        "moe_expert_down": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                     _c_p, _c_p, _c_p, _c_sz, _c_p]),
        "moe_combine": (_c_i32, [_c_p, _c_i32, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_i32,
                                 _c_i32, _c_p]),
        "moe_rmsnorm": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_float, _c_i32, _c_p]),
        "moe_stack_workspace_size": (_c_i32, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                              ctypes.POINTER(_c_sz)]),
        "moe_stack_forward": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_i64,
                                       _c_i64, _c_i32, _c_i32, ctypes.c_float, _c_i32, _c_p, _c_p,
                                       _c_sz, _c_p]),
        "swa_workspace_size": (_c_i32, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                        ctypes.POINTER(_c_sz)]),
        "swa_attention": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                   _c_i32, _c_i32, _c_i32, _c_p, _c_i32, _c_p, _c_sz, _c_p]),
        "swa_cache_append": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                                      _c_p, _c_p, _c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise MoeLibraryMissing(
            "%s speaks C ABI version %d, this binding version %d; rebuild it with "
            "`python -m sparse_mixture_experts_32_amd.build`" % (path, lib.moe_abi_version(),
                                                                ABI_VERSION))
    if path == library_path():
        _lib = lib
    return lib


def _check(status: int, lib=None):
    if status != 0:
        lib = lib or load_library()
        raise MoeError(status, lib.moe_status_str(status).decode(),
                       lib.moe_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])
    return arr


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def plan_for(T, d, d_ff, E, K, dtype) -> dict:
    """The kernel plan moe_forward (and the stage calls) use for a shape."""
    lib = load_library()
    p = _Plan()
    _check(lib.moe_plan_for(T, d, d_ff, E, K, dtype, ctypes.byref(p)), lib)
    return dict(swiglu_splits=p.swiglu_splits, down_splits=p.down_splits,
                swiglu_scratch_bytes=p.swiglu_scratch_bytes, streaming=bool(p.streaming),
                down_scratch_bytes=p.down_scratch_bytes, swiglu_mixed=bool(p.swiglu_mixed),
                weights_nt=bool(p.weights_nt))


def workspace_size(T, d, d_ff, E, K, dtype) -> int:
    lib = load_library()
    out = _c_sz(0)
    _check(lib.moe_workspace_size(T, d, d_ff, E, K, dtype, ctypes.byref(out)), lib)
    return out.value


def workspace_layout(T, d, d_ff, E, K, dtype) -> dict:
    lib = load_library()
    arr = (_c_sz * len(WS_ITEMS))()
    _check(lib.moe_workspace_layout(T, d, d_ff, E, K, dtype, arr), lib)
    return dict(zip(WS_ITEMS, list(arr)))


def workspace_views(ws: torch.Tensor, T, d, d_ff, E, K, dtype) -> dict:
    """Typed views of the intermediates moe_forward leaves in a workspace."""
    off = workspace_layout(T, d, d_ff, E, K, dtype)
    plan = plan_for(T, d, d_ff, E, K, dtype)
    S = plan["down_splits"]
    P = T * K
    hdt = torch.bfloat16 if dtype == BF16 else torch.float32

    def view(name, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[off[name]:off[name] + nbytes].view(dt)

    return dict(
        topk_idx=view("topk_idx", P, torch.int32).view(T, K),
        topk_w=view("topk_w", P, torch.float32).view(T, K),
        offsets=view("offsets", E + 1, torch.int32),
        sorted_token=view("sorted_token", P, torch.int32),
        pos=view("pos", P, torch.int32).view(T, K),
        H=view("H", P * d_ff, hdt).view(P, d_ff),
        O=view("O", S * P * d, torch.float32).view(S, P, d),
    )


def moe_forward(x, W_g, W1, W3, W2, K, y=None, y_dtype=None, accumulate=False, workspace=None,
                stream=None):
    """y = MoE(x) (or y += MoE(x) with accumulate=True) through the HIP kernels.

    x [T, d], W_g [d, E], W1[e]/W3[e] [d, d_ff], W2[e] [d_ff, d]: bf16 or fp32
    CUDA tensors of one dtype.  y_dtype defaults to x's dtype; a bf16 layer
    may write fp32 y.  Returns y."""
    lib = load_library()
    T, d = x.shape
    E = len(W1)
    d_ff = W1[0].shape[1]
    dt = _dtype_code(x)
    if y is None:
        ydt = x.dtype if y_dtype is None else y_dtype
        y = torch.empty((T, d), dtype=ydt, device=x.device)
    ycode = _dtype_code(y)
    need = workspace_size(T, d, d_ff, E, K, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib.moe_forward(_ptr(x), _ptr(W_g), _ptr_array(W1), _ptr_array(W3), _ptr_array(W2),
                           T, d, d_ff, E, K, dt, _ptr(y), ycode, 1 if accumulate else 0,
                           _ptr(workspace), workspace.numel(), _stream(stream)), lib)
    return y


def moe_forward_noalloc(x, W_g, W1, W3, W2, K, y=None, y_dtype=None, accumulate=False,
                        stream=None):
    """moe_forward with the library's static device scratch as workspace: the
    call allocates nothing on the device (pass ``y`` to allocate nothing at
    all).  Shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES raise
    MoeError (MOE_EWORKSPACE).  Calls that overlap in time on one device race
    on the scratch."""
    lib = load_library()
    T, d = x.shape
    E = len(W1)
    d_ff = W1[0].shape[1]
    dt = _dtype_code(x)
    if y is None:
        ydt = x.dtype if y_dtype is None else y_dtype
        y = torch.empty((T, d), dtype=ydt, device=x.device)
    _check(lib.moe_forward_noalloc(_ptr(x), _ptr(W_g), _ptr_array(W1), _ptr_array(W3),
                                   _ptr_array(W2), T, d, d_ff, E, K, dt, _ptr(y), _dtype_code(y),
                                   1 if accumulate else 0, _stream(stream)), lib)
    return y


def moe_router_topk(x, W_g, K, topk_idx=None, topk_w=None, logits=None, stream=None):
    lib = load_library()
    T, d = x.shape
    E = W_g.shape[1]
    if topk_idx is None:
        topk_idx = torch.empty((T, K), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=x.device)
    _check(lib.moe_router_topk(_ptr(x), _ptr(W_g), T, d, E, K, _dtype_code(x), _ptr(topk_idx),
                               _ptr(topk_w), _ptr(logits), _stream(stream)), lib)
    return topk_idx, topk_w


def moe_route_permute(topk_idx, E, offsets=None, sorted_token=None, pos=None, stream=None):
    lib = load_library()
    T, K = topk_idx.shape
    dev = topk_idx.device
    if offsets is None:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if sorted_token is None:
        sorted_token = torch.empty(T * K, dtype=torch.int32, device=dev)
    if pos is None:
        pos = torch.empty((T, K), dtype=torch.int32, device=dev)
    _check(lib.moe_route_permute(_ptr(topk_idx), T, E, K, _ptr(offsets), _ptr(sorted_token),
                                 _ptr(pos), _stream(stream)), lib)
    return offsets, sorted_token, pos


def moe_routing_stats(topk_idx, E, counts=None, repeats=None, stream=None):
    """Per-expert pair counts (int32 [E]) and the number of first-choice
    repeats between consecutive tokens (int32 [1]) of one layer's routing
    table topk_idx [T, K]."""
    lib = load_library()
    T, K = topk_idx.shape
    dev = topk_idx.device
    if counts is None:
        counts = torch.zeros(E, dtype=torch.int32, device=dev)
    if repeats is None:
        repeats = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(lib.moe_routing_stats(_ptr(topk_idx), T, E, K, _ptr(counts), _ptr(repeats),
                                 _stream(stream)), lib)
    return counts, repeats


def moe_expert_swiglu(x, W1, W3, K, offsets, sorted_token, H=None, scratch=None, stream=None,
                      finish=True):
    """H for every expert-sorted row.  When the plan's W1/W3 product leaves
    partial sums (plan_for(...)["swiglu_splits"] > 0, small batches) they land
    in ``scratch`` and, when ``finish`` is true, moe_swiglu_finish completes H
    (pass finish=False to launch it yourself)."""
    lib = load_library()
    T, d = x.shape
    E = len(W1)
    d_ff = W1[0].shape[1]
    dt = _dtype_code(x)
    if H is None:
        H = torch.empty((T * K, d_ff), dtype=x.dtype, device=x.device)
    need = plan_for(T, d, d_ff, E, K, dt)["swiglu_scratch_bytes"] if T else 0
    if scratch is None and need:
        scratch = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib.moe_expert_swiglu(_ptr(x), _ptr_array(W1), _ptr_array(W3), T, d, d_ff, E, K, dt,
                                 _ptr(offsets), _ptr(sorted_token), _ptr(H), _ptr(scratch),
                                 scratch.numel() if scratch is not None else 0,
                                 _stream(stream)), lib)
    if finish and T:
        moe_swiglu_finish(scratch, T, d, d_ff, E, K, dt, offsets, H, stream)
    return H


def moe_swiglu_finish(scratch, T, d, d_ff, E, K, dtype, offsets, H, stream=None):
    lib = load_library()
    _check(lib.moe_swiglu_finish(_ptr(scratch), T, d, d_ff, E, K, dtype, _ptr(offsets), _ptr(H),
                                 _stream(stream)), lib)
    return H


def moe_expert_down(H, W2, T, K, offsets, O=None, scratch=None, stream=None):
    """O has shape [down_splits, T*K, d] (see plan_for).  scratch: at least
    plan_for(...)["down_scratch_bytes"] bytes (allocated here when None)."""
    lib = load_library()
    E = len(W2)
    d_ff, d = W2[0].shape
    dt = _dtype_code(H)
    plan = plan_for(T, d, d_ff, E, K, dt) if T else None
    if O is None:
        S = plan["down_splits"] if T else 1
        O = torch.empty((S, T * K, d), dtype=torch.float32, device=H.device)
    need = plan["down_scratch_bytes"] if T else 0
    if scratch is None and need:
        scratch = torch.empty(need, dtype=torch.uint8, device=H.device)
    _check(lib.moe_expert_down(_ptr(H), _ptr_array(W2), T, d, d_ff, E, K, dt,
                               _ptr(offsets), _ptr(O), _ptr(scratch),
                               scratch.numel() if scratch is not None else 0, _stream(stream)),
           lib)
    return O


def moe_combine(O, topk_w, pos, y=None, y_dtype=torch.float32, accumulate=False, stream=None):
    """O is [splits, T*K, d] (or [T*K, d] for one split)."""
    lib = load_library()
    T, K = topk_w.shape
    O3 = O if O.dim() == 3 else O.unsqueeze(0)
    S, _, d = O3.shape
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=O.device)
    _check(lib.moe_combine(_ptr(O3), S, _ptr(topk_w), _ptr(pos), T, d, K, _ptr(y),
                           _dtype_code(y), 1 if accumulate else 0, _stream(stream)), lib)
    return y


def moe_rmsnorm(h, out=None, eps=1e-5, stream=None):
    lib = load_library()
    T, d = h.shape
    if out is None:
        out = torch.empty_like(h)
    _check(lib.moe_rmsnorm(_ptr(h), _ptr(out), T, d, eps, _dtype_code(h), _stream(stream)), lib)
    return out


def stack_workspace_size(T, d, d_ff, E, K, dtype) -> int:
    lib = load_library()
    out = _c_sz(0)
    _check(lib.moe_stack_workspace_size(T, d, d_ff, E, K, dtype, ctypes.byref(out)), lib)
    return out.value


def moe_stack_forward(h, blocks, K, eps=1e-5, workspace=None, stats=None, stream=None):
    """A stack of pre-norm MoE blocks, h <- round(h + MoE_l(RMSNorm(h))) for
    every block l, in place on h, in one library call
    ("【DL輪読会】Mixtral of Experts" slides, "Architecture – 全体").
    ``blocks`` is a sequence of (W_g, W1s, W3s, W2s).  ``stats``, if given, is
    an int32 device tensor [L, E + 1] that receives every block's expert loads
    and first-choice repeats.  Returns h."""
    lib = load_library()
    T, d = h.shape
    L = len(blocks)
    if L == 0:
        return h
    E = len(blocks[0][1])
    d_ff = blocks[0][1][0].shape[1]
    dt = _dtype_code(h)
    if workspace is None:
        workspace = torch.empty(max(stack_workspace_size(T, d, d_ff, E, K, dt), 1),
                                dtype=torch.uint8, device=h.device)
    if stats is not None and (stats.dtype != torch.int32 or stats.numel() != L * (E + 1)):
        raise ValueError("stats must be int32 with L * (E + 1) elements")
    W_g = _ptr_array([b[0] for b in blocks])
    W1 = _ptr_array([t for b in blocks for t in b[1]])
    W3 = _ptr_array([t for b in blocks for t in b[2]])
    W2 = _ptr_array([t for b in blocks for t in b[3]])
    _check(lib.moe_stack_forward(_ptr(h), W_g, W1, W3, W2, L, T, d, d_ff, E, K,
                                 ctypes.c_float(eps), dt, _ptr(stats), _ptr(workspace),
                                 workspace.numel(), _stream(stream)), lib)
    return h


# ---------------------------------------------------------------------------
# Attention sub-block: sliding-window grouped-query attention with a
# rolling-buffer cache ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析",
# aiqianji.com, sections 1.1 and 1.2.1-1.2.3).

def swa_workspace_size(B, T, W, n_heads, n_kv_heads, head_dim=128) -> int:
    lib = load_library()
    n = _c_sz()
    _check(lib.swa_workspace_size(B, T, W, n_heads, n_kv_heads, head_dim, ctypes.byref(n)), lib)
    return n.value


def swa_attention(q, k_new, v_new, k_cache, v_cache, pos0, W, out=None, out_dtype=None,
                  workspace=None, stream=None):
    """Attention of one chunk: q [B, T, H, hd], k_new/v_new [B, T, KVH, hd],
    caches [B, W, KVH, hd] (bf16), pos0 [B] int32 (device).  The cache is read
    as it stands; call ``swa_cache_append`` afterwards.  Returns out
    [B, T, H, hd] (bf16, or fp32 with out_dtype=torch.float32)."""
    lib = load_library()
    B, T, H, hd = q.shape
    KVH = k_new.shape[2]
    if pos0.dtype != torch.int32:
        raise TypeError("pos0 must be int32")
    if out is None:
        out = torch.empty((B, T, H, hd), dtype=out_dtype or q.dtype, device=q.device)
    need = swa_workspace_size(B, T, W, H, KVH, hd)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.swa_attention(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                             _ptr(pos0), B, T, W, H, KVH, hd, _ptr(out), _dtype_code(out),
                             _ptr(workspace) if need else None,
                             workspace.numel() if (need and workspace is not None) else 0,
                             _stream(stream)), lib)
    return out


def swa_cache_append(k_new, v_new, pos0, k_cache, v_cache, stream=None):
    """Write the chunk's keys and values into the rolling buffer, position p
    to slot p mod W (section 1.2.2)."""
    lib = load_library()
    B, T, KVH, hd = k_new.shape
    W = k_cache.shape[1]
    _check(lib.swa_cache_append(_ptr(k_new), _ptr(v_new), _ptr(pos0), B, T, W, KVH, hd,
                                _ptr(k_cache), _ptr(v_cache), _stream(stream)), lib)
    return k_cache, v_cache
