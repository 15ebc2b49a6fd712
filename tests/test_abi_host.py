"""Host-side checks of the C-ABI library: it loads, exports every entry point
the header declares, and rejects bad arguments before launching anything.

Only argument combinations that fail validation are passed here (with fake,
never-dereferenced addresses), so no kernel is ever launched by these tests.
"""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_32_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE = 0, 1, 2, 3
FAKE = 0x7F0000000000          # 256-byte aligned fake device address (never used)
FAKE2 = 0x7F0100000000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.build.library_path()):
        pytest.fail("libmoe_mi355x.so is not built; run python -m sparse_mixture_experts_32_amd.build")
    return M.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:moe|swa)_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(M.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", M.build.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 5 == M.ABI_VERSION
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(4) == b"MOE_EHIP"


def test_plan(lib):
    p = M.plan_for(8, 4096, 14336, 8, 2, M.BF16)
    assert p["streaming"] and p["swiglu_splits"] >= 1 and p["down_splits"] > 1
    assert p["swiglu_scratch_bytes"] == p["swiglu_splits"] * 2 * 16 * 14336 * 4
    p = M.plan_for(32, 4096, 14336, 8, 2, M.BF16)     # fused W1/W3: H written directly
    assert p["streaming"] and p["swiglu_splits"] == 0 and p["swiglu_scratch_bytes"] == 0
    # 4096 tokens fill at least 32 x 16 W2 tiles (two rounds of 256 compute
    # units): whole-K tiles with a split last round, one slice of O, 256
    # pieces of 256 rows x 256 fp32 features
    p = M.plan_for(4096, 4096, 14336, 8, 2, M.BF16)
    assert not p["streaming"] and p["swiglu_splits"] == 0 and p["swiglu_scratch_bytes"] == 0
    assert p["down_splits"] == 1 and p["down_scratch_bytes"] == 256 * 256 * 256 * 4
    assert not p["swiglu_mixed"]
    # 512 tokens (at least 4 x 16 tiles): K splits, no scratch; W1/W3 picks
    # its tile shape per expert (at most 192 rows per expert on average)
    p = M.plan_for(512, 4096, 14336, 8, 2, M.BF16)
    assert p["down_splits"] > 1 and p["down_scratch_bytes"] == 0 and p["swiglu_mixed"]
    assert not M.plan_for(1024, 4096, 14336, 8, 2, M.BF16)["swiglu_mixed"]
    assert not M.plan_for(512, 4096, 14208, 8, 2, M.BF16)["swiglu_mixed"]   # d_ff % 256
    # weight tiles read once (non-temporal copies) up to 192 rows per expert
    assert M.plan_for(512, 4096, 14336, 8, 2, M.BF16)["weights_nt"]
    assert M.plan_for(768, 4096, 14336, 8, 2, M.BF16)["weights_nt"]
    assert not M.plan_for(769, 4096, 14336, 8, 2, M.BF16)["weights_nt"]
    assert not M.plan_for(4096, 4096, 14336, 8, 2, M.BF16)["weights_nt"]
    assert not M.plan_for(8, 4096, 14336, 8, 2, M.BF16)["weights_nt"]     # streaming
    # the tiled W2 kernel addresses its token operand (H) with 32-bit byte
    # offsets: at d_ff = 65536, 32000 rows fit (K split 4), 33000 do not and
    # W2 falls back to the unsplit grouped kernel
    assert M.plan_for(16000, 256, 65536, 8, 2, M.BF16)["down_splits"] == 4
    assert M.plan_for(16500, 256, 65536, 8, 2, M.BF16)["down_splits"] == 1
    p = M.plan_for(8, 128, 256, 8, 2, M.F32)
    assert not p["streaming"]


def test_workspace_size_and_layout(lib):
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(4096, 4096, 14336, 8, 2, 1, ctypes.byref(n)) == OK
    lay = M.workspace_layout(4096, 4096, 14336, 8, 2, 1)
    P = 8192
    assert lay["topk_idx"] == 0 and all(v % 256 == 0 for v in lay.values())
    assert lay["O"] - lay["H"] >= P * 14336 * 2
    assert n.value >= lay["O"] + P * 4096 * 4
    assert lib.moe_workspace_size(8, 4096, 14336, 8, 2, 1, None) == EINVAL
    assert lib.moe_workspace_size(8, 4000, 14336, 8, 2, 1, ctypes.byref(n)) == EUNSUPPORTED
    # bf16: multiples of 64 (the grouped kernels take what the others cannot tile)
    assert lib.moe_workspace_size(8, 320, 448, 8, 2, 1, ctypes.byref(n)) == OK
    assert lib.moe_workspace_size(8, 96, 448, 8, 2, 1, ctypes.byref(n)) == EUNSUPPORTED
    assert lib.moe_workspace_size(8, 320, 480, 8, 2, 1, ctypes.byref(n)) == EUNSUPPORTED
    assert lib.moe_workspace_size(8, 4000, 14300, 8, 2, 0, ctypes.byref(n)) == OK  # fp32: any d


def _forward(lib, T=8, d=256, d_ff=256, E=8, K=2, dt=1, x=FAKE, y=FAKE2, ydt=None, ws=0x7F0200000000,
             ws_bytes=1 << 40, w_ptrs=None, wg=FAKE):
    ptrs = w_ptrs if w_ptrs is not None else [FAKE + 4096 * (i + 1) for i in range(E)]
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return lib.moe_forward(x, wg, arr, arr, arr, T, d, d_ff, E, K, dt, y,
                           dt if ydt is None else ydt, 0, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), EINVAL),
    (dict(wg=None), EINVAL),
    (dict(y=None), EINVAL),
    (dict(K=0), EINVAL),
    (dict(K=9), EINVAL),
    (dict(E=65, K=2), EINVAL),
    (dict(T=-1), EINVAL),
    (dict(dt=7), EINVAL),
    (dict(ydt=5), EINVAL),
    (dict(d=200), EUNSUPPORTED),
    (dict(d_ff=300), EUNSUPPORTED),
    (dict(dt=0, ydt=1), EUNSUPPORTED),
    (dict(x=FAKE + 2), EUNSUPPORTED),
    (dict(y=FAKE), EINVAL),                       # x aliases y
    (dict(ws=None), EWORKSPACE),
    (dict(ws_bytes=100), EWORKSPACE),
    (dict(ws=0x7F0200000010), EWORKSPACE),        # not 256-byte aligned
    (dict(ws=FAKE), EINVAL),                      # workspace overlaps x
    (dict(w_ptrs=[FAKE] * 7 + [0]), EINVAL),       # a NULL expert pointer
    (dict(w_ptrs=[FAKE + 2] * 8), EUNSUPPORTED),   # misaligned expert pointer
])
def test_forward_rejects_before_launch(lib, kwargs, status):
    got = _forward(lib, **kwargs)
    assert got == status, lib.moe_last_error()
    assert lib.moe_last_error() != b""


def test_forward_empty_batch_is_a_noop(lib):
    assert _forward(lib, T=0) == OK
    assert lib.moe_last_error() == b""


def _noalloc(lib, T, d=4096, d_ff=14336, E=8, K=2, dtype=1):
    ptrs = (ctypes.c_void_p * E)(*([FAKE] * E))
    return lib.moe_forward_noalloc(FAKE, FAKE, ptrs, ptrs, ptrs, T, d, d_ff, E, K, dtype, FAKE2,
                                   dtype, 0, None)


def test_noalloc_scratch_limit_and_noop(lib):
    """moe_forward_noalloc refuses, before touching the device, a shape whose
    workspace exceeds the static scratch; the limit in the header and in the
    binding agree; an empty batch is a no-op."""
    text = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == M.NOALLOC_SCRATCH_BYTES
    assert M.workspace_size(4096, 4096, 14336, 8, 2, M.BF16) > M.NOALLOC_SCRATCH_BYTES
    assert M.workspace_size(8, 4096, 14336, 8, 2, M.BF16) <= M.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, 4096) == EWORKSPACE
    assert b"static scratch" in lib.moe_last_error()
    assert _noalloc(lib, 8, d=100) == EUNSUPPORTED
    assert _noalloc(lib, 0) == OK


def test_stack_rejects_before_launch(lib):
    E, L = 8, 2
    ptrs = (ctypes.c_void_p * (L * E))(*([FAKE] * (L * E)))
    wg = (ctypes.c_void_p * L)(FAKE, FAKE)
    size = ctypes.c_size_t()
    assert lib.moe_stack_workspace_size(8, 4096, 14336, E, 2, 1, ctypes.byref(size)) == OK
    assert size.value >= M.workspace_size(8, 4096, 14336, E, 2, 1) + 8 * 4096 * 2

    def call(h=FAKE2, wg=wg, w1=ptrs, L=L, T=8, d=4096, ws=FAKE, nbytes=None, eps=1e-5):
        nbytes = size.value if nbytes is None else nbytes
        return lib.moe_stack_forward(h, wg, w1, ptrs, ptrs, L, T, d, 14336, E, 2,
                                     ctypes.c_float(eps), 1, None, ws, nbytes, None)

    assert call(L=0) == OK and call(T=0) == OK
    assert call(h=None) == EINVAL
    assert call(wg=(ctypes.c_void_p * L)(FAKE, None)) == EINVAL
    assert call(w1=(ctypes.c_void_p * (L * E))(*([FAKE] * (L * E - 1) + [None]))) == EINVAL
    assert call(nbytes=size.value - 1) == EWORKSPACE
    assert call(ws=FAKE + 16) == EWORKSPACE
    assert call(ws=FAKE2) == EINVAL                      # workspace overlaps h
    assert call(d=100) == EUNSUPPORTED
    assert call(L=-1) == EINVAL
    assert call(eps=-1.0) == EINVAL


def test_stage_entry_points_validate(lib):
    arr = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    assert lib.moe_router_topk(FAKE, FAKE, 4, 64, 8, 0, 1, FAKE, FAKE, None, None) == EINVAL
    assert lib.moe_router_topk(FAKE, FAKE, 4, 64, 8, 2, 3, FAKE, FAKE, None, None) == EINVAL
    assert lib.moe_router_topk(None, FAKE, 4, 64, 8, 2, 1, FAKE, FAKE, None, None) == EINVAL
    assert lib.moe_route_permute(FAKE, 4, 65, 2, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.moe_route_permute(FAKE, 4, 8, 2, None, FAKE, FAKE, None) == EINVAL
    assert lib.moe_expert_swiglu(FAKE, arr, arr, 4, 100, 256, 8, 2, 1, FAKE, FAKE, FAKE,
                                 None, 0, None) == EUNSUPPORTED
    assert lib.moe_expert_swiglu(FAKE, arr, arr, 4, 128, 256, 8, 2, 1, None, FAKE, FAKE,
                                 None, 0, None) == EINVAL
    # the streaming plan of an 8-token Mixtral-shape layer needs scratch
    assert lib.moe_expert_swiglu(FAKE, arr, arr, 8, 4096, 14336, 8, 2, 1, FAKE, FAKE, FAKE,
                                 None, 0, None) == EWORKSPACE
    assert lib.moe_expert_down(FAKE, arr, 4, 128, 256, 8, 2, 1, FAKE, None, None, 0,
                               None) == EINVAL
    # a 4096-token Mixtral-shape W2 product keeps the pieces of its last round
    # of tiles in scratch: refused before any launch without it, or too small
    assert lib.moe_expert_down(FAKE, arr, 4096, 4096, 14336, 8, 2, 1, FAKE, FAKE, None, 0,
                               None) == EWORKSPACE
    assert lib.moe_expert_down(FAKE, arr, 4096, 4096, 14336, 8, 2, 1, FAKE, FAKE, FAKE, 1 << 20,
                               None) == EWORKSPACE
    assert lib.moe_combine(FAKE, 1, FAKE, FAKE, 4, 128, 0, FAKE2, 0, 0, None) == EINVAL
    assert lib.moe_combine(FAKE, 1, FAKE, FAKE, 4, 128, 2, None, 0, 0, None) == EINVAL
    assert lib.moe_combine(FAKE, 0, FAKE, FAKE, 4, 128, 2, FAKE2, 0, 0, None) == EINVAL
    assert lib.moe_rmsnorm(FAKE, FAKE, 4, 128, 1e-5, 1, None) == EINVAL     # overlap
    assert lib.moe_rmsnorm(FAKE, FAKE2, 4, 128, -1.0, 1, None) == EINVAL
    for fn_args in [(FAKE, FAKE, 0, 64, 8, 2, 1, FAKE, FAKE, None, None)]:
        assert lib.moe_router_topk(*fn_args) == OK      # T = 0: nothing launched


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(M.MoeLibraryMissing):
        M.load_library(str(tmp_path / "missing.so"))


def _swa(lib, B=1, T=4, W=16, H=8, KVH=2, hd=128, q=FAKE, kn=FAKE + 0x100000, vn=FAKE + 0x200000,
         kc=FAKE + 0x300000, vc=FAKE + 0x400000, pos=FAKE + 0x500000, out=FAKE2, odt=1,
         ws=None, ws_bytes=0):
    return lib.swa_attention(q, kn, vn, kc, vc, pos, B, T, W, H, KVH, hd, out, odt, ws, ws_bytes,
                             None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), EINVAL),
    (dict(pos=None), EINVAL),
    (dict(out=None), EINVAL),
    (dict(B=-1), EINVAL),
    (dict(W=0), EINVAL),
    (dict(H=6, KVH=4), EINVAL),                 # not a multiple
    (dict(H=16, KVH=2), EUNSUPPORTED),          # group of 8
    (dict(hd=64), EUNSUPPORTED),
    (dict(T=17, W=16), EUNSUPPORTED),           # chunk longer than the window
    (dict(odt=7), EINVAL),
    (dict(q=FAKE + 8), EUNSUPPORTED),           # misaligned
    (dict(out=FAKE), EINVAL),                   # out overlaps q
    (dict(B=8, T=1, W=4096, H=32, KVH=8), EWORKSPACE),   # key splits need a workspace
])
def test_swa_attention_rejects_before_launch(lib, kwargs, status):
    got = _swa(lib, **kwargs)
    assert got == status, lib.moe_last_error()
    assert lib.moe_last_error() != b""


def test_swa_noops_and_workspace_size(lib):
    assert _swa(lib, T=0) == OK and _swa(lib, B=0) == OK
    assert M.swa_workspace_size(1, 4096, 4096, 32, 8) == 0        # prefill: no key splits
    n = M.swa_workspace_size(8, 1, 4096, 32, 8)                   # decode: split keys
    assert n >= 8 * 32 * 2 * (128 + 2) * 4
    assert lib.swa_cache_append(FAKE, FAKE, FAKE, 1, 0, 16, 2, 128, FAKE2, FAKE2, None) == OK
    assert lib.swa_cache_append(FAKE, FAKE, FAKE, 1, 4, 16, 2, 64, FAKE2, FAKE2, None) == EUNSUPPORTED
    assert lib.swa_cache_append(None, FAKE, FAKE, 1, 4, 16, 2, 128, FAKE2, FAKE2, None) == EINVAL
