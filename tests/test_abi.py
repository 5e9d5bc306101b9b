"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe_ep.h declares, and rejects bad arguments on the host before
enqueueing anything (all calls below return before any HIP runtime call)."""
import ctypes
import os
import re
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "moe_ep.h"
LIB = ROOT / "combine_top_expert_amd" / "libmoe_ep.so"

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*|int)\s+(moe_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not LIB.exists():
        import __graft_entry__
        __graft_entry__._build_module().build(verbose=False)
    return ctypes.CDLL(str(LIB))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ["moe_dispatch_layout", "moe_permute", "moe_grouped_gemm_w13", "moe_silu_mul",
                 "moe_grouped_gemm_w2", "moe_combine", "moe_router_topk",
                 "moe_grouped_gemm_workspace_bytes", "moe_pack_w13", "moe_combine_backward",
                 "moe_silu_mul_backward", "moe_permute_backward", "moe_transpose_weights",
                 "moe_grouped_gemm_wgrad", "moe_dispatch_layout_noalloc",
                 "moe_dispatch_layout_noalloc_max_bytes", "moe_grouped_gemm_w2_combine",
                 "moe_grouped_gemm_w13_silu_backward"]:
        assert name in fns
    assert len(fns) == 21


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(LIB)], capture_output=True, text=True)
    exported = set(re.findall(r" T (moe_\w+)$", out.stdout, flags=re.M))
    assert set(declared_functions()) <= exported
    # C linkage, and nothing but the declared entry points is exported
    assert not re.search(r" T _Z", out.stdout)
    assert exported == set(declared_functions())


def test_status_strings_and_version(lib):
    lib.moe_status_string.restype = ctypes.c_char_p
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(-2) == b"MOE_ERR_UNSUPPORTED"
    assert lib.moe_status_string(12345) == b"MOE_ERR_UNKNOWN"
    assert lib.moe_abi_version() == 9


def test_workspace_bytes(lib):
    f = lib.moe_dispatch_layout_workspace_bytes
    f.restype = ctypes.c_size_t
    # ceil(T*K / 1024) blocks, L counters each, a flag per block, 64 spare ints
    for T, K, L in [(8192, 8, 32), (16384, 6, 64), (0, 4, 8), (1, 1, 1)]:
        nblk = -(-(T * K) // 1024)
        assert f(T, K, L) == 4 * (nblk * L + nblk + 64)
    assert f(-1, 2, 3) == 0


def P(v=1):
    return ctypes.c_void_p(v)


def layout_call(lib, T=4, K=2, E=8, e0=0, L=8, R=16, BM=128, ws_bytes=1 << 20, null=None):
    f = lib.moe_dispatch_layout
    f.restype = ctypes.c_int
    ptrs = [P() for _ in range(8)]
    if null is not None:
        ptrs[null] = None
    ids, counts, offsets, slot_of, row_src, tiles, status, ws = ptrs
    return f(ids, T, K, E, e0, L, R, BM, counts, offsets, slot_of, row_src, tiles, status, ws,
             ctypes.c_size_t(ws_bytes), None)


def test_layout_argument_errors(lib):
    assert layout_call(lib, L=0) == INVALID
    assert layout_call(lib, L=2000, E=4000) == INVALID       # L beyond 1024
    assert layout_call(lib, e0=4, L=8, E=8) == INVALID       # experts beyond E
    assert layout_call(lib, R=-1) == INVALID
    assert layout_call(lib, BM=0) == INVALID
    assert layout_call(lib, ws_bytes=4) == WORKSPACE
    for i in range(8):
        assert layout_call(lib, null=i) == INVALID, i


def test_permute_argument_errors(lib):
    f = lib.moe_permute
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert f(P(), 1, 4, 2, 100, P(), 8, P(), 1, None, None) == UNSUPPORTED   # H % 128
    assert f(P(), 1, 4, 2, 256, P(), 8, P(), 0, None, None) == UNSUPPORTED   # bf16 -> fp32
    assert f(P(), 2, 4, 2, 256, P(), 8, P(), 2, P(), None) == UNSUPPORTED   # fp8 input
    assert f(P(), 1, 4, 2, 256, P(), 8, P(), 2, None, None) == INVALID      # fp8 without scales
    assert f(P(), 7, 4, 2, 256, P(), 8, P(), 1, None, None) == INVALID      # bad dtype enum
    assert f(P(), 1, 4, 65, 256, P(), 8, P(), 1, None, None) == UNSUPPORTED  # K > 64 routes
    assert f(None, 1, 0, 2, 256, None, 8, None, 1, None, None) == OK        # T = 0: nothing to do


def test_gemm_argument_errors(lib):
    w13 = lib.moe_grouped_gemm_w13
    w13.restype = ctypes.c_int
    w13.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                    ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                    ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def call(a_dt=2, w_dt=2, H=256, I=128, epi=1, out_dt=2, L=2, scales=True, ws=None, ws_bytes=0,
             layout=0, rows_cap=256):
        s = P() if scales else None
        return w13(P(), a_dt, s, P(), w_dt, s, layout, P(), P(), L, rows_cap, H, I, epi, P(), out_dt, s, ws,
                   ws_bytes, None)

    assert call(a_dt=1, w_dt=2) == UNSUPPORTED
    assert call(H=200) == UNSUPPORTED
    assert call(I=100) == UNSUPPORTED
    assert call(epi=0, out_dt=1) == UNSUPPORTED      # G is always fp32
    assert call(epi=5) == INVALID
    assert call(L=0) == INVALID
    assert call(scales=False) == INVALID
    assert call(ws=P(), ws_bytes=64) == WORKSPACE     # a workspace below the query's size
    assert call(layout=2) == INVALID                  # unknown weight layout
    # staged loads use 32-bit buffer offsets: A and one expert's W below 2 GiB
    assert call(H=16384, rows_cap=131072) == UNSUPPORTED            # A: 16 KiB x 131200 rows
    assert call(H=16384, I=65536, rows_cap=256) == UNSUPPORTED      # W13[e]: 131072 x 16 KiB
    assert call(a_dt=1, w_dt=1, H=16384, scales=False, rows_cap=65536) == UNSUPPORTED   # bf16 A
    assert call(H=16384 + 128) == UNSUPPORTED                       # FP8 K beyond 128 scale groups
    pk = lib.moe_pack_w13
    pk.restype = ctypes.c_int
    pk.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    assert pk(P(16), 2, 2, 200, 128, P(4096), None) == UNSUPPORTED   # H % 128
    assert pk(P(16), 2, 2, 256, 128, P(16), None) == INVALID         # in place
    assert pk(P(16), 2, 2, 256, 128, P(4104), None) == INVALID       # misaligned output
    assert pk(P(16), 2, 0, 256, 128, P(4096), None) == INVALID       # L = 0
    w2 = lib.moe_grouped_gemm_w2
    w2.restype = ctypes.c_int
    w2.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_void_p]
    assert w2(P(), 1, None, P(), 1, None, P(), P(), 2, 256, 256, 128, P(), 2, None, 0, None) == UNSUPPORTED
    assert w2(P(), 0, None, P(), 1, None, P(), P(), 2, 256, 256, 128, P(), 1, None, 0, None) == UNSUPPORTED
    assert w2(P(), 1, None, P(), 1, None, P(), P(), 2, 256, 256, 128, P(), 1, P(), 64, None) == WORKSPACE
    q = lib.moe_grouped_gemm_workspace_bytes
    q.restype, q.argtypes = ctypes.c_size_t, []
    assert q() >= 128 * 256 * 4 * 8                   # a partial tile per workgroup of a grid


def test_combine_and_silu_argument_errors(lib):
    c = lib.moe_combine
    c.restype = ctypes.c_int
    c.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_void_p]
    assert c(P(), 1, P(), P(), 4, 2, 100, 8, P(), 1, None) == UNSUPPORTED    # H % 8
    assert c(P(), 2, P(), P(), 4, 2, 256, 8, P(), 1, None) == UNSUPPORTED    # fp8 outputs
    assert c(P(), 1, P(), P(), 4, 65, 256, 8, P(), 1, None) == UNSUPPORTED   # K > 64 routes
    assert c(P(), 1, None, P(), 4, 2, 256, 8, P(), 1, None) == INVALID
    s = lib.moe_silu_mul
    s.restype = ctypes.c_int
    s.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert s(P(), P(), P(), 2, 256, 100, P(), 1, None, None) == UNSUPPORTED
    assert s(P(), P(), P(), 2, 256, 128, P(), 2, None, None) == INVALID


def test_python_binding_loads_and_matches_header(lib):
    import combine_top_expert_amd as ep
    for name in declared_functions():
        assert callable(getattr(ep, name)), name
    assert ep.moe_abi_version() == 9
    assert ep.moe_status_string(-1) == "MOE_ERR_INVALID_ARG"


def test_binding_fails_loudly_without_library(tmp_path):
    env = dict(os.environ, MOE_EP_LIB=str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", "import combine_top_expert_amd"], cwd=ROOT, env=env,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr


def test_product_never_touches_the_oracle():
    pkg = ROOT / "combine_top_expert_amd"
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.cpp")) + \
            list(pkg.rglob("*.h")):
        text = f.read_text()
        assert not re.search(r"^\s*(from|import)\s+(oracle|workloads)\b", text, flags=re.M), f
        assert "oracle/" not in text, f


def test_router_argument_errors(lib):
    r = lib.moe_router_topk
    r.restype = ctypes.c_int
    r.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert r(P(), None, 4, 8, 9, 1, P(), P(), None) == INVALID          # K > E
    assert r(P(), None, 4, 8, 0, 1, P(), P(), None) == INVALID          # K = 0
    assert r(P(), None, 4, 2048, 8, 1, P(), P(), None) == UNSUPPORTED   # E > 1024
    assert r(P(), None, 4, 256, 65, 1, P(), P(), None) == UNSUPPORTED   # K > 64
    assert r(None, None, 4, 256, 8, 1, P(), P(), None) == INVALID       # no logits
    assert r(None, None, 0, 256, 8, 1, None, None, None) == OK          # T = 0


def test_backward_argument_errors(lib):
    cb = lib.moe_combine_backward
    cb.restype = ctypes.c_int
    cb.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert cb(P(), 1, P(), 1, P(), P(), 4, 2, 100, 8, P(), 1, P(), None) == UNSUPPORTED  # H % 8
    assert cb(P(), 2, P(), 1, P(), P(), 4, 2, 256, 8, P(), 1, P(), None) == UNSUPPORTED  # fp8 dy
    assert cb(P(), 1, P(), 1, P(), None, 4, 2, 256, 8, P(), 1, P(), None) == INVALID     # no weights
    assert cb(None, 1, None, 1, None, None, 0, 2, 256, 8, None, 1, None, None) == OK     # T = 0
    sb = lib.moe_silu_mul_backward
    sb.restype = ctypes.c_int
    sb.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert sb(P(), P(), 1, P(), P(), 2, 256, 126, P(), 1, None) == UNSUPPORTED            # I % 4
    assert sb(P(), P(), 2, P(), P(), 2, 256, 128, P(), 1, None) == UNSUPPORTED            # fp8 dz
    assert sb(None, P(), 1, P(), P(), 2, 256, 128, P(), 1, None) == INVALID
    pb = lib.moe_permute_backward
    pb.restype = ctypes.c_int
    pb.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert pb(P(), 1, P(), 4, 65, 256, 8, P(), 1, None) == UNSUPPORTED                   # K > 64
    assert pb(P(), 1, None, 4, 2, 256, 8, P(), 1, None) == INVALID
    tw = lib.moe_transpose_weights
    tw.restype = ctypes.c_int
    tw.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    assert tw(P(), 2, 2, 128, 128, P(8), None) == UNSUPPORTED                            # fp8
    assert tw(P(), 1, 2, 128, 128, P(), None) == INVALID                                 # in place
    assert tw(P(), 1, 0, 128, 128, P(8), None) == INVALID
    wg = lib.moe_grouped_gemm_wgrad
    wg.restype = ctypes.c_int
    wg.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_void_p]
    A = P(256)
    assert wg(A, A, 2, A, A, 4, 64, 128, 128, A, None) == UNSUPPORTED                   # fp8
    assert wg(A, A, 1, A, A, 4, 64, 192, 128, A, None) == UNSUPPORTED                   # N % 128
    assert wg(A, A, 1, A, A, 4, 64, 128, 96, A, None) == UNSUPPORTED                    # K % 128
    assert wg(A, A, 1, A, A, 0, 64, 128, 128, A, None) == INVALID                       # L = 0
    assert wg(A, A, 1, A, A, 4, 64, 128, 128, None, None) == INVALID                    # no c
    assert wg(P(258), A, 1, A, A, 4, 64, 128, 128, A, None) == INVALID                  # misaligned b
    assert wg(A, None, 1, A, A, 4, 64, 128, 128, A, None) == INVALID                    # no a
    assert wg(A, A, 1, A, A, 4, 64, 128, 128, P(260), None) == INVALID                  # misaligned c
    fb = lib.moe_grouped_gemm_w13_silu_backward
    fb.restype = ctypes.c_int
    fb.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def fcall(a_dt=1, w_dt=1, dz_dt=1, dg_dt=1, H=256, I=128, L=2, layout=0, dz=True, ws=None, ws_bytes=0):
        return fb(P(), a_dt, P(), w_dt, layout, P(), P(), L, 256, H, I, P() if dz else None, dz_dt, P(), dg_dt,
                  ws, ws_bytes, None)

    assert fcall(a_dt=2, w_dt=2) == UNSUPPORTED                                           # no FP8 backward
    assert fcall(a_dt=0) == UNSUPPORTED                                                   # a_dt != w_dt
    assert fcall(dz_dt=2) == UNSUPPORTED
    assert fcall(dg_dt=2) == UNSUPPORTED
    assert fcall(H=200) == UNSUPPORTED
    assert fcall(I=100) == UNSUPPORTED
    assert fcall(L=0) == INVALID
    assert fcall(layout=2) == INVALID
    assert fcall(dz=False) == INVALID
    assert fcall(ws=P(), ws_bytes=64) == WORKSPACE


def test_layout_noalloc_argument_errors(lib):
    """The allocation-free layout reports argument errors like the workspace
    entry point and rejects sizes beyond its scratch before any device call."""
    f = lib.moe_dispatch_layout_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 7 + [ctypes.c_void_p] * 7
    mx = lib.moe_dispatch_layout_noalloc_max_bytes
    mx.restype = ctypes.c_size_t
    ws = lib.moe_dispatch_layout_workspace_bytes
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int] * 3
    assert mx() == 4 << 20
    p = [P()] * 6

    def call(T=64, K=8, E=256, e0=0, L=32, R=128, BM=128):
        return f(P(), T, K, E, e0, L, R, BM, *p, None)

    assert call(L=0) == INVALID
    assert call(K=0) == INVALID
    assert call(e0=250) == INVALID                   # owned range past E_global
    assert call(T=1 << 28, K=8) == UNSUPPORTED       # more than 2^30 routes
    # T*K routes need ceil(T*K/1024) * (L + 1) + 64 ints of histogram table
    assert ws(1 << 20, 8, 1024) > mx()
    assert call(T=1 << 20, K=8, E=1024, L=1024) == WORKSPACE
    assert ws(1 << 21, 8, 32) <= mx()                # 16M routes at L = 32 fit


def test_w2_combine_argument_errors(lib):
    """The down GEMM with the combine in its epilogue checks every argument,
    pointers included, before its first launch (the y_acc clear)."""
    f = lib.moe_grouped_gemm_w2_combine
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]

    def call(z_dt=2, w_dt=2, scales=True, L=2, rows_cap=256, H=256, I=128, row_src=True, T=4, K=2,
             y_acc=16, y=16, y_dt=1):
        s = P() if scales else None
        return f(P(), z_dt, s, P(), w_dt, s, P(), P(), L, rows_cap, H, I, P() if row_src else None,
                 P(), T, K, P(y_acc) if y_acc else None, P(y) if y else None, y_dt, None)

    assert call(z_dt=1) == UNSUPPORTED               # Z and W2 in different formats
    assert call(H=200) == UNSUPPORTED                 # H % 128
    assert call(I=100) == UNSUPPORTED                 # I % 128
    assert call(y_dt=2) == UNSUPPORTED                # y in FP8
    assert call(L=0) == INVALID
    assert call(K=0) == INVALID
    assert call(y_acc=0) == INVALID
    assert call(y=24) == INVALID                      # y not 16-byte aligned
    assert call(row_src=False) == INVALID             # rows without their (t, k)
    assert call(scales=False) == INVALID              # FP8 without block scales
