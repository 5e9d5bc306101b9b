"""Python binding of libmoe_ep.so -- the MI355X (gfx950) MoE hot path.

Argument marshalling only: every function below checks tensor placement,
dtype, contiguity and shapes, derives sizes from shapes, and calls the C
entry point of the same name in ``include/moe_ep.h`` on torch's current HIP
stream.  With ``bind=True`` it returns that call, marshalled once, as a
zero-argument callable instead (a step loop then pays no Python-side checks).
All computation happens in the library's HIP kernels; there is no CPU or
PyTorch fallback.  Importing this package fails loudly if the library has
not been built (``python combine_top_expert_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

__all__ = [
    "MoEError", "LIB_PATH", "lib", "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3",
    "MOE_EPI_STORE_G", "MOE_EPI_SILU_MUL", "MOE_FLAG_CAPACITY", "MOE_FLAG_BAD_EXPERT_ID",
    "moe_status_string", "moe_abi_version", "moe_dispatch_layout_workspace_bytes",
    "moe_grouped_gemm_workspace_bytes", "moe_pack_w13", "MOE_W_ROW_MAJOR", "MOE_W_PACKED",
    "moe_combine_backward", "moe_silu_mul_backward", "moe_permute_backward", "moe_transpose_weights",
    "moe_grouped_gemm_wgrad", "moe_grouped_gemm_w13_silu_backward", "moe_dispatch_layout",
    "moe_dispatch_layout_noalloc",
    "moe_dispatch_layout_noalloc_max_bytes", "moe_permute", "moe_grouped_gemm_w13", "moe_silu_mul",
    "moe_grouped_gemm_w2", "moe_grouped_gemm_w2_combine", "moe_combine", "moe_router_topk",
    "dtype_code",
]

LIB_PATH = Path(os.environ.get("MOE_EP_LIB", Path(__file__).resolve().parent / "libmoe_ep.so"))

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_EPI_STORE_G, MOE_EPI_SILU_MUL = 0, 1
MOE_W_ROW_MAJOR, MOE_W_PACKED = 0, 1
MOE_FLAG_CAPACITY, MOE_FLAG_BAD_EXPERT_ID = 1, 2

if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is not built; run `python combine_top_expert_amd/build.py` "
                      "(the MoE path has no fallback without its HIP library)")
lib = ctypes.CDLL(str(LIB_PATH))

_p, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_SIG = {
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_abi_version": (_i, []),
    "moe_dispatch_layout_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_dispatch_layout": (_i, [_p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_dispatch_layout_noalloc": (_i, [_p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]),
    "moe_dispatch_layout_noalloc_max_bytes": (_sz, []),
    "moe_permute": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _i, _p, _p]),
    "moe_grouped_gemm_w13": (_i, [_p, _i, _p, _p, _i, _p, _i, _p, _p, _i, _i64, _i, _i, _i, _p, _i,
                                  _p, _p, _sz, _p]),
    "moe_pack_w13": (_i, [_p, _i, _i, _i, _i, _p, _p]),
    "moe_grouped_gemm_workspace_bytes": (_sz, []),
    "moe_silu_mul": (_i, [_p, _p, _p, _i, _i64, _i, _p, _i, _p, _p]),
    "moe_grouped_gemm_w2": (_i, [_p, _i, _p, _p, _i, _p, _p, _p, _i, _i64, _i, _i, _p, _i, _p, _sz,
                                 _p]),
    "moe_combine": (_i, [_p, _i, _p, _p, _i, _i, _i, _i64, _p, _i, _p]),
    "moe_grouped_gemm_w2_combine": (_i, [_p, _i, _p, _p, _i, _p, _p, _p, _i, _i64, _i, _i, _p, _p, _i, _i,
                                         _p, _p, _i, _p]),
    "moe_router_topk": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _p]),
    "moe_combine_backward": (_i, [_p, _i, _p, _i, _p, _p, _i, _i, _i, _i64, _p, _i, _p, _p]),
    "moe_silu_mul_backward": (_i, [_p, _p, _i, _p, _p, _i, _i64, _i, _p, _i, _p]),
    "moe_permute_backward": (_i, [_p, _i, _p, _i, _i, _i, _i64, _p, _i, _p]),
    "moe_transpose_weights": (_i, [_p, _i, _i, _i, _i, _p, _p]),
    "moe_grouped_gemm_wgrad": (_i, [_p, _p, _i, _p, _p, _i, _i64, _i, _i, _p, _p]),
    "moe_grouped_gemm_w13_silu_backward": (_i, [_p, _i, _p, _i, _i, _p, _p, _i, _i64, _i, _i, _p, _i, _p, _i,
                                                _p, _sz, _p]),
}
for _name, (_res, _args) in _SIG.items():
    if not hasattr(lib, _name):
        raise ImportError(f"{LIB_PATH} lacks {_name}: it predates these sources; rebuild with "
                          "`python combine_top_expert_amd/build.py`")
    _f = getattr(lib, _name)
    _f.restype, _f.argtypes = _res, _args


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {moe_status_string(status)} ({status})")
        self.status = status


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def moe_abi_version() -> int:
    return int(lib.moe_abi_version())


def moe_dispatch_layout_workspace_bytes(T: int, K: int, L: int) -> int:
    return int(lib.moe_dispatch_layout_workspace_bytes(T, K, L))


def moe_grouped_gemm_workspace_bytes() -> int:
    return int(lib.moe_grouped_gemm_workspace_bytes())


# ---------------------------------------------------------------- marshalling helpers

def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MOE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: torch.Tensor | None, name: str) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _i32(t: torch.Tensor | None, name: str) -> int | None:
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _ptr(t, name)


def _f32(t: torch.Tensor | None, name: str) -> int | None:
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t, name)


def _shape(t: torch.Tensor | None, name: str, *dims: int) -> None:
    """Raise ValueError unless t has exactly the shape dims (None passes).
    The C ABI receives sizes, not buffer extents, so a mis-sized tensor would
    otherwise become an out-of-bounds device access."""
    if t is not None and tuple(t.shape) != tuple(int(d) for d in dims):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(d) for d in dims)}")


def _offsets(t: torch.Tensor, L: int) -> None:
    """Expert offsets as the kernels read them: one dimension, entries
    [0, L) (moe_dispatch_layout writes L + 1; the last is not read here)."""
    if t.dim() != 1 or t.shape[0] < L:
        raise ValueError(f"offsets has shape {tuple(t.shape)}, expected ({L},) or longer")


def _need(t: torch.Tensor | None, name: str, when: bool) -> None:
    if when and t is None:
        raise ValueError(f"{name} is required here")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoEError(fn, status)


def _run(fn: str, bind: bool, args: tuple):
    """Call C entry point ``fn`` with the marshalled ``args``; with ``bind``,
    return a zero-argument callable that makes the same call later instead
    (all checks and pointer lookups done once: the tensors must stay alive
    and keep their shapes; the stream is the one current now)."""
    f = getattr(lib, fn)
    if bind:
        def call():
            st = f(*args)
            if st != 0:
                raise MoEError(fn, st)
        return call
    _check(fn, f(*args))
    return None


# ---------------------------------------------------------------- entry points

def moe_dispatch_layout(topk_ids, E_global, expert_begin, L, R, BM, counts, offsets, slot_of,
                        row_src, tile_offsets, dev_status, workspace, bind=False):
    """topk_ids [T,K] int32 -> counts [L], offsets [L+1], slot_of [T,K],
    row_src [rows_cap], tile_offsets [L+1], dev_status [2] (all int32)."""
    T, K = topk_ids.shape
    rows_cap = L * R if R > 0 else T * K
    _shape(counts, "counts", L)
    _shape(offsets, "offsets", L + 1)
    _shape(slot_of, "slot_of", T, K)
    _shape(row_src, "row_src", rows_cap)
    _shape(tile_offsets, "tile_offsets", L + 1)
    _shape(dev_status, "dev_status", 2)
    return _run("moe_dispatch_layout", bind, (
        _i32(topk_ids, "topk_ids"), T, K, E_global, expert_begin, L, R, BM,
        _i32(counts, "counts"), _i32(offsets, "offsets"), _i32(slot_of, "slot_of"),
        _i32(row_src, "row_src"), _i32(tile_offsets, "tile_offsets"),
        _i32(dev_status, "dev_status"), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(topk_ids)))


def moe_dispatch_layout_noalloc_max_bytes() -> int:
    return int(lib.moe_dispatch_layout_noalloc_max_bytes())


def moe_dispatch_layout_noalloc(topk_ids, E_global, expert_begin, L, R, BM, counts, offsets, slot_of,
                                row_src, tile_offsets, dev_status, bind=False):
    """moe_dispatch_layout with the library's per-device scratch in place of
    a workspace (the C call allocates nothing; see moe_ep.h for the size
    limit and the sharing rule)."""
    T, K = topk_ids.shape
    rows_cap = L * R if R > 0 else T * K
    _shape(counts, "counts", L)
    _shape(offsets, "offsets", L + 1)
    _shape(slot_of, "slot_of", T, K)
    _shape(row_src, "row_src", rows_cap)
    _shape(tile_offsets, "tile_offsets", L + 1)
    _shape(dev_status, "dev_status", 2)
    return _run("moe_dispatch_layout_noalloc", bind, (
        _i32(topk_ids, "topk_ids"), T, K, E_global, expert_begin, L, R, BM,
        _i32(counts, "counts"), _i32(offsets, "offsets"), _i32(slot_of, "slot_of"),
        _i32(row_src, "row_src"), _i32(tile_offsets, "tile_offsets"),
        _i32(dev_status, "dev_status"), _stream(topk_ids)))


def moe_permute(x, slot_of, buf, buf_scales=None, bind=False):
    """x [T,H] (fp32|bf16), slot_of [T,K] -> buf [rows_cap,H] (+ scales for FP8)."""
    T, H = x.shape
    K = slot_of.shape[1]
    _shape(slot_of, "slot_of", T, K)
    _shape(buf, "buf", buf.shape[0], H)
    fp8 = dtype_code(buf) == MOE_FP8_E4M3
    _need(buf_scales, "buf_scales", fp8)
    if fp8:
        _shape(buf_scales, "buf_scales", buf.shape[0], H // 128)
    return _run("moe_permute", bind, (
        _ptr(x, "x"), dtype_code(x), T, K, H, _i32(slot_of, "slot_of"), buf.shape[0],
        _ptr(buf, "buf"), dtype_code(buf), _f32(buf_scales, "buf_scales"), _stream(x)))


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()


def moe_pack_w13(w13, w13_packed, bind=False):
    """w13 [L,2I,H] -> w13_packed (same shape and dtype, bytes in the GEMM's
    staging order; see moe_ep.h)."""
    L, N, H = w13.shape
    if w13_packed.shape != w13.shape or w13_packed.dtype != w13.dtype:
        raise ValueError("w13_packed must match w13 in shape and dtype")
    return _run("moe_pack_w13", bind, (
        _ptr(w13, "w13"), dtype_code(w13), L, H, N // 2, _ptr(w13_packed, "w13_packed"), _stream(w13)))


def moe_grouped_gemm_w13(a, a_scales, w13, w13_scales, counts, offsets, epi, out,
                         out_scales=None, workspace=None, w13_layout=MOE_W_ROW_MAJOR, bind=False):
    """a [rows_cap,H], w13 [L,2I,H] -> G [rows_cap,2I] fp32 or Z [rows_cap,I].
    workspace: None, or a device buffer of moe_grouped_gemm_workspace_bytes().
    w13_layout: MOE_W_PACKED when w13 was written by moe_pack_w13."""
    L, N, H = w13.shape
    rows_cap, I = a.shape[0], N // 2
    _shape(a, "a", rows_cap, H)
    fp8 = dtype_code(a) == MOE_FP8_E4M3
    _need(a_scales, "a_scales", fp8)
    _need(w13_scales, "w13_scales", fp8)
    if fp8:
        _shape(a_scales, "a_scales", rows_cap, H // 128)
        _shape(w13_scales, "w13_scales", L, N // 128, H // 128)
    _shape(counts, "counts", L)
    _offsets(offsets, L)
    if int(epi) == MOE_EPI_STORE_G:
        _shape(out, "out (G)", rows_cap, N)
    else:
        _shape(out, "out (Z)", rows_cap, I)
        _need(out_scales, "out_scales", dtype_code(out) == MOE_FP8_E4M3)
        if dtype_code(out) == MOE_FP8_E4M3:
            _shape(out_scales, "out_scales", rows_cap, I // 128)
    wp, wb = _ws(workspace)
    return _run("moe_grouped_gemm_w13", bind, (
        _ptr(a, "a"), dtype_code(a), _f32(a_scales, "a_scales"), _ptr(w13, "w13"),
        dtype_code(w13), _f32(w13_scales, "w13_scales"), int(w13_layout), _i32(counts, "counts"),
        _i32(offsets, "offsets"), L, a.shape[0], H, N // 2, int(epi), _ptr(out, "out"),
        dtype_code(out), _f32(out_scales, "out_scales"), wp, wb, _stream(a)))


def moe_grouped_gemm_w13_silu_backward(a, w13, counts, offsets, dz, dg, workspace=None,
                                       w13_layout=MOE_W_ROW_MAJOR, bind=False):
    """a [rows_cap,H], w13 [L,2I,H] (bf16|fp32), dz [rows_cap,I] -> dg
    [rows_cap,2I]: G recomputed with the SiLU*up gradient in the GEMM's
    epilogue (same values as MOE_EPI_STORE_G followed by moe_silu_mul_backward)."""
    L, N, H = w13.shape
    rows_cap, I = a.shape[0], N // 2
    _shape(a, "a", rows_cap, H)
    _shape(counts, "counts", L)
    _offsets(offsets, L)
    _shape(dz, "dz", rows_cap, I)
    _shape(dg, "dg", rows_cap, N)
    wp, wb = _ws(workspace)
    return _run("moe_grouped_gemm_w13_silu_backward", bind, (
        _ptr(a, "a"), dtype_code(a), _ptr(w13, "w13"), dtype_code(w13), int(w13_layout),
        _i32(counts, "counts"), _i32(offsets, "offsets"), L, rows_cap, H, I, _ptr(dz, "dz"), dtype_code(dz),
        _ptr(dg, "dg"), dtype_code(dg), wp, wb, _stream(a)))


def moe_silu_mul(g, counts, offsets, z, z_scales=None, bind=False):
    """g [rows_cap,2I] fp32 -> z [rows_cap,I] (fp32|bf16|FP8 + scales)."""
    rows_cap, N = g.shape
    L = counts.shape[0]
    _offsets(offsets, L)
    _shape(z, "z", rows_cap, N // 2)
    _need(z_scales, "z_scales", dtype_code(z) == MOE_FP8_E4M3)
    if dtype_code(z) == MOE_FP8_E4M3:
        _shape(z_scales, "z_scales", rows_cap, N // 2 // 128)
    return _run("moe_silu_mul", bind, (
        _f32(g, "g"), _i32(counts, "counts"), _i32(offsets, "offsets"), counts.shape[0],
        rows_cap, N // 2, _ptr(z, "z"), dtype_code(z), _f32(z_scales, "z_scales"), _stream(g)))


def moe_grouped_gemm_w2(z, z_scales, w2, w2_scales, counts, offsets, out, workspace=None, bind=False):
    """z [rows_cap,I], w2 [L,H,I] -> out [rows_cap,H] (fp32|bf16).
    workspace: None, or a device buffer of moe_grouped_gemm_workspace_bytes()."""
    L, H, I = w2.shape
    rows_cap = z.shape[0]
    _shape(z, "z", rows_cap, I)
    fp8 = dtype_code(z) == MOE_FP8_E4M3
    _need(z_scales, "z_scales", fp8)
    _need(w2_scales, "w2_scales", fp8)
    if fp8:
        _shape(z_scales, "z_scales", rows_cap, I // 128)
        _shape(w2_scales, "w2_scales", L, H // 128, I // 128)
    _shape(counts, "counts", L)
    _offsets(offsets, L)
    _shape(out, "out", rows_cap, H)
    wp, wb = _ws(workspace)
    return _run("moe_grouped_gemm_w2", bind, (
        _ptr(z, "z"), dtype_code(z), _f32(z_scales, "z_scales"), _ptr(w2, "w2"), dtype_code(w2),
        _f32(w2_scales, "w2_scales"), _i32(counts, "counts"), _i32(offsets, "offsets"), L,
        z.shape[0], H, I, _ptr(out, "out"), dtype_code(out), wp, wb, _stream(z)))


def moe_grouped_gemm_w2_combine(z, z_scales, w2, w2_scales, counts, offsets, row_src, topk_weights,
                                y_acc, y, bind=False):
    """Down GEMM with the combine in its epilogue: z [rows_cap,I], w2 [L,H,I],
    row_src [rows_cap], topk_weights [T,K] -> y [T,H] (y_acc [T,H] fp32
    scratch).  Not bit-reproducible (fp32 atomic adds); see moe_ep.h."""
    L, H, I = w2.shape
    rows_cap = z.shape[0]
    T, K = topk_weights.shape
    _shape(z, "z", rows_cap, I)
    fp8 = dtype_code(z) == MOE_FP8_E4M3
    _need(z_scales, "z_scales", fp8)
    _need(w2_scales, "w2_scales", fp8)
    if fp8:
        _shape(z_scales, "z_scales", rows_cap, I // 128)
        _shape(w2_scales, "w2_scales", L, H // 128, I // 128)
    _shape(counts, "counts", L)
    _offsets(offsets, L)
    _shape(row_src, "row_src", rows_cap)
    _shape(y_acc, "y_acc", T, H)
    _shape(y, "y", T, H)
    return _run("moe_grouped_gemm_w2_combine", bind, (
        _ptr(z, "z"), dtype_code(z), _f32(z_scales, "z_scales"), _ptr(w2, "w2"), dtype_code(w2),
        _f32(w2_scales, "w2_scales"), _i32(counts, "counts"), _i32(offsets, "offsets"), L, rows_cap, H, I,
        _i32(row_src, "row_src"), _f32(topk_weights, "topk_weights"), T, K, _f32(y_acc, "y_acc"),
        _ptr(y, "y"), dtype_code(y), _stream(y)))


def moe_combine(expert_out, slot_of, topk_weights, y, bind=False):
    """expert_out [rows_cap,H], slot_of [T,K], topk_weights [T,K] -> y [T,H]."""
    T, K = slot_of.shape
    H = y.shape[1]
    _shape(y, "y", T, H)
    _shape(expert_out, "expert_out", expert_out.shape[0], H)
    _shape(topk_weights, "topk_weights", T, K)
    return _run("moe_combine", bind, (
        _ptr(expert_out, "expert_out"), dtype_code(expert_out), _i32(slot_of, "slot_of"),
        _f32(topk_weights, "topk_weights"), T, K, H, expert_out.shape[0], _ptr(y, "y"),
        dtype_code(y), _stream(y)))


def moe_router_topk(logits, K, topk_ids, topk_weights, bias=None, bias_in_weights=True, bind=False):
    """logits [T,E] fp32 (+ bias [E] fp32) -> topk_ids [T,K] int32, topk_weights [T,K] fp32."""
    T, E = logits.shape
    _shape(bias, "bias", E)
    _shape(topk_ids, "topk_ids", T, K)
    _shape(topk_weights, "topk_weights", T, K)
    return _run("moe_router_topk", bind, (
        _f32(logits, "logits"), _f32(bias, "bias"), T, E, K, 1 if bias_in_weights else 0,
        _i32(topk_ids, "topk_ids"), _f32(topk_weights, "topk_weights"), _stream(logits)))


# ---------------------------------------------------------------- backward

def moe_combine_backward(dy, expert_out, slot_of, topk_weights, d_out, d_weights, bind=False):
    """dy [T,H], expert_out [rows_cap,H] -> d_out [rows_cap,H] (local rows),
    d_weights [T,K] fp32."""
    T, K = slot_of.shape
    H = dy.shape[1]
    rows_cap = expert_out.shape[0]
    _shape(dy, "dy", T, H)
    _shape(expert_out, "expert_out", rows_cap, H)
    _shape(topk_weights, "topk_weights", T, K)
    _shape(d_out, "d_out", rows_cap, H)
    _shape(d_weights, "d_weights", T, K)
    return _run("moe_combine_backward", bind, (
        _ptr(dy, "dy"), dtype_code(dy), _ptr(expert_out, "expert_out"), dtype_code(expert_out),
        _i32(slot_of, "slot_of"), _f32(topk_weights, "topk_weights"), T, K, dy.shape[1],
        expert_out.shape[0], _ptr(d_out, "d_out"), dtype_code(d_out), _f32(d_weights, "d_weights"),
        _stream(dy)))


def moe_silu_mul_backward(g, dz, counts, offsets, dg, bind=False):
    """g [rows_cap,2I] fp32 (forward G), dz [rows_cap,I] -> dg [rows_cap,2I]."""
    rows_cap, N = g.shape
    _shape(dz, "dz", rows_cap, N // 2)
    _offsets(offsets, counts.shape[0])
    _shape(dg, "dg", rows_cap, N)
    return _run("moe_silu_mul_backward", bind, (
        _f32(g, "g"), _ptr(dz, "dz"), dtype_code(dz), _i32(counts, "counts"), _i32(offsets, "offsets"),
        counts.shape[0], rows_cap, N // 2, _ptr(dg, "dg"), dtype_code(dg), _stream(g)))


def moe_permute_backward(d_buf, slot_of, dx, bind=False):
    """d_buf [rows_cap,H] -> dx [T,H] = sum over each token's local rows."""
    T, K = slot_of.shape
    H = dx.shape[1]
    _shape(dx, "dx", T, H)
    _shape(d_buf, "d_buf", d_buf.shape[0], H)
    return _run("moe_permute_backward", bind, (
        _ptr(d_buf, "d_buf"), dtype_code(d_buf), _i32(slot_of, "slot_of"), T, K, dx.shape[1],
        d_buf.shape[0], _ptr(dx, "dx"), dtype_code(dx), _stream(dx)))


def moe_transpose_weights(w, wt, bind=False):
    """w [L,N,K] -> wt [L,K,N]."""
    L, N, K = w.shape
    if tuple(wt.shape) != (L, K, N) or wt.dtype != w.dtype:
        raise ValueError("wt must be [L,K,N] of w's dtype")
    return _run("moe_transpose_weights", bind, (
        _ptr(w, "w"), dtype_code(w), L, N, K, _ptr(wt, "wt"), _stream(w)))


def moe_grouped_gemm_wgrad(b, a, counts, offsets, c, bind=False):
    """b [rows_cap,N], a [rows_cap,K] (same dtype) -> c [L,N,K] fp32 with
    c[e] = sum over expert e's valid rows of b^T a."""
    rows_cap, N = b.shape
    K = a.shape[1]
    L = counts.shape[0]
    if a.shape[0] != rows_cap or a.dtype != b.dtype or tuple(c.shape) != (L, N, K):
        raise ValueError("wgrad needs b [R,N], a [R,K] of one dtype and c [L,N,K]")
    _offsets(offsets, L)
    return _run("moe_grouped_gemm_wgrad", bind, (
        _ptr(b, "b"), _ptr(a, "a"), dtype_code(b), _i32(counts, "counts"), _i32(offsets, "offsets"),
        L, rows_cap, N, K, _f32(c, "c"), _stream(b)))
