"""The Python binding rejects operands whose shapes disagree with the sizes it
passes to the library, before any device work (CPU only: the checks run
before the device-placement check, so host tensors reach them).

The C ABI receives sizes, not buffer extents; a mis-sized output or index
tensor would otherwise turn into an out-of-bounds device access."""
import pytest
import torch

ep = pytest.importorskip("combine_top_expert_amd")

T, K, L, R, H, I = 16, 2, 4, 10, 256, 128
RC = L * R
i32 = dict(dtype=torch.int32)


def z(*shape, dtype=torch.float32):
    return torch.zeros(*shape, dtype=dtype)


def shape_error(fn, *args, **kw):
    """The call must fail with a shape complaint (not the later 'must be a
    device tensor' that correctly shaped host tensors would hit)."""
    with pytest.raises(ValueError, match="shape|required"):
        fn(*args, **kw)


def ok_until_device(fn, *args, **kw):
    with pytest.raises(ValueError, match="device tensor"):
        fn(*args, **kw)


def test_dispatch_layout_shapes():
    ids = z(T, K, **i32)
    args = dict(counts=z(L, **i32), offsets=z(L + 1, **i32), slot_of=z(T, K, **i32),
                row_src=z(RC, **i32), tile_offsets=z(L + 1, **i32), dev_status=z(2, **i32),
                workspace=z(64, dtype=torch.uint8))

    def call(**over):
        a = dict(args, **over)
        return ep.moe_dispatch_layout(ids, 8, 0, L, R, 128, a["counts"], a["offsets"], a["slot_of"],
                                      a["row_src"], a["tile_offsets"], a["dev_status"], a["workspace"])
    ok_until_device(call)
    for name, bad in [("counts", z(L + 1, **i32)), ("offsets", z(L, **i32)),
                      ("slot_of", z(T, K + 1, **i32)), ("row_src", z(RC - 1, **i32)),
                      ("tile_offsets", z(L, **i32)), ("dev_status", z(1, **i32))]:
        shape_error(call, **{name: bad})
    # exact-fit: rows_cap = T*K
    shape_error(lambda: ep.moe_dispatch_layout(ids, 8, 0, L, 0, 128, *[args[k] for k in
                ("counts", "offsets", "slot_of", "row_src", "tile_offsets", "dev_status", "workspace")]))


def test_permute_shapes():
    x = z(T, H, dtype=torch.bfloat16)
    slot = z(T, K, **i32)
    ok_until_device(ep.moe_permute, x, slot, z(RC, H, dtype=torch.uint8), z(RC, H // 128))
    shape_error(ep.moe_permute, x, z(T + 1, K, **i32), z(RC, H, dtype=torch.uint8), z(RC, H // 128))
    shape_error(ep.moe_permute, x, slot, z(RC, H + 128, dtype=torch.uint8), z(RC, H // 128))
    shape_error(ep.moe_permute, x, slot, z(RC, H, dtype=torch.uint8), z(RC - 1, H // 128))
    shape_error(ep.moe_permute, x, slot, z(RC, H, dtype=torch.uint8), None)


def test_gemm_w13_shapes():
    a, a_s = z(RC, H, dtype=torch.uint8), z(RC, H // 128)
    w, w_s = z(L, 2 * I, H, dtype=torch.uint8), z(L, 2 * I // 128, H // 128)
    c, o = z(L, **i32), z(L + 1, **i32)
    zz, zs = z(RC, I, dtype=torch.uint8), z(RC, I // 128)
    fused = ep.MOE_EPI_SILU_MUL
    ok_until_device(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, o, fused, zz, zs)
    shape_error(ep.moe_grouped_gemm_w13, z(RC, H + 128, dtype=torch.uint8), a_s, w, w_s, c, o, fused, zz, zs)
    shape_error(ep.moe_grouped_gemm_w13, a, z(RC, 1), w, w_s, c, o, fused, zz, zs)
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, z(L, 1, 1), c, o, fused, zz, zs)
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, z(L - 1, **i32), o, fused, zz, zs)
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, z(L - 1, **i32), fused, zz, zs)
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, o, fused, z(RC - 1, I, dtype=torch.uint8), zs)
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, o, fused, zz, z(RC, 2))
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, o, fused, zz, None)
    shape_error(ep.moe_grouped_gemm_w13, a, None, w, w_s, c, o, fused, zz, zs)
    # the stored-G epilogue writes [rows_cap, 2I] fp32
    shape_error(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, o, ep.MOE_EPI_STORE_G, z(RC, I))
    ok_until_device(ep.moe_grouped_gemm_w13, a, a_s, w, w_s, c, o, ep.MOE_EPI_STORE_G, z(RC, 2 * I))


def test_silu_mul_and_gemm_w2_shapes():
    g, c, o = z(RC, 2 * I), z(L, **i32), z(L + 1, **i32)
    ok_until_device(ep.moe_silu_mul, g, c, o, z(RC, I, dtype=torch.uint8), z(RC, I // 128))
    shape_error(ep.moe_silu_mul, g, c, o, z(RC, 2 * I, dtype=torch.uint8), z(RC, I // 128))
    shape_error(ep.moe_silu_mul, g, c, z(L - 1, **i32), z(RC, I, dtype=torch.uint8), z(RC, I // 128))
    shape_error(ep.moe_silu_mul, g, c, o, z(RC, I, dtype=torch.uint8), None)

    zz, zs = z(RC, I, dtype=torch.uint8), z(RC, I // 128)
    w2, w2s = z(L, H, I, dtype=torch.uint8), z(L, H // 128, I // 128)
    out = z(RC, H, dtype=torch.bfloat16)
    ok_until_device(ep.moe_grouped_gemm_w2, zz, zs, w2, w2s, c, o, out)
    shape_error(ep.moe_grouped_gemm_w2, zz, zs, w2, w2s, c, o, z(RC, H - 128, dtype=torch.bfloat16))
    shape_error(ep.moe_grouped_gemm_w2, zz, zs, w2, w2s, c, o, z(RC + 1, H, dtype=torch.bfloat16))
    shape_error(ep.moe_grouped_gemm_w2, z(RC, 2 * I, dtype=torch.uint8), zs, w2, w2s, c, o, out)
    shape_error(ep.moe_grouped_gemm_w2, zz, zs, w2, z(L, 1, 1), c, o, out)
    shape_error(ep.moe_grouped_gemm_w2, zz, zs, w2, w2s, z(L + 1, **i32), o, out)
    shape_error(ep.moe_grouped_gemm_w2, zz, None, w2, w2s, c, o, out)


def test_combine_router_and_backward_shapes():
    eo, slot, w = z(RC, H, dtype=torch.bfloat16), z(T, K, **i32), z(T, K)
    ok_until_device(ep.moe_combine, eo, slot, w, z(T, H, dtype=torch.bfloat16))
    shape_error(ep.moe_combine, z(RC, H + 8, dtype=torch.bfloat16), slot, w, z(T, H, dtype=torch.bfloat16))
    shape_error(ep.moe_combine, eo, slot, z(T, K + 1), z(T, H, dtype=torch.bfloat16))
    shape_error(ep.moe_combine, eo, slot, w, z(T + 1, H, dtype=torch.bfloat16))

    E = 8
    ok_until_device(ep.moe_router_topk, z(T, E), K, z(T, K, **i32), z(T, K), bias=z(E))
    shape_error(ep.moe_router_topk, z(T, E), K, z(T, K + 1, **i32), z(T, K))
    shape_error(ep.moe_router_topk, z(T, E), K, z(T, K, **i32), z(T - 1, K))
    shape_error(ep.moe_router_topk, z(T, E), K, z(T, K, **i32), z(T, K), bias=z(E + 1))

    dy = z(T, H, dtype=torch.bfloat16)
    ok_until_device(ep.moe_combine_backward, dy, eo, slot, w, z(RC, H, dtype=torch.bfloat16), z(T, K))
    shape_error(ep.moe_combine_backward, dy, eo, slot, w, z(RC, H // 2, dtype=torch.bfloat16), z(T, K))
    shape_error(ep.moe_combine_backward, dy, eo, slot, w, z(RC, H, dtype=torch.bfloat16), z(T, K + 2))
    c, o = z(L, **i32), z(L + 1, **i32)
    ok_until_device(ep.moe_silu_mul_backward, z(RC, 2 * I), z(RC, I, dtype=torch.bfloat16), c, o,
                    z(RC, 2 * I, dtype=torch.bfloat16))
    shape_error(ep.moe_silu_mul_backward, z(RC, 2 * I), z(RC, 2 * I, dtype=torch.bfloat16), c, o,
                z(RC, 2 * I, dtype=torch.bfloat16))
    shape_error(ep.moe_silu_mul_backward, z(RC, 2 * I), z(RC, I, dtype=torch.bfloat16), c, o,
                z(RC, I, dtype=torch.bfloat16))
    ok_until_device(ep.moe_permute_backward, eo, slot, z(T, H, dtype=torch.bfloat16))
    shape_error(ep.moe_permute_backward, z(RC, H // 2, dtype=torch.bfloat16), slot,
                z(T, H, dtype=torch.bfloat16))
    shape_error(ep.moe_grouped_gemm_wgrad, z(RC, 2 * I, dtype=torch.bfloat16), z(RC, H, dtype=torch.bfloat16),
                c, z(L - 1, **i32), z(L, 2 * I, H))
