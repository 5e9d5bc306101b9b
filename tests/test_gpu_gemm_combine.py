"""GPU parity: grouped GEMMs, SiLU*up and combine, stage by stage.

Each stage gets the oracle's own inputs for that stage (so upstream rounding
differences do not mix in) and is compared element by element on every valid
row, with the bounds of tests/parity_bounds.py: every G and expert-output
element within the dot product's error bound (eps(dtype, K) * sum |a w|)
of the oracle's float64 result, plus one unit of the stored format; every Z
element (fp32, bf16, or FP8 code and group scale) a correct rounding of an
SiLU(gate)*up within the bound that G's bound implies.  Combine, given
identical expert outputs, is bit-exact (same fp32 operations in the same
order)."""
import numpy as np
import pytest
import torch

import parity_bounds as PB
from gpu_util import (GEMM_REL_L2, announce, dev, host_bits, host_vals, layer_shape, need_gpu,
                      rel_l2, upload_weights)
from oracle import formats as F
from oracle import moe
from workloads import get_config, make_routing, make_share_buffer, make_workload

pytestmark = pytest.mark.gpu

# the last three: few experts with hundreds of rows each (many row tiles per
# expert), odd and single-stage K loops
GEMM_CASES = ["toy_fp32", "share_bf16", "toy_bf16_fp8w", "decode_fp8_small", "prefill_fp8_small",
              "skewed_bf16_small", "manyrow_bf16_small", "manyrow_fp8_small", "manyrow_fp32_small"]


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


def oracle_stage_inputs(wl):
    """The oracle's expert-major buffer (valid rows), counts and offsets."""
    cfg = wl.cfg
    if cfg.routing == "given":
        sh = wl.share
        rows = moe.valid_rows(sh["counts"], sh["offsets"])
        return {"counts": sh["counts"], "offsets": sh["offsets"], "rows": rows,
                "data": sh["buf"][rows], "scales": None, "slot_of": sh["slot_of"]}
    lay = moe.dispatch_layout(wl.ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    perm = moe.permute(wl.x, cfg.act, lay["row_src"], cfg.K, cfg.buf_dt)
    return {"counts": lay["counts"], "offsets": lay["offsets"], "rows": perm["rows"],
            "data": perm["data"], "scales": perm.get("scales"), "slot_of": lay["slot_of"]}


def make_layer_with_buffer(wl, inp, fused):
    from combine_top_expert_amd.pipeline import MoELayer
    cfg = wl.cfg
    layer = MoELayer(layer_shape(cfg), fused=fused)
    upload_weights(layer, wl)
    layer.counts.copy_(dev(inp["counts"]))
    layer.offsets.copy_(dev(inp["offsets"]))
    layer.slot_of.copy_(dev(inp["slot_of"]))
    # NaN in every padding row of the A buffer: it must never reach a result
    full = np.zeros((cfg.rows_cap, cfg.H), inp["data"].dtype)
    if cfg.buf_dt == "fp8":
        full[:] = 0x7F
    elif cfg.buf_dt == "bf16":
        full[:] = 0xFFFF
    else:
        full[:] = np.nan
    full[inp["rows"]] = inp["data"]
    layer.buf.copy_(dev(full, "bf16" if cfg.buf_dt == "bf16" else None))
    if cfg.buf_dt == "fp8":
        sc = np.full((cfg.rows_cap, cfg.H // 128), np.nan, np.float32)
        sc[inp["rows"]] = inp["scales"]
        layer.buf_scales.copy_(dev(sc))
    return layer


def oracle_mlp(wl, inp):
    cfg = wl.cfg
    a_vals = moe.buffer_values(inp["data"], cfg.buf_dt, inp["scales"])
    e_of = {int(q): int(np.searchsorted(inp["offsets"], q, side="right") - 1) for q in inp["rows"]}
    a_by = {int(q): a_vals[i] for i, q in enumerate(inp["rows"])}
    return moe.expert_mlp_rows(cfg, a_by, e_of, moe.ExpertWeights(cfg, wl.w))


def per_expert(inp):
    """(expert, positions in inp["rows"]) for every expert with rows."""
    e_of = np.searchsorted(inp["offsets"], inp["rows"], side="right") - 1
    return [(int(e), np.nonzero(e_of == e)[0]) for e in np.unique(e_of)]


def g_reference(wl, inp, ref):
    """The oracle's G on the stage's rows and its per-element bound."""
    cfg = wl.cfg
    ew = moe.ExpertWeights(cfg, wl.w)
    a_vals = moe.buffer_values(inp["data"], cfg.buf_dt, inp["scales"])
    rows = inp["rows"]
    g_ref = np.stack([ref["G"][int(q)] for q in rows])
    bound = np.zeros_like(g_ref, dtype=np.float64)
    for e, idx in per_expert(inp):
        bound[idx] = PB.eps(cfg.wdt, cfg.H) * PB.abs_dot(a_vals[idx], ew.w13(e))
    return g_ref, bound


def check_out(wl, inp, out_rows, z_codes, z_scales, tag):
    """Expert outputs against the oracle's down GEMM on the given Z rows."""
    cfg = wl.cfg
    ew = moe.ExpertWeights(cfg, wl.w)
    zv = moe.buffer_values(z_codes, cfg.z_dt, z_scales)
    reps = []
    for e, idx in per_expert(inp):
        w2 = ew.w2(e)
        reps.append(PB.check_values(out_rows[idx], moe.gemm_w2(zv[idx], w2),
                                    PB.eps(cfg.wdt, cfg.I) * PB.abs_dot(zv[idx], w2), cfg.out_dt,
                                    f"{tag} e{e}"))
    return max(r["worst_ratio"] for r in reps) if reps else 0.0


def z_host(layer, rows):
    codes = host_bits(layer.z)[rows]
    scales = layer.z_scales.cpu().numpy()[rows] if layer.z_scales is not None else None
    return codes, scales


@pytest.mark.parametrize("name", GEMM_CASES)
def test_gemm_w13_store_g(ep, name):
    announce("w13 G", name)
    wl = make_workload(name)
    inp = oracle_stage_inputs(wl)
    layer = make_layer_with_buffer(wl, inp, fused=False)
    layer.g.fill_(float("nan"))
    layer.gemm_w13()
    torch.cuda.synchronize()
    ref = oracle_mlp(wl, inp)
    g = layer.g.cpu().numpy()
    rows = inp["rows"]
    ref_g, bound = g_reference(wl, inp, ref)
    rep = PB.check_values(g[rows], ref_g, bound, "f32", f"G {name}")
    err = rel_l2(g[rows], ref_g)
    print(f"[metric] G {name} rel_l2={err:.3e} worst/bound={rep['worst_ratio']:.3e}", flush=True)
    assert err < GEMM_REL_L2[wl.cfg.wdt]
    pad = np.ones(wl.cfg.rows_cap, bool)
    pad[rows] = False
    assert np.all(np.isnan(g[pad])), "padding rows of G were written"


@pytest.mark.parametrize("name", GEMM_CASES)
def test_silu_mul_standalone(ep, name):
    """moe_silu_mul on the oracle's G: every Z element a correct rounding of
    SiLU(gate)*up (FP8 codes and scales by the recipe), up to the hardware
    SiLU's few fp32 ulps."""
    announce("silu_mul", name)
    wl = make_workload(name)
    cfg = wl.cfg
    inp = oracle_stage_inputs(wl)
    ref = oracle_mlp(wl, inp)
    layer = make_layer_with_buffer(wl, inp, fused=False)
    rows = inp["rows"]
    g = np.full((cfg.rows_cap, 2 * cfg.I), np.nan, np.float32)
    g[rows] = np.stack([ref["G"][int(q)] for q in rows])
    layer.g.copy_(dev(g))
    layer.silu_mul()
    torch.cuda.synchronize()
    # G is the oracle's exactly: only the hardware SiLU's few ulps remain
    codes, scales = z_host(layer, rows)
    rep = PB.check_z(codes, scales, cfg.z_dt, g[rows], np.zeros((len(rows), 2 * cfg.I)), cfg.I,
                     f"silu_mul {name}")
    print(f"[metric] silu_mul {name} {rep}", flush=True)


@pytest.mark.parametrize("name", GEMM_CASES)
def test_gemm_w13_fused_silu(ep, name):
    announce("w13 fused", name)
    wl = make_workload(name)
    cfg = wl.cfg
    inp = oracle_stage_inputs(wl)
    ref = oracle_mlp(wl, inp)
    layer = make_layer_with_buffer(wl, inp, fused=True)
    layer.gemm_w13()
    torch.cuda.synchronize()
    rows = inp["rows"]
    g_ref, bound = g_reference(wl, inp, ref)
    codes, scales = z_host(layer, rows)
    rep = PB.check_z(codes, scales, cfg.z_dt, g_ref, bound, cfg.I, f"w13 fused {name}")
    print(f"[metric] w13 fused {name} {rep}", flush=True)


@pytest.mark.parametrize("name", GEMM_CASES)
def test_gemm_w2(ep, name):
    """Down GEMM on the oracle's Z."""
    announce("w2", name)
    wl = make_workload(name)
    cfg = wl.cfg
    inp = oracle_stage_inputs(wl)
    ref = oracle_mlp(wl, inp)
    layer = make_layer_with_buffer(wl, inp, fused=True)
    rows = inp["rows"]
    zfull = np.zeros((cfg.rows_cap, cfg.I), {"fp8": np.uint8, "bf16": np.uint16, "f32": np.float32}[cfg.z_dt])
    zfull[rows] = np.stack([ref["Z"][int(q)] for q in rows])
    layer.z.copy_(dev(zfull, "bf16" if cfg.z_dt == "bf16" else None))
    if cfg.z_dt == "fp8":
        zs = np.zeros((cfg.rows_cap, cfg.I // 128), np.float32)
        zs[rows] = np.stack([ref["Zs"][int(q)] for q in rows])
        layer.z_scales.copy_(dev(zs))
    if layer.out.dtype == torch.bfloat16:
        layer.out.view(torch.int16).fill_(-1)
    else:
        layer.out.fill_(float("nan"))
    layer.gemm_w2()
    torch.cuda.synchronize()
    out = host_vals(layer.out)
    zc = np.stack([ref["Z"][int(q)] for q in rows])
    zs = np.stack([ref["Zs"][int(q)] for q in rows]) if cfg.z_dt == "fp8" else None
    worst = check_out(wl, inp, out[rows], zc, zs, f"w2 {name}")
    print(f"[metric] w2 {name} worst/bound={worst:.3e}", flush=True)
    pad = np.ones(cfg.rows_cap, bool)
    pad[rows] = False
    assert np.all(np.isnan(out[pad])), "padding rows of the expert output were written"


@pytest.mark.parametrize("name", GEMM_CASES + ["decode_fp8", "skewed_bf16"])
def test_combine_bit_exact(ep, name):
    """Combine of the oracle's expert outputs equals the oracle bit for bit."""
    announce("combine", name)
    cfg = get_config(name)
    rng = np.random.default_rng(0)
    if cfg.routing == "given":
        sh = make_share_buffer(cfg)
        slot_of, weights = sh["slot_of"], sh["weights"]
    else:
        ids, weights = make_routing(cfg)
        slot_of = moe.dispatch_layout(ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)["slot_of"]
    vals = rng.standard_normal((cfg.rows_cap, cfg.H)).astype(np.float32)
    if cfg.out_dt == "bf16":
        bits = F.f32_to_bf16(vals)
        vals = F.bf16_to_f32(bits)
        eo = dev(bits, "bf16")
    else:
        eo = dev(vals)
    out_rows = {q: vals[q] for q in range(cfg.rows_cap)}
    ref = moe.combine(out_rows, slot_of, weights, cfg.out_dt)
    y = torch.full((cfg.T, cfg.H), float("nan"), dtype=eo.dtype, device="cuda")
    ep.moe_combine(eo, dev(slot_of), dev(weights), y)
    torch.cuda.synchronize()
    assert np.array_equal(host_vals(y), ref)


def test_combine_weighted_sum_fact(ep, gold):
    """0.25 * 4 + 0.75 * 12 = 10 through the device combine."""
    announce("combine 4/12")
    g = gold("combine_weighted_sum.json")
    eo = torch.zeros(4, 8, device="cuda")
    eo[1, 0], eo[3, 0] = g["expert_outputs"][0], g["expert_outputs"][1]
    slot_of = torch.tensor([[1, 3], [-1, -1]], dtype=torch.int32, device="cuda")
    w = torch.tensor([g["weights"], [0.5, 0.5]], dtype=torch.float32, device="cuda")
    y = torch.full((2, 8), 7.0, device="cuda")
    ep.moe_combine(eo, slot_of, w, y)
    torch.cuda.synchronize()
    assert y[0, 0].item() == g["combined"]
    assert torch.all(y[1] == 0)         # no local route -> 0


def k_split_plan(n_tiles, grid, kstages, min_pieces=4, min_stages=32):
    """The kernel's work plan per XCD group of workgroups: (whole rounds,
    tiles in the last round, pieces per last-round tile).  The last round is
    split only for K of at least `min_stages` stages, and only into at least
    `min_pieces` pieces of at least two stages."""
    if grid >= 8 and grid % 8 == 0:
        slots, chunks = grid // 8, [((n_tiles * x) >> 3, (n_tiles * (x + 1)) >> 3) for x in range(8)]
    else:
        slots, chunks = grid, [(0, n_tiles)]
    plan = []
    for b, e in chunks:
        full, tail = divmod(e - b, slots)
        S = min(slots // tail, kstages // 2) if tail and kstages >= min_stages else 1
        plan.append((full, tail, S if S >= min_pieces else 1))
    return plan


def gemm_grid(rows_cap, L, nb_count):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mt = min(rows_cap // 128 + L, -(-rows_cap // 128) + L)
    g = min(mt * nb_count, cus)
    return g & ~7 if g >= 8 else g


# shapes whose last GEMM round is split along K (asserted below): few tiles
# against a large capacity-sized grid, at least 32 K stages; between them
# every epilogue kind of both GEMMs runs split
K_SPLIT_CASES = {
    "fp8_w13": ("prefill_fp8_small", dict(T=128, H=4096, I=1024)),
    "bf16_w13": ("skewed_bf16_small", dict(T=128, E=8, L=8, H=2048, I=512, R=512)),
    "bf16_w2": ("skewed_bf16_small", dict(T=64, E=8, L=8, H=2048, I=2048, R=512)),
    "f32": ("toy_fp32", dict(H=1024, I=1024)),
}


@pytest.mark.parametrize("case", sorted(K_SPLIT_CASES))
def test_gemm_k_split_matches_unsplit(ep, case):
    """With a workspace the GEMMs split an incomplete last round along K and
    add the pieces in a second kernel.  Both launches (with and without the
    workspace) are checked element by element against the oracle: G within
    its bound, Z a correct rounding, and the expert output of each launch's
    own Z within the down GEMM's bound; split and unsplit G agree to 1e-6
    relative L2 (only the fp32 summation order differs)."""
    base, kw = K_SPLIT_CASES[case]
    cfg = get_config(base).scaled(name=f"ksplit_{case}", **kw)
    announce("k-split", cfg.name)
    wl = make_workload(cfg)
    inp = oracle_stage_inputs(wl)
    esz = {"fp8": 1, "bf16": 2, "f32": 4}[cfg.wdt]
    mts = int(sum(-(-int(c) // 128) for c in inp["counts"]))
    splits = {}
    for g, K, nb in [("w13", cfg.H, cfg.I // 128), ("w2", cfg.I, -(-cfg.H // 256))]:
        plan = k_split_plan(mts * nb, gemm_grid(cfg.rows_cap, cfg.L, nb), K * esz // 128)
        splits[g] = max(S for _, _, S in plan)
    assert max(splits.values()) > 1, f"{cfg.name}: no K split in this shape ({splits})"
    layer = make_layer_with_buffer(wl, inp, fused=True)
    g_buf = torch.empty(cfg.rows_cap, 2 * cfg.I, dtype=torch.float32, device="cuda")
    rows = inp["rows"]
    outs = {}
    for use_ws in (False, True):
        ws = layer.gemm_workspace if use_ws else None
        g_buf.zero_()
        ep.moe_grouped_gemm_w13(layer.buf, layer.buf_scales, layer.w13, layer.w13_scales,
                                layer.counts, layer.offsets, ep.MOE_EPI_STORE_G, g_buf, workspace=ws)
        layer.z.zero_()
        ep.moe_grouped_gemm_w13(layer.buf, layer.buf_scales, layer.w13, layer.w13_scales,
                                layer.counts, layer.offsets, ep.MOE_EPI_SILU_MUL, layer.z,
                                layer.z_scales, workspace=ws)
        torch.cuda.synchronize()
        z_codes, z_scales = z_host(layer, rows)
        if not use_ws:
            z_in = layer.z.clone()
            zs_in = None if layer.z_scales is None else layer.z_scales.clone()
        layer.out.zero_()
        ep.moe_grouped_gemm_w2(z_in, zs_in, layer.w2, layer.w2_scales, layer.counts,
                               layer.offsets, layer.out, workspace=ws)
        torch.cuda.synchronize()
        outs[use_ws] = (host_vals(g_buf)[rows], z_codes, z_scales, host_vals(layer.out)[rows],
                        z_in, zs_in)
    ref = oracle_mlp(wl, inp)
    g_ref, bound = g_reference(wl, inp, ref)
    zc0, zs0 = outs[False][1], outs[False][2]
    for use_ws, (g_, zc, zs, o_, _, _) in outs.items():
        tag = f"{cfg.name} {'split' if use_ws else 'unsplit'}"
        PB.check_values(g_, g_ref, bound, "f32", f"G {tag}")
        rep = PB.check_z(zc, zs, cfg.z_dt, g_ref, bound, cfg.I, f"Z {tag}")
        # the down GEMM of both launches ran on the unsplit launch's Z
        worst = check_out(wl, inp, o_, zc0, zs0, f"out {tag}")
        print(f"[metric] {tag} split {splits} Z {rep} out worst/bound={worst:.3e}", flush=True)
    eg = rel_l2(outs[True][0], outs[False][0])
    print(f"[metric] {cfg.name} split vs unsplit G rel_l2={eg:.2e}", flush=True)
    assert eg < 1e-6


@pytest.mark.parametrize("name", ["toy_fp32", "toy_bf16_fp8w", "decode_fp8_small", "prefill_fp8_small",
                                  "skewed_bf16_small", "manyrow_fp8_small"])
def test_pack_w13_and_packed_gemm(ep, name):
    """moe_pack_w13 writes the row-major weights' bytes in the staging order
    [L][I/128][H*esz/128][gate 128 rows, up 128 rows][128 bytes], and the
    gate/up GEMM gives bit-identical G and Z from either layout (same loads
    into the same LDS positions, only the global addresses differ)."""
    announce("pack w13", name)
    wl = make_workload(name)
    cfg = wl.cfg
    inp = oracle_stage_inputs(wl)
    layer = make_layer_with_buffer(wl, inp, fused=True)
    L, H, I = cfg.L, cfg.H, cfg.I
    rb = layer.w13.view(torch.uint8).cpu().numpy().reshape(L, 2 * I, -1)
    ks = rb.shape[2] // 128
    want = rb.reshape(L, 2, I // 128, 128, ks, 128).transpose(0, 2, 4, 1, 3, 5).ravel()
    got = layer.w13_packed.view(torch.uint8).cpu().numpy().ravel()
    assert np.array_equal(got, want)
    g = torch.empty(cfg.rows_cap, 2 * I, dtype=torch.float32, device="cuda")
    res = {}
    for lay, w in [(ep.MOE_W_ROW_MAJOR, layer.w13), (ep.MOE_W_PACKED, layer.w13_packed)]:
        g.fill_(float("nan"))
        ep.moe_grouped_gemm_w13(layer.buf, layer.buf_scales, w, layer.w13_scales, layer.counts,
                                layer.offsets, ep.MOE_EPI_STORE_G, g, w13_layout=lay,
                                workspace=layer.gemm_workspace)
        layer.z.zero_()
        ep.moe_grouped_gemm_w13(layer.buf, layer.buf_scales, w, layer.w13_scales, layer.counts,
                                layer.offsets, ep.MOE_EPI_SILU_MUL, layer.z, layer.z_scales,
                                w13_layout=lay, workspace=layer.gemm_workspace)
        torch.cuda.synchronize()
        zs = None if layer.z_scales is None else layer.z_scales.cpu().numpy().copy()
        res[lay] = (host_bits(g), host_bits(layer.z), zs)
    rows = inp["rows"]
    (g0, z0, s0), (g1, z1, s1) = res[ep.MOE_W_ROW_MAJOR], res[ep.MOE_W_PACKED]
    assert np.array_equal(g0[rows].view(np.uint32), g1[rows].view(np.uint32))
    assert np.array_equal(z0[rows], z1[rows])
    if s0 is not None:
        assert np.array_equal(s0[rows].view(np.uint32), s1[rows].view(np.uint32))
