"""Pins for the oracle's expert MLP, combine and whole layer (CPU only).

* expert MLP vs torch's float64 F.linear / F.silu composition (a library
  implementation of the gated-SiLU expert of "SGLang Expert Compute Backend"
  §1.1), SiLU vs torch's fp32 silu, special cases that fix gate/up order and
  weight orientation (zero gate -> zero output, zero down -> zero output);
* storage layouts vs the element offsets printed in §3.5-§3.7 of that page;
* combine: 0.25*4 + 0.75*12 = 10 ("SGLang、NCCL 与 MoE EP" §1.1/§3.2),
  invariance under 50 shuffled slot orders (§B.4 of that page), partial-sum
  linearity across disjoint local expert ranges, zero for no local route;
* whole layer vs a dense brute-force MoE that enumerates each token's routes
  from the source ids and never uses the layout ("SGLang、NCCL 与 MoE EP"
  §5.1), and capacity invariance (same output at R and 2R).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import formats as F
from oracle import moe
from workloads import get_config, make_workload


def rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_silu_matches_torch():
    v = np.concatenate([rand(100_000, 0, 6.0), np.array([0, -0.0, 88, -88, 100, -100], np.float32)])
    ref = TF.silu(torch.from_numpy(v)).numpy()
    assert np.allclose(moe.silu(v), ref, rtol=3e-7, atol=1e-30)
    assert moe.silu(np.array([0.0], np.float32))[0] == 0.0


@pytest.mark.parametrize("z_dt", ["f32", "bf16", "fp8"])
def test_expert_mlp_matches_torch_float64(z_dt):
    H, I, m = 256, 384, 37
    a = rand((m, H), 1).astype(np.float64)
    w13 = rand((2 * I, H), 2, H ** -0.5).astype(np.float64)
    w2 = rand((H, I), 3, I ** -0.5).astype(np.float64)
    g = moe.gemm_w13(a, w13)
    z = moe.silu_mul(g, I)
    zf = moe.z_to_format(z, z_dt)
    zv = moe.buffer_values(zf["data"], z_dt, zf.get("scales"))
    out = moe.gemm_w2(zv, w2)
    ta, t13, t2 = (torch.from_numpy(v) for v in (a, w13, w2))
    tg = TF.linear(ta, t13)
    tz = TF.silu(tg[:, :I]) * tg[:, I:]
    assert np.allclose(g, tg.numpy(), rtol=1e-6, atol=1e-6)
    assert np.allclose(z, tz.numpy(), rtol=1e-5, atol=1e-6)
    ref = TF.linear(tz, t2).numpy()
    tol = {"f32": 1e-5, "bf16": 1e-2, "fp8": 8e-2}[z_dt]
    err = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert err < tol
    if z_dt == "f32":
        assert np.allclose(out, ref, rtol=1e-5, atol=1e-6)


def test_gate_is_first_half_and_weights_are_out_by_in():
    H, I = 128, 128
    a = rand((4, H), 5).astype(np.float64)
    w13 = rand((2 * I, H), 6).astype(np.float64)
    w2 = rand((H, I), 7).astype(np.float64)
    zero_gate = w13.copy()
    zero_gate[:I] = 0           # SiLU(0) = 0 kills every output
    z = moe.silu_mul(moe.gemm_w13(a, zero_gate), I)
    assert np.all(z == 0)
    zero_up = w13.copy()
    zero_up[I:] = 0             # up = 0 also kills it; gate alone does not
    assert np.all(moe.silu_mul(moe.gemm_w13(a, zero_up), I) == 0)
    z = moe.silu_mul(moe.gemm_w13(a, w13), I)
    assert np.all(moe.gemm_w2(z.astype(np.float64), np.zeros((H, I))) == 0)
    # orientation: a weight whose row n is e_j makes G[:, n] = A[:, j]
    w = np.zeros((2 * I, H))
    w[3, 17] = 1.0
    assert np.array_equal(moe.gemm_w13(a, w)[:, 3], a[:, 17].astype(np.float32))


def test_storage_layouts_match_printed_offsets(gold):
    g = gold("address_offsets.json")
    cfg = get_config("share_bf16")
    L, R, H, I = cfg.L, cfg.R, cfg.H, cfg.I
    fp8 = cfg.scaled(wdt="fp8")
    wl = make_workload(fp8)
    shapes = {
        "A": (L * R, H), "W13": wl.w["w13"].shape, "A_scale": (L * R, H // 128),
        "W13_scale": wl.w["w13_scales"].shape, "G": (L * R, 2 * I), "Z": (L * R, I),
        "W2": wl.w["w2"].shape, "Z_scale": (L * R, I // 128), "W2_scale": wl.w["w2_scales"].shape,
        "OUT": (L * R, H),
    }
    assert shapes["W13"] == (L, 2 * I, H) and shapes["W2"] == (L, H, I)
    for o in g["offsets"]:
        assert np.ravel_multi_index(tuple(o["index"]), shapes[o["tensor"]]) == o["offset"], o
    for v in g["view_restore"]:
        assert divmod(v["q"], R) == (v["expert"], v["s"])
    # the quantised activation scale layout is [rows, H/128]
    codes, scales = F.quant_fp8_groups(rand((3, H), 9))
    assert scales.shape == (3, H // 128)


def test_combine_weighted_sum(gold):
    g = gold("combine_weighted_sum.json")
    out_rows = {0: np.array([g["expert_outputs"][0]], np.float32),
                1: np.array([g["expert_outputs"][1]], np.float32)}
    slot_of = np.array([[0, 1]], np.int32)
    w = np.array([g["weights"]], np.float32)
    y = moe.combine(out_rows, slot_of, w, "f32")
    assert y[0, 0] == g["combined"]
    # the weight multiplies the expert output, not its input: a nonlinear
    # expert gives a different value if the weight is applied first
    v = np.float32(3.0)
    assert moe.silu(np.float32(0.25) * v) != np.float32(0.25) * moe.silu(v)


def test_combine_invariant_under_50_slot_orders():
    rng = np.random.default_rng(0)
    T, K, H, nrows = 40, 3, 16, 200
    rows = rng.choice(nrows, T * K, replace=False)
    slot_of = rows.reshape(T, K).astype(np.int32)
    slot_of[rng.random((T, K)) < 0.2] = -1
    w = rng.random((T, K)).astype(np.float32)
    vals = rand((nrows, H), 1)
    base = moe.combine({q: vals[q] for q in range(nrows)}, slot_of, w, "f32")
    for trial in range(50):
        perm = rng.permutation(nrows)            # move every row somewhere else
        moved = np.empty_like(vals)
        moved[perm] = vals
        so = np.where(slot_of >= 0, perm[np.maximum(slot_of, 0)], -1).astype(np.int32)
        y = moe.combine({q: moved[q] for q in range(nrows)}, so, w, "f32")
        assert np.array_equal(y, base)


def test_combine_partial_sums_and_empty_tokens():
    # two disjoint local expert ranges, each token has one route in each:
    # the two partial combines sum to the full combine exactly
    wl = make_workload("toy_fp32")
    cfg = wl.cfg
    full = moe.moe_layer(wl)
    lo = make_workload(cfg.scaled(L=4, expert_begin=0, R=128))
    hi = make_workload(cfg.scaled(L=4, expert_begin=4, R=128))
    lo.w = {k: v[:4] for k, v in wl.w.items()}
    hi.w = {k: v[4:] for k, v in wl.w.items()}
    y_lo, y_hi = moe.moe_layer(lo)["y"], moe.moe_layer(hi)["y"]
    assert np.array_equal(y_lo + y_hi, full["y"])
    # a GPU share with no local route for any token returns zeros
    none = make_workload(cfg.scaled(L=2, expert_begin=2, R=128))
    none.w = {k: v[2:4] for k, v in wl.w.items()}
    assert np.all(moe.moe_layer(none)["y"] == 0)


# ---------------------------------------------------------------- brute force

def ieee_div(num: float, den: torch.Tensor) -> torch.Tensor:
    """Correctly rounded fp32 quotient.  torch's CPU ``scalar / tensor`` can be
    one ulp off (it is not an IEEE division), which flips an FP8 code when the
    product lands on a rounding tie; dividing in float64 and rounding once to
    fp32 gives the IEEE fp32 quotient (float64 has more than 2*24+2 bits)."""
    return (num / den.double()).float()


def dense_reference(wl, tokens):
    """Dense MoE that never uses the layout: for each token and each k, run
    its expert on x[t] with torch float64 ops and add w * output."""
    cfg = wl.cfg
    out = []
    xv = moe.x_values(wl.x, cfg.act) if wl.x is not None else None
    for t in tokens:
        acc = torch.zeros(cfg.H, dtype=torch.float32)
        for k in range(cfg.K):
            if cfg.routing == "given":
                q = int(wl.share["slot_of"][t, k])
                e = q // cfg.R
                a = torch.from_numpy(F.bf16_to_f32(wl.share["buf"][q]).astype(np.float64))
            else:
                gid = int(wl.ids[t, k])
                if not (cfg.expert_begin <= gid < cfg.expert_begin + cfg.L):
                    continue
                e = gid - cfg.expert_begin
                row = torch.from_numpy(xv[t].copy())
                if cfg.buf_dt == "fp8":   # the activation cast, written with torch ops
                    b = row.view(-1, 128)
                    amax = b.abs().amax(dim=1).clamp(min=1e-4)
                    c8 = (b * ieee_div(448.0, amax)[:, None]).to(torch.float8_e4m3fn)
                    a = (c8.to(torch.float64) * (amax / 448.0).double()[:, None]).reshape(-1)
                else:
                    a = row.double()
            w13 = torch.from_numpy(moe.weight_values(wl.w["w13"][e], cfg.wdt,
                                                     wl.w.get("w13_scales", [None] * (e + 1))[e]))
            w2 = torch.from_numpy(moe.weight_values(wl.w["w2"][e], cfg.wdt,
                                                    wl.w.get("w2_scales", [None] * (e + 1))[e]))
            g = TF.linear(a, w13).float()
            z = TF.silu(g[:cfg.I]) * g[cfg.I:]
            if cfg.z_dt == "fp8":
                b = z.view(-1, 128)
                amax = b.abs().amax(dim=1).clamp(min=1e-4)
                c8 = (b * ieee_div(448.0, amax)[:, None]).to(torch.float8_e4m3fn)
                zd = (c8.to(torch.float64) * (amax / 448.0).double()[:, None]).reshape(-1)
            elif cfg.z_dt == "bf16":
                zd = z.to(torch.bfloat16).double()
            else:
                zd = z.double()
            o = TF.linear(zd, w2).float()
            if cfg.out_dt == "bf16":
                o = o.to(torch.bfloat16).float()
            acc = acc + float(wl.weights[t, k]) * o
        if cfg.out_dt == "bf16":
            acc = acc.to(torch.bfloat16).float()
        out.append(acc.numpy())
    return np.stack(out)


@pytest.mark.parametrize("name", ["toy_fp32", "share_bf16", "toy_bf16_fp8w", "decode_fp8_small",
                                  "skewed_bf16_small"])
def test_layer_matches_dense_brute_force(name):
    wl = make_workload(name)
    T = wl.cfg.T
    tokens = np.arange(T) if T <= 128 else np.random.default_rng(0).choice(T, 64, replace=False)
    got = moe.moe_layer(wl, tokens=tokens)["y"]
    ref = dense_reference(wl, tokens)
    # the fp32 path differs only by SiLU's last-ulp rounding (numpy vs torch);
    # where Z and the outputs are rounded to bf16 / FP8 those ulps vanish and
    # the two agree exactly
    if wl.cfg.z_dt == "f32":
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel < 1e-6, rel
    else:
        assert np.array_equal(got, ref)


def test_layer_subset_equals_full():
    wl = make_workload("decode_fp8_small")
    full = moe.moe_layer(wl)
    tokens = np.array([0, 7, 31, 63])
    sub = moe.moe_layer(wl, tokens=tokens)
    assert np.array_equal(sub["y"], full["y"][tokens])


def test_capacity_invariance():
    wl = make_workload("toy_fp32")
    y1 = moe.moe_layer(wl)["y"]
    wl2 = make_workload(wl.cfg.scaled(R=256))
    wl3 = make_workload(wl.cfg.scaled(R=0))
    assert np.array_equal(moe.moe_layer(wl2)["y"], y1)
    assert np.array_equal(moe.moe_layer(wl3)["y"], y1)


def test_token5_layer_is_weighted_expert_outputs():
    wl = make_workload("toy_fp32")
    res = moe.moe_layer(wl)
    out = res["mlp"]["out"]
    so = res["layout"]["slot_of"]
    y5 = (np.float32(0.25) * out[so[5, 0]]).astype(np.float32) + \
        (np.float32(0.75) * out[so[5, 1]]).astype(np.float32)
    assert np.array_equal(res["y"][5], y5.astype(np.float32))
    assert so[5].tolist() == [128, 768]


def test_gemm_flops():
    assert moe.gemm_flops(7168, 2048, 1) == 6 * 7168 * 2048
    assert moe.gemm_flops(256, 128, 224) == 224 * 6 * 256 * 128
