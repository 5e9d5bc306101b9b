"""GPU parity of the backward (bf16 / fp32 layers) against oracle/backward.py.

Stage by stage, each GPU step gets the GPU's own inputs for that step (so
upstream rounding differences do not mix in) and is compared with the
oracle's step on the same values:
  * combine backward: d_out bit-exact (one fp32 product, same rounding),
    d_w to 1e-5 relative (fp32 vs float64 dot);
  * down-GEMM data gradient dZ and gate/up data gradient dA: the grouped
    GEMM on transposed weights against float64 products, bars of the
    forward GEMM tests;
  * SiLU*up backward: hardware exp2/reciprocal against numpy's exp, 1e-5
    relative L2 (fp32) or the bf16 step;
  * permute backward: bit-exact (fp32 sums in k order);
  * weight gradients dW2 = d_out^T Z and dW13 = dG^T A: fp32 sums of exact
    products against float64, 1e-5 relative L2 per expert, exact zeros for
    experts without rows;
and end to end, dx, d_w, dW2 and dW13 against the oracle's own backward (its
own forward values), to the bars the rounding chain allows."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev, host_vals, layer_shape, need_gpu, rel_l2, upload_weights
from oracle import backward as B
from oracle import moe
from workloads import get_config, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


def _config(name):
    if name == "share_fp32":
        # 4 of 8 experts local: non-local routes and tokens with no local route
        return get_config("toy_fp32").scaled(name="toy_fp32_share", L=4, expert_begin=2, T=48,
                                             routing="softmax")
    return get_config(name)


# ":saved_g" runs the unfused forward, which keeps G for the backward (no recompute)
CASES = ["toy_fp32", "share_fp32", "manyrow_fp32_small", "skewed_bf16_small", "manyrow_bf16_small",
         "share_fp32:saved_g", "skewed_bf16_small:saved_g"]


def _run(ep, case):
    from combine_top_expert_amd.pipeline import MoELayer
    name, _, mode = case.partition(":")
    cfg = _config(name)
    wl = make_workload(cfg)
    layer = MoELayer(layer_shape(cfg), fused=(mode != "saved_g"))
    upload_weights(layer, wl)
    bf = cfg.act == "bf16"
    x = dev(wl.x, "bf16" if bf else None)
    w = dev(wl.weights)
    layer.forward(x, dev(wl.ids), w)
    rng = np.random.default_rng(11)
    dy32 = rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)
    dy_vals = B.to_format(dy32, "bf16" if bf else "f32")
    dy = torch.from_numpy(dy_vals).cuda().to(torch.bfloat16 if bf else torch.float32)
    names = [n for n, _ in layer.backward_stages(dy, w)]
    assert ("gemm_g_silu_bw" in names) == (mode != "saved_g")     # G recomputed with dG in its epilogue
    assert "gemm_g" not in names
    dx, d_w = layer.backward(dy, w)
    torch.cuda.synchronize()
    return cfg, wl, layer, dy_vals, host_vals(dx), d_w.cpu().numpy()


@pytest.mark.parametrize("name", CASES)
def test_backward_stages(ep, name):
    announce("backward stages", name)
    cfg, wl, layer, dy_vals, _, d_w = _run(ep, name)
    gdt = "bf16" if cfg.act == "bf16" else "f32"
    slot_of = layer.slot_of.cpu().numpy()
    counts, offsets = layer.counts.cpu().numpy(), layer.offsets.cpu().numpy()
    rows = moe.valid_rows(counts, offsets)
    out = host_vals(layer.out)
    # combine backward on the GPU's own expert outputs
    d_out_ref, d_w_ref = B.combine_backward(dy_vals, {int(q): out[q] for q in rows}, slot_of,
                                            wl.weights, gdt)
    d_out = host_vals(layer.d_out)
    assert np.array_equal(np.stack([d_out[q] for q in rows]).view(np.uint32),
                          np.stack([d_out_ref[int(q)] for q in rows]).view(np.uint32))
    assert rel_l2(d_w, d_w_ref) < 1e-5
    assert np.all(d_w[slot_of < 0] == 0)
    # dZ = d_out W2[e] and dA = dG W13[e] on the GPU's inputs
    ew = moe.ExpertWeights(cfg, wl.w)
    e_of = {int(q): int(np.searchsorted(offsets, q, side="right") - 1) for q in rows}
    dz = host_vals(layer.dz)
    dg = host_vals(layer.dg)
    da = host_vals(layer.da)
    a_gpu = host_vals(layer.buf)
    if layer.g is not None:                      # kept by the unfused forward
        g = layer.g.cpu().numpy()
    else:                                        # never stored: float64 G on the GPU's A
        g = np.zeros((cfg.rows_cap, 2 * cfg.I))
        for q in rows:
            g[q] = a_gpu[q].astype(np.float64) @ ew.w13(e_of[int(q)]).T
    dz_ref = np.stack([d_out[q].astype(np.float64) @ ew.w2(e_of[int(q)]) for q in rows])
    da_ref = np.stack([dg[q].astype(np.float64) @ ew.w13(e_of[int(q)]) for q in rows])
    tol = 1e-5 if gdt == "f32" else 4e-3
    assert rel_l2(dz[rows], dz_ref) < tol
    assert rel_l2(da[rows], da_ref) < tol
    # SiLU*up backward on the GPU's G and dZ
    dg_ref = B.to_format(B.silu_mul_backward(g[rows], dz[rows]), gdt)
    assert rel_l2(dg[rows], dg_ref) < (1e-5 if gdt == "f32" else 4e-3)
    # permute backward on the GPU's dA: bit-exact
    dx_ref = B.permute_backward({int(q): da[q] for q in rows}, slot_of, cfg.H, gdt)
    dx = host_vals(layer.dx)
    assert np.array_equal(dx.view(np.uint32), dx_ref.view(np.uint32))
    # weight gradients on the GPU's own d_out, Z, dG and A
    z, a = host_vals(layer.z), host_vals(layer.buf)
    dw2, dw13 = layer.dw2.cpu().numpy(), layer.dw13.cpu().numpy()
    for e in range(cfg.L):
        qs = [q for q in rows if e_of[int(q)] == e]
        for got, bb, aa in ((dw2[e], d_out, z), (dw13[e], dg, a)):
            ref = B.wgrad(bb[qs], aa[qs], got.shape[0], got.shape[1])
            if not qs:
                assert not np.any(got)
            else:
                assert rel_l2(got, ref) < 1e-5, (e, len(qs))
    print(f"[metric] backward {name}: d_w rel {rel_l2(d_w, d_w_ref):.1e}", flush=True)


@pytest.mark.parametrize("name", CASES)
def test_backward_end_to_end(ep, name):
    """dx, d_w against the oracle's whole backward (its own forward values)."""
    announce("backward e2e", name)
    cfg, wl, layer, dy_vals, dx, d_w = _run(ep, name)
    res = B.layer_backward(wl, dy_vals, moe.ExpertWeights(cfg, wl.w))
    ex, ew_ = rel_l2(dx, res["dx"]), rel_l2(d_w, res["d_w"])
    print(f"[metric] backward e2e {name}: dx rel_l2 {ex:.2e}, d_w rel_l2 {ew_:.2e}", flush=True)
    bar = 1e-5 if cfg.act == "f32" else 2e-2
    assert ex < bar and ew_ < bar
    e2, e13 = rel_l2(layer.dw2.cpu().numpy(), res["dw2"]), rel_l2(layer.dw13.cpu().numpy(), res["dw13"])
    print(f"[metric] backward e2e {name}: dW2 rel_l2 {e2:.2e}, dW13 rel_l2 {e13:.2e}", flush=True)
    assert e2 < bar and e13 < bar
    no_local = ~(layer.slot_of.cpu().numpy() >= 0).any(axis=1)
    assert np.all(dx[no_local] == 0)


@pytest.mark.parametrize("shape", [(3, 200, 136), (3, 192, 320), (2, 2816, 4096)])
def test_transpose_weights(ep, shape):
    """Ragged sizes (element-wise kernel) and multiples of 64 (the 16-byte
    bf16 kernel), including the skewed shape's W13."""
    L, N, K = shape
    for dt in (torch.float32, torch.bfloat16):
        w = torch.randn(L, N, K, device="cuda").to(dt)
        wt = torch.empty(L, K, N, device="cuda", dtype=dt)
        ep.moe_transpose_weights(w, wt)
        torch.cuda.synchronize()
        assert torch.equal(wt.cpu(), w.cpu().transpose(1, 2))


@pytest.mark.parametrize("N,K", [(256, 384), (384, 256)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wgrad_ragged_experts(ep, dt, N, K):
    """Ragged expert row counts (0, 1, one chunk short, one chunk over, many
    chunks), padding rows filled with NaN (never read), several tiles and a
    128-column tail in either output dimension: against float64 per expert."""
    announce("wgrad ragged", dt, f"N={N} K={K}")
    counts = np.array([0, 1, 31, 33, 100, 0, 257], np.int32)
    R = 288                                   # capacity per expert; rows past the count are padding
    offsets = (np.arange(len(counts)) * R).astype(np.int32)
    rows_cap = R * len(counts)
    rng = np.random.default_rng(21)
    b = np.full((rows_cap, N), np.nan, np.float32)
    a = np.full((rows_cap, K), np.nan, np.float32)
    for e, c in enumerate(counts):
        b[offsets[e]:offsets[e] + c] = rng.standard_normal((c, N))
        a[offsets[e]:offsets[e] + c] = rng.standard_normal((c, K))
    if dt == "bf16":
        b, a = B.to_format(b, "bf16"), B.to_format(a, "bf16")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    c_dev = torch.full((len(counts), N, K), 7.0, device="cuda")
    ep.moe_grouped_gemm_wgrad(torch.from_numpy(b).cuda().to(tdt), torch.from_numpy(a).cuda().to(tdt),
                              dev(counts), dev(offsets), c_dev)
    torch.cuda.synchronize()
    got = c_dev.cpu().numpy()
    assert np.isfinite(got).all()
    for e, c in enumerate(counts):
        rs = slice(offsets[e], offsets[e] + c)
        ref = B.wgrad(b[rs], a[rs], N, K)
        if c == 0:
            assert not np.any(got[e])
        else:
            assert rel_l2(got[e], ref) < 1e-5, (e, c, rel_l2(got[e], ref))


def test_backward_full_size_sampled(ep):
    """The skewed bf16 shape at full size (T=16384, top-6 of 64, H=4096,
    I=1408) in the launch configuration the benchmark times: every stage on
    the GPU's own inputs at sampled tokens / rows, the weight gradients at
    sampled elements (column dot products over the expert's rows)."""
    from combine_top_expert_amd.pipeline import MoELayer
    announce("backward full", "skewed_bf16")
    cfg = get_config("skewed_bf16")
    wl = make_workload(cfg)
    layer = MoELayer(layer_shape(cfg))
    upload_weights(layer, wl)
    x, w = dev(wl.x, "bf16"), dev(wl.weights)
    layer.forward(x, dev(wl.ids), w)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    dy = torch.randn(cfg.T, cfg.H, device="cuda", generator=g).to(torch.bfloat16)
    # G recomputed with the SiLU*up gradient in the GEMM's epilogue (K-split
    # last round included at this shape), then again as stored fp32 G and a
    # separate SiLU*up backward: every gradient bit-identical
    names = [n for n, _ in layer.backward_stages(dy, w)]
    assert "gemm_g_silu_bw" in names and "silu_mul_bw" not in names
    layer.backward(dy, w)
    fused = {k: getattr(layer, k).clone() for k in ("dg", "da", "dx", "d_w", "dw2", "dw13")}
    layer.backward(dy, w, fuse_silu=False)
    torch.cuda.synchronize()
    for k, v in fused.items():
        assert torch.equal(v, getattr(layer, k)), f"{k}: fused and separate SiLU*up backward differ"
    del fused
    ew = moe.ExpertWeights(cfg, wl.w, cache=False)
    slot_of = layer.slot_of.cpu().numpy()
    counts, offsets = layer.counts.cpu().numpy(), layer.offsets.cpu().numpy()
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(cfg.T, 12, replace=False))
    hot = np.nonzero((slot_of >= offsets[0]) & (slot_of < offsets[0] + counts[0]))[0]
    tokens = np.unique(np.concatenate([tokens, hot[-2:]]))          # the hottest expert's tail
    rows = sorted({int(q) for t in tokens for q in slot_of[t] if q >= 0})

    def rows_of(t):
        return host_vals(t[torch.tensor(rows, device="cuda")])

    dyv = host_vals(dy[torch.tensor(tokens, device="cuda")])
    out, d_out = rows_of(layer.out), rows_of(layer.d_out)
    z, a, gg = rows_of(layer.z), rows_of(layer.buf), rows_of(layer.g_saved)
    dz, dg, da = rows_of(layer.dz), rows_of(layer.dg), rows_of(layer.da)
    ri = {q: i for i, q in enumerate(rows)}
    e_of = {q: int(np.searchsorted(offsets, q, side="right") - 1) for q in rows}
    wts = wl.weights
    d_w = layer.d_w.cpu().numpy()
    for j, t in enumerate(tokens):
        for k in range(cfg.K):
            q = int(slot_of[t, k])
            if q < 0:
                assert d_w[t, k] == 0
                continue
            ref = B.to_format((np.float32(wts[t, k]) * dyv[j]).astype(np.float32), "bf16")
            assert np.array_equal(d_out[ri[q]].view(np.uint32), ref.view(np.uint32))
            dot = float(dyv[j].astype(np.float64) @ out[ri[q]].astype(np.float64))
            assert abs(d_w[t, k] - dot) <= 1e-5 * max(1.0, abs(dot))
    for q in rows:
        i, e = ri[q], e_of[q]
        g_ref = a[i].astype(np.float64) @ ew.w13(e).T
        assert rel_l2(gg[i], g_ref) < 1e-5
        assert rel_l2(dz[i], d_out[i].astype(np.float64) @ ew.w2(e)) < 4e-3
        assert rel_l2(dg[i], B.to_format(B.silu_mul_backward(gg[i:i + 1], dz[i:i + 1])[0], "bf16")) < 4e-3
        assert rel_l2(da[i], dg[i].astype(np.float64) @ ew.w13(e)) < 4e-3
    dx = host_vals(layer.dx[torch.tensor(tokens, device="cuda")])
    for j, t in enumerate(tokens):
        acc = np.zeros(cfg.H, np.float32)
        for k in range(cfg.K):
            q = int(slot_of[t, k])
            if q >= 0:
                acc = (acc + da[ri[q]]).astype(np.float32)
        assert np.array_equal(dx[j].view(np.uint32), B.to_format(acc, "bf16").view(np.uint32))
    # weight gradients at sampled elements: experts 0 (hottest), a middle one, the last
    for e in sorted({0, cfg.L // 2, cfg.L - 1}):
        lo, n = int(offsets[e]), int(counts[e])
        sl = slice(lo, lo + n)
        for (mat, bsrc, asrc, N, K) in ((layer.dw2, layer.d_out, layer.z, cfg.H, cfg.I),
                                        (layer.dw13, layer.dg, layer.buf, 2 * cfg.I, cfg.H)):
            ns = rng.choice(N, 4, replace=False)
            ks = rng.choice(K, 4, replace=False)
            bcols = host_vals(bsrc[sl][:, torch.tensor(ns, device="cuda")]).astype(np.float64)
            acols = host_vals(asrc[sl][:, torch.tensor(ks, device="cuda")]).astype(np.float64)
            ref = bcols.T @ acols                                    # [4, 4]
            got = mat[e][torch.tensor(ns, device="cuda")][:, torch.tensor(ks, device="cuda")].cpu().numpy()
            if n == 0:
                assert not np.any(got)
            else:
                # fp32 sums over up to ~15k rows of exact products against float64
                assert np.max(np.abs(got - ref)) <= 1e-4 * max(1.0, np.max(np.abs(ref))), (e, n)
    assert torch.isfinite(layer.dw13).all() and torch.isfinite(layer.dw2).all()
    print(f"[metric] backward full skewed_bf16: {len(tokens)} tokens, {len(rows)} rows checked", flush=True)


@pytest.mark.parametrize("saved_g", [False, True])
def test_backward_hip_graph_replay(ep, saved_g):
    """Forward + backward captured once in a HIP graph; replayed with new
    upstream gradients copied into the captured dy, eager work and syncs in
    between.  Every replay must equal the eager result bit for bit (dx, d_w,
    dW2, dW13)."""
    from combine_top_expert_amd.pipeline import MoELayer
    announce("backward hip graph", f"saved_g={saved_g}")
    cfg = get_config("skewed_bf16_small")
    wl = make_workload(cfg)
    layer = MoELayer(layer_shape(cfg), fused=not saved_g)
    upload_weights(layer, wl)
    x, ids, w = dev(wl.x, "bf16"), dev(wl.ids), dev(wl.weights)
    dy = torch.zeros(cfg.T, cfg.H, device="cuda", dtype=torch.bfloat16)

    def step():
        layer.forward(x, ids, w)
        layer.backward(dy, w)

    step()                                         # allocations and transposes outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    outs = lambda: [t.clone() for t in (layer.dx, layer.d_w, layer.dw2, layer.dw13)]
    for rep in range(3):
        dy.copy_(torch.randn(cfg.T, cfg.H, device="cuda", generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs()
        step()
        torch.cuda.synchronize()
        ref = outs()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
        assert torch.isfinite(ref[3]).all() and ref[3].abs().sum() > 0


@pytest.mark.parametrize("H", [512, 4608])
def test_combine_backward_direct(ep, H):
    """moe_combine_backward on its own, all bf16: H = 512 takes the
    register-cached kernel, H = 4608 the general one.  Non-local routes
    (slot -1) and padding rows; d_out bit-exact, d_w within 1e-5."""
    announce("combine backward", f"H={H}")
    rng = np.random.default_rng(H)
    T, K, rows_cap = 96, 6, 640
    slot_of = np.full((T, K), -1, np.int32)
    perm = rng.permutation(rows_cap)[: T * K].reshape(T, K)
    keep = rng.random((T, K)) < 0.7
    slot_of[keep] = perm[keep]
    weights = rng.random((T, K)).astype(np.float32)
    dy = B.to_format(rng.standard_normal((T, H)).astype(np.float32), "bf16")
    out = B.to_format(rng.standard_normal((rows_cap, H)).astype(np.float32), "bf16")
    rows = sorted(int(q) for q in slot_of[slot_of >= 0])
    d_out_ref, d_w_ref = B.combine_backward(dy, {q: out[q] for q in rows}, slot_of, weights, "bf16")
    bf = torch.bfloat16
    d_out = torch.full((rows_cap, H), float("nan"), device="cuda", dtype=bf)
    d_w = torch.full((T, K), 7.0, device="cuda")
    ep.moe_combine_backward(torch.from_numpy(dy).cuda().to(bf), torch.from_numpy(out).cuda().to(bf),
                            dev(slot_of), dev(weights), d_out, d_w)
    torch.cuda.synchronize()
    got = host_vals(d_out)
    assert np.array_equal(np.stack([got[q] for q in rows]).view(np.uint32),
                          np.stack([d_out_ref[q] for q in rows]).view(np.uint32))
    untouched = np.setdiff1d(np.arange(rows_cap), rows)
    assert np.isnan(got[untouched]).all()
    dw = d_w.cpu().numpy()
    assert np.all(dw[slot_of < 0] == 0)
    assert rel_l2(dw, d_w_ref) < 1e-5


@pytest.mark.parametrize("name", ["skewed_bf16_small", "manyrow_fp32_small", "ksplit_bf16"])
def test_fused_silu_backward_matches_separate(ep, name):
    """moe_grouped_gemm_w13_silu_backward (G recomputed, dG in the GEMM's
    epilogue) against MOE_EPI_STORE_G followed by moe_silu_mul_backward on
    the same inputs: every gradient bit-identical.  ksplit_bf16 splits the
    gate/up GEMM's last round along K, so the piece reduce's epilogue runs."""
    from combine_top_expert_amd.pipeline import MoELayer
    from test_gpu_gemm_combine import gemm_grid, k_split_plan
    announce("fused SiLU*up backward", name)
    cfg = (get_config("skewed_bf16_small").scaled(name="ksplit_bf16", T=128, E=8, L=8, H=2048, I=512, R=512)
           if name == "ksplit_bf16" else get_config(name))
    wl = make_workload(cfg)
    layer = MoELayer(layer_shape(cfg))
    upload_weights(layer, wl)
    bf = cfg.act == "bf16"
    x, w = dev(wl.x, "bf16" if bf else None), dev(wl.weights)
    layer.forward(x, dev(wl.ids), w)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(23)
    dy = torch.randn(cfg.T, cfg.H, device="cuda", generator=gen).to(layer.out.dtype)
    if name == "ksplit_bf16":
        mts = int(sum(-(-int(c) // 128) for c in layer.counts.cpu().numpy()))
        nb = cfg.I // 128
        plan = k_split_plan(mts * nb, gemm_grid(cfg.rows_cap, cfg.L, nb), cfg.H * 2 // 128)
        assert max(S for _, _, S in plan) > 1, plan
    names = [n for n, _ in layer.backward_stages(dy, w)]
    assert "gemm_g_silu_bw" in names and "silu_mul_bw" not in names
    layer.backward(dy, w)
    fused = {k: getattr(layer, k).clone() for k in ("dg", "da", "dx", "d_w", "dw2", "dw13")}
    names = [n for n, _ in layer.backward_stages(dy, w, fuse_silu=False)]
    assert "gemm_g" in names and "silu_mul_bw" in names
    layer.backward(dy, w, fuse_silu=False)
    torch.cuda.synchronize()
    for k, v in fused.items():
        assert torch.equal(v, getattr(layer, k)), f"{name} {k}: fused and separate backward differ"
    assert torch.isfinite(layer.dw13).all() and layer.dg.float().abs().sum() > 0
