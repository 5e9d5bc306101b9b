"""GPU parity at the full sizes, in the launch configuration the benchmark
times (fused gate/up epilogue, packed gate/up weights, GEMM workspace so the
last round splits along K).

prefill_fp8 (8192 tokens, top-8 of 256, 32 local experts, H=7168, I=2048,
block-FP8) and decode_fp8 compare every token and every routed row:
layout and permute bit-exact, every G element (from a second gate/up launch
with the stored-G epilogue), every FP8 Z code and scale, every expert-output
element and combine, with the bars of gpu_util.check_layer.  skewed_bf16
(16384 tokens, 64 experts, 98304 rows) compares the tokens that own the
first and last 16 rows of every expert's first and last 128-row tile, plus
512 random tokens, and every row those tokens route to."""
import numpy as np
import pytest
import torch

from gpu_util import announce, check_layer, dev, host_bits, layer_shape, need_gpu, upload_weights
from oracle import moe
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


def run_bench_config(ep, wl):
    from combine_top_expert_amd.pipeline import MoELayer
    cfg = wl.cfg
    layer = MoELayer(layer_shape(cfg), fused=True)
    upload_weights(layer, wl)
    layer.forward(dev(wl.x, "bf16" if cfg.act == "bf16" else None), dev(wl.ids), dev(wl.weights))
    torch.cuda.synchronize()
    st = layer.dev_status.cpu().numpy()
    assert st[0] == 0 and st[1] == 0, f"device status {st}"
    # G from the same kernel configuration with the stored-G epilogue
    g = torch.full((cfg.rows_cap, 2 * cfg.I), float("nan"), dtype=torch.float32, device="cuda")
    w, lay = ((layer.w13_packed, ep.MOE_W_PACKED) if layer.w13_packed is not None
              else (layer.w13, ep.MOE_W_ROW_MAJOR))
    ep.moe_grouped_gemm_w13(layer.buf, layer.buf_scales, w, layer.w13_scales, layer.counts,
                            layer.offsets, ep.MOE_EPI_STORE_G, g, workspace=layer.gemm_workspace,
                            w13_layout=lay)
    torch.cuda.synchronize()
    return layer, g


def check_permute(layer, wl, rows):
    cfg = wl.cfg
    lay = moe.dispatch_layout(wl.ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    for k in ("counts", "offsets"):
        assert np.array_equal(getattr(layer, k).cpu().numpy(), lay[k]), k
    perm = moe.permute(wl.x, cfg.act, lay["row_src"], cfg.K, cfg.buf_dt, rows)
    got = host_bits(layer.buf)[perm["rows"]]
    assert np.array_equal(got, perm["data"]), "permuted rows differ"
    if cfg.buf_dt == "fp8":
        sc = layer.buf_scales.cpu().numpy()[perm["rows"]]
        assert np.array_equal(sc.view(np.uint32), perm["scales"].view(np.uint32)), "FP8 scales differ"


@pytest.mark.parametrize("name", ["decode_fp8", "prefill_fp8"])
def test_full_size_every_token(ep, name):
    announce("full size, every token", name)
    wl = make_workload(name)
    layer, g = run_bench_config(ep, wl)
    lay_rows = np.nonzero(layer.row_src.cpu().numpy() >= 0)[0]
    check_permute(layer, wl, lay_rows)
    m = check_layer(wl, layer, ew=moe.ExpertWeights(wl.cfg, wl.w), tag=f"{name} full", g=g)
    assert m["tokens"] == wl.cfg.T


def skewed_tokens(wl, layer, n_random=512, seed=2024):
    cfg = wl.cfg
    counts = layer.counts.cpu().numpy()
    offsets = layer.offsets.cpu().numpy()
    row_src = layer.row_src.cpu().numpy()
    pick = []
    for e in range(cfg.L):
        c, o = int(counts[e]), int(offsets[e])
        if c == 0:
            continue
        last = (c - 1) // 128 * 128
        for t0 in (0, last):
            for r in list(range(t0, min(t0 + 16, c))) + list(range(max(t0, min(t0 + 128, c) - 16), min(t0 + 128, c))):
                pick.append(row_src[o + r] // cfg.K)
    rng = np.random.default_rng(seed)
    pick += list(rng.choice(cfg.T, n_random, replace=False))
    return np.unique(np.asarray(pick, np.int64))


def test_full_size_skewed_sampled(ep):
    announce("full size, sampled tokens", "skewed_bf16")
    wl = make_workload("skewed_bf16")
    layer, g = run_bench_config(ep, wl)
    tokens = skewed_tokens(wl, layer)
    slot = layer.slot_of.cpu().numpy()
    rows = np.unique(slot[tokens].ravel())
    rows = rows[rows >= 0]
    check_permute(layer, wl, rows)
    m = check_layer(wl, layer, tokens=tokens, ew=moe.ExpertWeights(wl.cfg, wl.w), tag="skewed_bf16 sampled",
                    g=g)
    assert m["tokens"] == len(tokens)
