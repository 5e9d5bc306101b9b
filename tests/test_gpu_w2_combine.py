"""GPU parity of moe_grouped_gemm_w2_combine, the down GEMM with the combine
folded into its epilogue (fp32 atomic adds of w * out into the token sums).

Its sums run in arrival order and skip the bf16 rounding of the expert
outputs, so it is compared by the layer bars against the oracle (rel-L2 and
max|dy|/RMS as in gpu_util.check_layer) and against the unfused path's y
(relative L2 <= 5e-3: the unfused path rounds every expert output to bf16
before the weighted sum).  Tokens without a local route must be 0."""
import numpy as np
import pytest
import torch

from gpu_util import (FLOOR_FACTOR, LAYER_MAXABS, LAYER_REL_L2, announce, dev, host_vals, layer_shape,
                      need_gpu, upload_weights)
import parity_bounds as PB
from oracle import moe
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


@pytest.mark.parametrize("name", ["toy_fp32", "toy_bf16_fp8w", "decode_fp8_small", "prefill_fp8_small",
                                  "skewed_bf16_small", "manyrow_fp8_small", "decode_fp8", "prefill_fp8"])
def test_w2_combine_matches_oracle(ep, name):
    from combine_top_expert_amd.pipeline import MoELayer
    announce("w2_combine", name)
    wl = make_workload(name)
    cfg = wl.cfg
    layer = MoELayer(layer_shape(cfg), fused=True)
    upload_weights(layer, wl)
    w = dev(wl.weights)
    layer.forward(dev(wl.x, "bf16" if cfg.act == "bf16" else None), dev(wl.ids), w)
    y_acc = torch.empty(cfg.T, cfg.H, dtype=torch.float32, device="cuda")
    y2 = torch.full_like(layer.y, float("nan"))
    for _ in range(2):           # a second call must not accumulate onto the first
        ep.moe_grouped_gemm_w2_combine(layer.z, layer.z_scales, layer.w2, layer.w2_scales, layer.counts,
                                       layer.offsets, layer.row_src, w, y_acc, y2)
    torch.cuda.synchronize()
    got = host_vals(y2)
    std = host_vals(layer.y)
    ew = moe.ExpertWeights(cfg, wl.w)
    ref = moe.moe_layer(wl, ew=ew)["y"]
    floor = PB.maxabs_over_rms(moe.moe_layer(wl, ew=ew, acc="f32")["y"], ref)
    m = {"rel_l2": PB.rel_l2(got, ref), "maxabs_rms": PB.maxabs_over_rms(got, ref), "floor": floor,
         "rel_l2_vs_unfused": PB.rel_l2(got, std)}
    print(f"[metric] w2_combine {name} " + " ".join(f"{k}={v:.3e}" for k, v in m.items()), flush=True)
    assert np.all(np.isfinite(got))
    no_route = ~(layer.slot_of.cpu().numpy() >= 0).any(axis=1)
    assert np.all(got[no_route] == 0)
    assert m["rel_l2"] <= LAYER_REL_L2
    assert m["maxabs_rms"] <= max(LAYER_MAXABS, FLOOR_FACTOR * floor)
    assert m["rel_l2_vs_unfused"] <= 5e-3
