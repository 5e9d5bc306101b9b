"""moe_dispatch_layout_noalloc (the library's per-device scratch in place of
a caller workspace) against moe_dispatch_layout, through the C ABI: two
calls in a row, the second with a smaller input, each bit-exact to the
workspace entry point on the same routing."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev, need_gpu
from oracle import moe
from workloads import get_config, make_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


def _outputs(T, K, L, R):
    rc = L * R if R > 0 else T * K
    i32 = dict(dtype=torch.int32, device="cuda")
    return {"counts": torch.full((L,), -7, **i32), "offsets": torch.full((L + 1,), -7, **i32),
            "slot_of": torch.full((T, K), -7, **i32), "row_src": torch.full((rc,), -7, **i32),
            "tile_offsets": torch.full((L + 1,), -7, **i32), "dev_status": torch.full((2,), -7, **i32)}


def _run(ep, ids, cfg, noalloc):
    T, K = ids.shape
    o = _outputs(T, K, cfg.L, cfg.R)
    args = (dev(ids), cfg.E, cfg.expert_begin, cfg.L, cfg.R, 128, o["counts"], o["offsets"], o["slot_of"],
            o["row_src"], o["tile_offsets"], o["dev_status"])
    if noalloc:
        ep.moe_dispatch_layout_noalloc(*args)
    else:
        ws = torch.zeros(ep.moe_dispatch_layout_workspace_bytes(T, K, cfg.L), dtype=torch.uint8,
                         device="cuda")
        ep.moe_dispatch_layout(*args, ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


@pytest.mark.parametrize("first,second", [("skewed_bf16", "prefill_fp8"), ("prefill_fp8", "decode_fp8")])
def test_noalloc_layout_matches_workspace_layout(ep, first, second):
    for name in (first, second):
        announce("layout noalloc", name)
        cfg = get_config(name)
        ids, _ = make_routing(cfg)
        a = _run(ep, ids, cfg, noalloc=True)
        b = _run(ep, ids, cfg, noalloc=False)
        for k in a:
            assert np.array_equal(a[k], b[k]), (name, k)
        ref = moe.dispatch_layout(ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
        assert np.array_equal(a["slot_of"], ref["slot_of"])
        assert np.array_equal(a["counts"], ref["counts"])


def test_noalloc_rejects_oversize(ep):
    announce("layout noalloc oversize")
    T, K, L = 1 << 20, 8, 1024
    assert ep.moe_dispatch_layout_workspace_bytes(T, K, L) > ep.moe_dispatch_layout_noalloc_max_bytes()
    ids = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    o = _outputs(T, K, L, 0)
    with pytest.raises(ep.MoEError, match="WORKSPACE"):
        ep.moe_dispatch_layout_noalloc(ids, 1024, 0, L, 0, 128, o["counts"], o["offsets"], o["slot_of"],
                                       o["row_src"], o["tile_offsets"], o["dev_status"])
