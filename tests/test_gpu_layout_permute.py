"""GPU parity: moe_dispatch_layout and moe_permute against the oracle.

Integer and byte outputs must match bit for bit: counts, offsets, slot_of,
row_src, tile_offsets, status flags, permuted rows, FP8 codes and scales."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev, host_bits, layer_shape, need_gpu
from oracle import formats as F
from oracle import moe
from workloads import get_config, make_activations, make_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


def run_layout(ep, ids: np.ndarray, E, e0, L, R, BM=128):
    T, K = ids.shape
    rc = L * R if R > 0 else T * K
    i32 = dict(dtype=torch.int32, device="cuda")
    out = {
        "counts": torch.full((L,), -7, **i32), "offsets": torch.full((L + 1,), -7, **i32),
        "slot_of": torch.full((T, K), -7, **i32), "row_src": torch.full((max(rc, 1),), -7, **i32)[:rc],
        "tile_offsets": torch.full((L + 1,), -7, **i32), "dev_status": torch.full((2,), -7, **i32),
    }
    ws = torch.zeros(max(ep.moe_dispatch_layout_workspace_bytes(T, K, L), 4), dtype=torch.uint8,
                     device="cuda")
    tids = dev(ids.astype(np.int32)) if T * K else torch.zeros((T, K), **i32)
    ep.moe_dispatch_layout(tids, E, e0, L, R, BM, out["counts"], out["offsets"], out["slot_of"],
                           out["row_src"], out["tile_offsets"], out["dev_status"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_layout(got, ref):
    for k in ("counts", "offsets", "slot_of", "row_src", "tile_offsets"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["dev_status"][0] == ref["flags"]
    assert got["dev_status"][1] == ref["dropped"]


@pytest.mark.parametrize("name", ["toy_fp32", "decode_fp8", "prefill_fp8", "skewed_bf16",
                                  "prefill_fp8_small", "skewed_bf16_small"])
def test_layout_bit_exact(ep, name):
    cfg = get_config(name)
    announce("layout", name)
    ids, _ = make_routing(cfg)
    ref = moe.dispatch_layout(ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    check_layout(run_layout(ep, ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R), ref)


# The launch shape depends on T*K and L: one launch while T*K <= 1024
# (all_invalid, overflow, single_*), two while ceil(T*K/1024) * L <= 16384,
# three beyond (large_table).
@pytest.mark.parametrize("case", ["empty", "all_invalid", "bad_ids", "overflow", "duplicates",
                                  "many_experts", "exact_fit_random", "ragged", "bm64",
                                  "single_many_experts", "single_exact_fit", "large_table"])
def test_layout_edge_cases(ep, case):
    announce("layout edge", case)
    rng = np.random.default_rng(3)
    E, e0, L, R, BM = 8, 0, 8, 128, 128
    if case == "empty":
        ids = np.zeros((0, 4), np.int32)
    elif case == "all_invalid":
        ids = np.full((300, 2), -1, np.int32)
    elif case == "bad_ids":
        ids = rng.integers(-3, 11, (500, 3)).astype(np.int32)
    elif case == "overflow":                      # the worked routing with R = 64
        ids = np.tile(np.array([0, 7], np.int32), (112, 1))
        ids[5] = [1, 6]
        R = 64
    elif case == "duplicates":
        ids = rng.integers(0, 3, (777, 4)).astype(np.int32)
    elif case == "many_experts":                  # L > 64 takes the ordered-chunk path
        E, e0, L, R = 512, 100, 300, 40
        ids = rng.integers(-1, E, (3000, 8)).astype(np.int32)
    elif case == "exact_fit_random":
        E, e0, L, R = 64, 16, 32, 0
        ids = rng.integers(-1, E, (5000, 6)).astype(np.int32)
    elif case == "ragged":                        # T*K not a multiple of the block size
        E, e0, L, R = 32, 0, 32, 96
        ids = rng.integers(0, E, (1025, 3)).astype(np.int32)
    elif case == "single_many_experts":           # one block, L > 64 ordered-chunk path
        E, e0, L, R = 512, 100, 300, 6
        ids = rng.integers(-1, E, (120, 8)).astype(np.int32)
    elif case == "single_exact_fit":              # one block, offsets from the scan
        E, e0, L, R = 64, 16, 32, 0
        ids = rng.integers(-1, E, (150, 6)).astype(np.int32)
    elif case == "large_table":                   # 20 blocks x 1024 experts: separate scan launch
        E, e0, L, R = 2048, 512, 1024, 12
        ids = rng.integers(-1, E, (4000, 5)).astype(np.int32)
    else:
        E, e0, L, R, BM = 16, 4, 8, 200, 64
        ids = rng.integers(-1, E, (999, 5)).astype(np.int32)
    ref = moe.dispatch_layout(ids, E, e0, L, R, BM)
    check_layout(run_layout(ep, ids, E, e0, L, R, BM), ref)


def test_layout_replay_same_buffers(ep):
    """Same device buffers, token 5 rerouted to (E0, E7): counts become
    112/0/0/112 and every stale slot is rewritten."""
    announce("layout replay")
    cfg = get_config("toy_fp32")
    ids, _ = make_routing(cfg)
    shape = layer_shape(cfg)
    from combine_top_expert_amd.pipeline import MoELayer
    layer = MoELayer(shape)
    for trial in range(2):
        cur = ids.copy()
        if trial == 1:
            cur[5] = [0, 7]
        layer.layout(dev(cur))
        torch.cuda.synchronize()
        ref = moe.dispatch_layout(cur, cfg.E, 0, cfg.L, cfg.R)
        assert np.array_equal(layer.counts.cpu().numpy(), ref["counts"])
        assert np.array_equal(layer.slot_of.cpu().numpy(), ref["slot_of"])
        assert np.array_equal(layer.row_src.cpu().numpy(), ref["row_src"])
    c = layer.counts.cpu().numpy()
    assert [c[0], c[1], c[6], c[7]] == [112, 0, 0, 112]


# ---------------------------------------------------------------- permute

def run_permute(ep, cfg, x, ids):
    from combine_top_expert_amd.pipeline import MoELayer
    layer = MoELayer(layer_shape(cfg))
    # padding rows pre-filled with NaN patterns; they must stay untouched
    if layer.buf.dtype == torch.uint8:
        layer.buf.fill_(0x7F)
    elif layer.buf.dtype == torch.bfloat16:
        layer.buf.view(torch.int16).fill_(-1)
    else:
        layer.buf.fill_(float("nan"))
    if layer.buf_scales is not None:
        layer.buf_scales.fill_(float("nan"))
    layer.layout(dev(ids))
    layer.permute(dev(x, "bf16" if cfg.act == "bf16" else None))
    torch.cuda.synchronize()
    return layer


def _permute_config(name):
    """'<config>@<H>' is <config> with hidden size H: the permute kernels work on
    1024-column (bf16 -> FP8) and 4 KB (copy) parts of a row, so H = 1152 and
    2176 leave a ragged last part after one or two full ones."""
    if "@" not in name:
        return get_config(name)
    base, h = name.split("@")
    return get_config(base).scaled(name=name, H=int(h))


@pytest.mark.parametrize("name", ["toy_fp32", "toy_bf16_fp8w", "decode_fp8", "prefill_fp8",
                                  "skewed_bf16_small", "skewed_bf16", "prefill_fp8_small",
                                  "manyrow_bf16_small", "manyrow_fp8_small", "manyrow_fp32_small",
                                  "prefill_fp8_small@1152", "prefill_fp8_small@2176",
                                  "skewed_bf16_small@1152", "skewed_bf16_small@2176",
                                  "toy_fp32@1152"])
def test_permute_bit_exact(ep, name):
    cfg = _permute_config(name)
    announce("permute", name)
    ids, _ = make_routing(cfg)
    x = make_activations(cfg)
    lay = moe.dispatch_layout(ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    ref = moe.permute(x, cfg.act, lay["row_src"], cfg.K, cfg.buf_dt)
    layer = run_permute(ep, cfg, x, ids)
    got = host_bits(layer.buf)
    rows = ref["rows"]
    if cfg.buf_dt == "f32":
        assert np.array_equal(got[rows].view(np.uint32), ref["data"].view(np.uint32))
    else:
        assert np.array_equal(got[rows], ref["data"])
    if cfg.buf_dt == "fp8":
        sc = layer.buf_scales.cpu().numpy()
        assert np.array_equal(sc[rows].view(np.uint32), ref["scales"].view(np.uint32))
    pad = np.ones(cfg.rows_cap, bool)
    pad[rows] = False
    if cfg.buf_dt == "fp8":
        assert np.all(got[pad] == 0x7F)
        assert np.all(np.isnan(layer.buf_scales.cpu().numpy()[pad]))
    elif cfg.buf_dt == "bf16":
        assert np.all(got[pad] == 0xFFFF)
    else:
        assert np.all(np.isnan(got[pad]))


def test_permute_fp8_encoder_every_bf16_value(ep):
    """Every finite bf16 value v with |v| <= 448, placed in groups whose amax
    is 448 (factor 448/amax = 1), must encode exactly as the oracle's e4m3
    rounding of v; a second pass with amax 3.5 exercises the product."""
    announce("permute fp8 exhaustive")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(bits)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    for amax in (448.0, 3.5):
        vals = v[np.abs(v) <= amax]
        per = 127
        ng = -(-len(vals) // per)
        g = np.zeros((ng, 128), np.float32)
        flat = np.zeros(ng * per, np.float32)
        flat[:len(vals)] = vals
        g[:, :per] = flat.reshape(ng, per)
        g[:, per] = amax
        H = 1024
        rows = -(-ng // (H // 128))
        xs = np.zeros((rows * (H // 128), 128), np.float32)
        xs[:ng] = g
        xs[ng:, 127] = amax
        x = xs.reshape(rows, H)
        xb = F.f32_to_bf16(x)
        assert np.array_equal(F.bf16_to_f32(xb), x)
        ids = np.zeros((rows, 1), np.int32)
        cfg = get_config("toy_bf16_fp8w").scaled(T=rows, K=1, E=1, L=1, H=H, R=rows)
        layer = run_permute(ep, cfg, xb, ids)
        codes_ref, sc_ref = F.quant_fp8_groups(x)
        assert np.array_equal(host_bits(layer.buf), codes_ref)
        assert np.array_equal(layer.buf_scales.cpu().numpy(), sc_ref)
