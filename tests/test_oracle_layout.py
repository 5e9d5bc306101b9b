"""Pins for the oracle's dispatch layout (CPU only).

Checked against the worked routing of "SGLang、NCCL 与 MoE EP" (counts,
replay, the E1 row q), the tile and fill tables of "SGLang Expert Compute
Backend" §2.4/§4.3/§5.3, the compact-storage map of §4.1, closed forms for
the slot of every token of the worked routing, and invariants on random
routings (bijection, inverse, histogram, monotone offsets)."""
import math

import numpy as np
import pytest

from oracle import moe
from workloads import get_config, make_routing


def token5_ids(T=112, to=(1, 6)):
    ids = np.tile(np.array([0, 7], np.int32), (T, 1))
    ids[5] = to
    return ids


def test_token5_counts(gold):
    g = gold("token5_routing.json")
    ids = token5_ids(g["T"])
    lay = moe.dispatch_layout(ids, g["E"], 0, 8, 128)
    assert lay["counts"].tolist() == g["counts_by_global_expert"]
    assert int(lay["counts"].sum()) == g["routes"] == g["T"] * g["K"]
    # per-rank view: L=2 experts per rank, rank r owns [2r, 2r+2)
    lay0 = moe.dispatch_layout(ids, 8, 0, 2, 128)
    lay3 = moe.dispatch_layout(ids, 8, 6, 2, 128)
    assert lay0["counts"].tolist() == g["per_rank_counts"]["rank0"]
    assert lay3["counts"].tolist() == g["per_rank_counts"]["rank3"]
    assert lay["flags"] == 0 and lay["dropped"] == 0


def test_token5_replay_counts(gold):
    g = gold("token5_routing.json")
    ids = token5_ids(g["T"], to=tuple(g["replay_token5_to"]))
    c = moe.dispatch_layout(ids, 8, 0, 8, 128)["counts"]
    assert [c[0], c[1], c[6], c[7]] == g["replay_counts_E0_E1_E6_E7"]


def test_token5_slots_closed_form():
    """Stable (t, k) order: E0's slot of token t is t for t < 5 and t-1 for
    t > 5; E7 likewise at 7*R; E1 and E6 hold only token 5 at slot 0."""
    R = 128
    lay = moe.dispatch_layout(token5_ids(), 8, 0, 8, R)
    so = lay["slot_of"]
    for t in range(112):
        if t == 5:
            assert so[t].tolist() == [1 * R + 0, 6 * R + 0]
        else:
            s = t if t < 5 else t - 1
            assert so[t].tolist() == [0 * R + s, 7 * R + s]
    assert lay["row_src"][128] == 5 * 2 + 0 and lay["row_src"][768] == 5 * 2 + 1


def test_expert_row_q(gold):
    """E1's single row lands at q = e*M + s = 256 for M = W*C = 256."""
    g = gold("expert_row_q.json")
    M = g["W"] * g["C"]
    assert M == g["M"]
    ids = token5_ids()
    lay = moe.dispatch_layout(ids, 8, 0, g["L"], M)    # rank 0 owns E0, E1
    assert lay["counts"].tolist() == [g["E0_count"], g["E1_count"]]
    assert lay["slot_of"][5, 0] == g["E1_row_q"] != g["not_q"]


def test_tile_counts_70_12(gold):
    g = gold("grouped_gemm_70_12.json")
    counts = g["counts"]
    n_blocks = math.ceil(2 * g["I"] / g["BN"])
    m_tiles = moe.m_tile_count(counts, 64)
    assert m_tiles * n_blocks == len(g["tiles_BM64"]) == 6
    # tile_offsets from the layout agree
    ids = np.full((82, 1), -1, np.int32)
    ids[:70, 0] = 0
    ids[70:, 0] = 1
    lay = moe.dispatch_layout(ids, 2, 0, 2, g["R"], BM=64)
    assert lay["counts"].tolist() == counts
    assert lay["tile_offsets"].tolist() == [0, 2, 3]
    assert g["H"] // g["BK"] == g["k_rounds_gate_up"]
    for row in g["bm_sweep"]:
        mb = moe.m_tile_count(counts, row["BM"])
        assert mb == row["m_blocks"]
        assert mb * row["BM"] == row["covered_rows"]
        assert round(100 * sum(counts) / (mb * row["BM"]), 1) == row["fill_pct"]
        assert mb * n_blocks == row["dot_tiles"]
    sp = g["split_35_6"]
    mb = 2 * moe.m_tile_count([35, 6], 64)
    assert mb == sp["m_blocks_BM64"] and mb * 64 == sp["covered_rows"]
    assert round(100 * sum(counts) / (mb * 64), 1) == sp["fill_pct"]


def test_compact_offsets(gold):
    g = gold("compact_rows.json")
    ids = np.zeros((82, 1), np.int32)
    ids[70:] = 1
    cap = moe.dispatch_layout(ids, 2, 0, 2, g["R"])
    fit = moe.dispatch_layout(ids, 2, 0, 2, 0)
    assert fit["offsets"].tolist() == [0, 70, 82]
    old_to_new = {int(cap["slot_of"][t, 0]): int(fit["slot_of"][t, 0]) for t in range(82)}
    for m in g["map"]:
        for o, n in zip(range(m["old_q"][0], m["old_q"][1] + 1),
                        range(m["compact"][0], m["compact"][1] + 1)):
            assert old_to_new[o] == n
    assert old_to_new[130] == g["old_q_130_compact"]


def check_invariants(ids, E, e0, L, R, lay):
    T, K = ids.shape
    counts, offsets, so, rs = lay["counts"], lay["offsets"], lay["slot_of"], lay["row_src"]
    local = (ids >= e0) & (ids < e0 + L)
    true = np.bincount(ids[local] - e0, minlength=L)
    assert np.array_equal(counts, np.minimum(true, R) if R else true)
    assert np.all(np.diff(offsets) >= 0)
    if R:
        assert offsets.tolist() == [e * R for e in range(L + 1)]
        assert len(rs) == L * R
    else:
        assert offsets[-1] == counts.sum() and len(rs) == T * K
    # slot_of is a bijection onto the valid rows; row_src is its inverse
    placed = so[so >= 0]
    assert len(np.unique(placed)) == len(placed) == counts.sum()
    valid = moe.valid_rows(counts, offsets)
    assert np.array_equal(np.sort(placed), valid)
    for t, k in zip(*np.nonzero(so >= 0)):
        q = so[t, k]
        assert rs[q] == t * K + k
        e = ids[t, k] - e0
        assert offsets[e] <= q < offsets[e] + counts[e]
    pad = np.ones(len(rs), bool)
    pad[valid] = False
    assert np.all(rs[pad] == -1)
    # non-local and invalid routes have no slot
    assert np.all(so[~local] == -1)
    # stable order within each expert: rows increase with t*K + k
    for e in range(L):
        seg = rs[offsets[e]:offsets[e] + counts[e]]
        assert np.all(np.diff(seg) > 0)


@pytest.mark.parametrize("seed", range(5))
def test_random_routing_invariants(seed):
    rng = np.random.default_rng(seed)
    T, K, E = 300, 4, 16
    ids = rng.integers(-1, E, (T, K)).astype(np.int32)
    for e0, L, R in [(0, 16, 128), (4, 8, 0), (8, 8, 100), (0, 16, 0)]:
        lay = moe.dispatch_layout(ids, E, e0, L, R)
        assert lay["flags"] == 0
        check_invariants(ids, E, e0, L, R, lay)


@pytest.mark.parametrize("name", ["decode_fp8", "prefill_fp8", "skewed_bf16_small"])
def test_config_routing_invariants(name):
    cfg = get_config(name)
    ids, w = make_routing(cfg)
    lay = moe.dispatch_layout(ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    assert lay["flags"] == 0, "capacity must cover the seeded routing"
    check_invariants(ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R, lay)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_capacity_overflow_flags_and_drops_tail_routes():
    ids = token5_ids()
    lay = moe.dispatch_layout(ids, 8, 0, 8, 64)
    assert lay["flags"] & moe.FLAG_CAPACITY
    assert lay["counts"].tolist() == [64, 1, 0, 0, 0, 0, 1, 64]
    assert lay["dropped"] == 2 * (111 - 64)
    # the first 64 routes (in t order) are kept, later ones get slot -1
    kept = [t for t in range(112) if t != 5][:64]
    assert all(lay["slot_of"][t, 0] >= 0 for t in kept)
    assert all(lay["slot_of"][t, 0] == -1 for t in range(112) if t != 5 and t not in kept)
    assert lay["row_src"].max() < 112 * 2 and len(lay["row_src"]) == 8 * 64


def test_bad_and_empty_ids():
    ids = np.array([[0, -1], [9, 1], [-5, 2], [-1, -1]], np.int32)
    lay = moe.dispatch_layout(ids, 8, 0, 8, 4)
    assert lay["flags"] == moe.FLAG_BAD_EXPERT_ID
    assert lay["counts"].tolist() == [1, 1, 1, 0, 0, 0, 0, 0]
    assert lay["slot_of"].tolist() == [[0, -1], [-1, 4], [-1, 8], [-1, -1]]
    # zero tokens
    lay = moe.dispatch_layout(np.zeros((0, 3), np.int32), 8, 0, 8, 4)
    assert lay["counts"].sum() == 0 and np.all(lay["row_src"] == -1)
    lay = moe.dispatch_layout(np.zeros((0, 3), np.int32), 8, 0, 8, 0)
    assert len(lay["row_src"]) == 0 and lay["offsets"].tolist() == [0] * 9


def test_duplicate_expert_in_one_token_gets_two_rows():
    ids = np.array([[3, 3], [3, 1]], np.int32)
    lay = moe.dispatch_layout(ids, 4, 0, 4, 0)
    assert lay["counts"].tolist() == [0, 1, 0, 3]
    assert lay["slot_of"].tolist() == [[1, 2], [3, 0]]
