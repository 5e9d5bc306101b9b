"""bench.py's algorithmic byte counts pinned by the byte facts of "SGLang、NCCL
与 MoE EP" §2.3.7 / §5.3 (tests/golden/byte_accounting.json): at H = 4096 a
bf16 route row is 8192 bytes and the 112-token top-2 routing moves 224 rows
= 1.75 MiB; rank 0 (experts 0..3) holds 112 valid rows = 896 KiB; the
capacity areas [2, 256, 4096] are 4 MiB in bf16, 2 MiB in FP8 plus 64 KiB of
fp32 scales, i.e. 8192, 4096 and 128 bytes per row.  Every reported GB/s and
roofline fraction rests on these counts."""
from types import SimpleNamespace

import pytest

import numpy as np

import bench

# the worked routing: token 5 -> (E1, E6), every other token -> (E0, E7)
COUNTS = np.array([111, 1, 0, 0, 0, 0, 1, 111])


def _cfg(H, dt, T=112, K=2):
    return SimpleNamespace(H=H, I=128, T=T, K=K, wdt=dt, buf_dt=dt, z_dt=dt, out_dt="bf16", act="bf16")


def test_route_and_share_bytes(gold):
    g = gold("byte_accounting.json")
    H = g["H"]
    w = bench.algorithmic_work(_cfg(H, "bf16"), COUNTS, tok_local=112)
    assert w["rows"] == g["routes"] == 224
    assert w["a_bytes"] == g["route_bytes"] == 224 * g["bytes_per_bf16_row"]
    assert w["a_bytes"] / 2 ** 20 == g["route_MiB"]
    r0 = bench.algorithmic_work(_cfg(H, "bf16"), COUNTS[:4], tok_local=112)
    assert r0["rows"] == g["rank0_valid_rows"]
    assert r0["a_bytes"] == g["rank0_valid_KiB"] * 1024


def test_per_row_bytes_match_the_capacity_areas(gold):
    g = gold("byte_accounting.json")
    H = g["H"]
    L, M, _ = g["recv_bf16_shape"]
    area_rows = L * M
    one = np.array([1])
    bf16 = bench.algorithmic_work(_cfg(H, "bf16"), one)["a_bytes"]
    fp8 = bench.algorithmic_work(_cfg(H, "fp8"), one)["a_bytes"]
    assert bf16 * area_rows == g["recv_bf16_MiB"] * 2 ** 20
    assert fp8 * area_rows == g["recv_fp8_MiB"] * 2 ** 20 + g["scales_KiB"] * 1024


def test_permute_and_combine_move_the_valid_rows():
    """Permute reads each token with a local route once and writes its rows;
    combine reads every row and writes every token; routing metadata: ids
    (4 B) for permute, slots and weights (8 B) for combine."""
    H, T, K = 4096, 112, 2
    w = bench.algorithmic_work(_cfg(H, "bf16", T, K), COUNTS, tok_local=112)
    assert w["permute_bytes"] == 112 * H * 2 + 224 * H * 2 + T * K * 4
    assert w["combine_bytes"] == 224 * H * 2 + T * H * 2 + T * K * 8
    # the GEMMs: weights of active experts once, valid rows once
    active = 4
    assert w["w13_bytes"] == active * 256 * H * 2 + 224 * H * 2 + 224 * 128 * 2
    assert w["w13_flops"] == 2 * 224 * H * 256
    assert w["gemm_flops"] == 6 * H * 128 * 224


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    """bench.py measures one GPU's share: --gpus N > 1 exits with status 2 and
    says why, before touching a GPU."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
