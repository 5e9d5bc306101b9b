"""Benchmark of one GPU's MoE layer: dispatch layout -> permute (FP8) ->
grouped W13 GEMM with fused SiLU*up -> grouped W2 GEMM -> combine.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_fp8]

A step is one pass of the whole path over one batch of seeded synthetic
input already resident in HBM.  Prints ONE JSON line with the metric,
per-stage times, the dominant kernel's roofline (measured with HIP events on
the stream the kernels run on) and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0, "f32": 157.3}
METRIC = "MoE layer token-expert rows/s + grouped-GEMM TFLOP/s (% MFMA peak), 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="prefill_fp8")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--skip-backward", action="store_true",
                    help="do not time the backward (bf16 / fp32 workloads)")
    ap.add_argument("--skip-cpu-baseline", action="store_true",
                    help="omit the oracle timing (profiling runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    ap.add_argument("--extra-workloads", default="decode_fp8,skewed_bf16",
                    help="comma-separated workloads also timed after the main one (stage and "
                         "kernel times only); empty for none")
    return ap.parse_args()


KERNEL_SOURCES = ["combine_top_expert_amd/csrc/gemm.hip", "combine_top_expert_amd/csrc/moe_common.h"]


def kernel_digest() -> str:
    """sha256 over the grouped-GEMM sources, to tell whether recorded counter
    readings still describe the kernel that is built."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM-side bytes per W13 launch, from the FETCH_SIZE / WRITE_SIZE counter
    runs summarised in profiles/traffic_<workload>.md (each counter scaled by
    its reading for a plain 1 GiB copy).  None when there is no such record
    or it was taken on other kernel sources."""
    import re
    p = ROOT / "profiles" / f"traffic_{workload}.md"
    if not p.exists():
        return None
    kv = dict(re.findall(r"^([a-z0-9_]+): (\S+)$", p.read_text(), re.M))
    if kv.get("kernel_sources_sha256") != kernel_digest():
        return None
    return float(kv["gemm_w13_bytes_per_launch"])


def algorithmic_work(cfg, counts, tok_local=None):
    """Bytes and FLOPs each kernel must move / compute at minimum.

    Weights of experts with at least one row are read once; every valid row
    of A, Z and the expert output is read or written once; padding rows do
    not count ("SGLang、NCCL 与 MoE EP" §2.3.7: the valid rows' bytes, not the
    receive area's, are the traffic).  Permute reads each token with a local
    route once (tok_local of them) and writes its rows; combine reads every
    row and writes every token."""
    rows = int(counts.sum())
    active = int((counts > 0).sum())
    H, I = cfg.H, cfg.I
    wb = {"fp8": 1, "bf16": 2, "f32": 4}[cfg.wdt]
    ab = {"fp8": 1, "bf16": 2, "f32": 4}[cfg.buf_dt]
    zb = {"fp8": 1, "bf16": 2, "f32": 4}[cfg.z_dt]
    ob = {"bf16": 2, "f32": 4}[cfg.out_dt]
    xb = {"bf16": 2, "f32": 4}[cfg.act]
    fp8 = cfg.wdt == "fp8"
    w13 = active * 2 * I * H * wb + (active * (2 * I // 128) * (H // 128) * 4 if fp8 else 0)
    w2 = active * H * I * wb + (active * (H // 128) * (I // 128) * 4 if fp8 else 0)
    a_bytes = rows * H * ab + (rows * (H // 128) * 4 if fp8 else 0)
    z_bytes = rows * I * zb + (rows * (I // 128) * 4 if fp8 else 0)
    out_bytes = rows * H * ob
    work = {
        "rows": rows,
        "a_bytes": a_bytes,
        "w13_bytes": w13 + a_bytes + z_bytes,
        "w13_flops": 2.0 * rows * H * 2 * I,
        "w2_bytes": w2 + z_bytes + out_bytes,
        "w2_flops": 2.0 * rows * I * H,
        "gemm_flops": 6.0 * H * I * rows,
    }
    if tok_local is not None:
        work["permute_bytes"] = tok_local * H * xb + a_bytes + cfg.T * cfg.K * 4
        work["combine_bytes"] = out_bytes + cfg.T * H * ob + cfg.T * cfg.K * 8
    return work


def cpu_baseline(wl, n_tokens):
    """The oracle, as is, on the first n_tokens tokens of the workload."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import moe

    cores = len(os.sched_getaffinity(0))
    tokens = np.arange(min(n_tokens, wl.cfg.T))
    with threadpool_limits(limits=cores):
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        t0 = time.perf_counter()
        res = moe.moe_layer(wl, tokens=tokens, ew=moe.ExpertWeights(wl.cfg, wl.w, cache=False))
        dt = time.perf_counter() - t0
    rows = int((res["layout"]["slot_of"][tokens] >= 0).sum())
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": rows / dt, "unit": "rows/s", "cores": int(blas), "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"first {len(tokens)} of {wl.cfg.T} tokens ({rows} routed rows) of the same "
                      f"workload through the whole numpy oracle (layout, FP8 permute, per-expert "
                      f"weight dequantisation, fp64 GEMMs, combine); {dt:.1f} s"}


def router_timing(cfg, steps, dev):
    """moe_router_topk on the workload's router inputs, timed on its own (it
    produces the routing the step starts from, so it is not part of a step).
    Bytes: logits read + bias read + ids and weights written."""
    import torch

    import combine_top_expert_amd as ep
    from workloads import make_router_inputs

    logits, bias = make_router_inputs(cfg)
    lg = torch.from_numpy(logits).to(dev)
    b = None if bias is None else torch.from_numpy(bias).to(dev)
    ids = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device=dev)
    for _ in range(3):
        ep.moe_router_topk(lg, cfg.K, ids, w, bias=b)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(steps, 10)
    e0.record(stream)
    for _ in range(n):
        ep.moe_router_topk(lg, cfg.K, ids, w, bias=b)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    nbytes = cfg.T * cfg.E * 4 + cfg.E * 4 + cfg.T * cfg.K * 8
    res = {"us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
           "shape": {"T": cfg.T, "E": cfg.E, "K": cfg.K, "bias": cfg.bias}}
    return res


def _time_stages(stages, steps, dev):
    """Median microseconds of each (name, launch) stage over ``steps`` passes,
    an event between stages, and the median of the pass totals."""
    import torch

    for _ in range(3):
        for _, f in stages:
            f()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        ev[s][0].record(stream)
        for i, (_, f) in enumerate(stages):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(stages))]
                    for s in range(steps)]) * 1e3
    return ({name: float(np.median(per[:, i])) for i, (name, _) in enumerate(stages)},
            float(np.median(per.sum(axis=1))),
            {name: [float(np.percentile(per[:, i], 10)), float(np.percentile(per[:, i], 90))]
             for i, (name, _) in enumerate(stages)})


def backward_timing(cfg, layer, x, ids, w, steps, dev):
    """The layer's backward (bf16 / fp32 weights), each stage timed with
    events around it over ``steps`` passes (medians), in two settings:
    after the fused forward (the backward recomputes G), and after the
    unfused forward, which stores fp32 G (gate/up GEMM + SiLU*up, also timed)
    so the backward skips the recompute.  GEMM stages report TFLOP/s,
    streaming stages GB/s of algorithmic bytes."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 17)
    gb = {"bf16": 2, "f32": 4}[cfg.out_dt]
    dy = torch.randn(cfg.T, cfg.H, device=dev, generator=g).to(layer.out.dtype)
    layer.forward(x, ids, w)
    us, total, us_p = _time_stages(layer.backward_stages(dy, w), steps, dev)
    # the same backward with G stored in fp32 and a separate SiLU*up backward
    us_sep, total_sep, _ = _time_stages(layer.backward_stages(dy, w, fuse_silu=False), steps, dev)
    tr_us, _, _ = _time_stages([("transpose_weights", layer.refresh_transposed_weights)], steps, dev)
    # unfused forward keeping G, then the backward without the recompute
    layer.set_fused(False)
    layer.forward(x, ids, w)
    fwd_us, _, _ = _time_stages([("gemm_w13_store_g", layer.gemm_w13), ("silu_mul", layer.silu_mul)],
                                steps, dev)
    layer.forward(x, ids, w)
    us_saved, total_saved, _ = _time_stages(layer.backward_stages(dy, w), steps, dev)
    layer.set_fused(True)
    layer.forward(x, ids, w)

    rows = int(layer.counts.cpu().numpy().sum())
    T, K, H, I = cfg.T, cfg.K, cfg.H, cfg.I
    tok_local = int((layer.slot_of.cpu().numpy() >= 0).any(axis=1).sum())
    flops = {"gemm_dz": 2 * rows * H * I, "gemm_g_silu_bw": 4 * rows * H * I, "gemm_da": 4 * rows * H * I,
             "wgrad_w2": 2 * rows * H * I, "wgrad_w13": 4 * rows * H * I}
    nbytes = {
        # dy once per token with a local route, out rows in, d_out rows out, ids/weights/d_w
        "combine_bw": tok_local * H * gb + 2 * rows * H * gb + T * K * 12,
        # G (fp32) and dZ in, dG out
        "silu_mul_bw": rows * 2 * I * 4 + rows * I * gb + rows * 2 * I * gb,
        # dA rows in, dx out, ids
        "permute_bw": rows * H * gb + T * H * gb + T * K * 4,
    }
    peak = MFMA_PEAK_TFLOPS[cfg.wdt]
    res = {"us": us, "p10_p90_us": us_p, "total_us": total, "rows": rows,
           "transpose_weights_us": tr_us["transpose_weights"],
           "transpose_note": "W2^T and W13^T, written once per weight update (not part of a pass)",
           "timing": "medians over the passes, an event between stages; after the fused forward "
                     "(G recomputed by the gate/up GEMM with the SiLU*up gradient in its epilogue)",
           "tflops": {k: v / (us[k] * 1e-6) / 1e12 for k, v in flops.items() if k in us},
           "gbs": {k: v / (us[k] * 1e-6) / 1e9 for k, v in nbytes.items() if k in us},
           "separate_silu": {"us": {k: us_sep[k] for k in ("gemm_g", "silu_mul_bw")},
                             "backward_total_us": total_sep,
                             "note": "G stored in fp32 by the gate/up GEMM, then a separate SiLU*up "
                                     "backward (same results, bit for bit)"},
           "saved_g": {"backward_us": us_saved, "backward_total_us": total_saved,
                       "forward_unfused_us": fwd_us,
                       "note": "unfused forward (gate/up GEMM storing fp32 G, then SiLU*up) keeps G; "
                               "the backward then skips the recompute"}}
    res["mfma_frac"] = {k: v / peak for k, v in res["tflops"].items()}
    res["hbm_frac"] = {k: v / HBM_PEAK_GBS for k, v in res["gbs"].items()}
    return res


def build_layer(cfg, dev):
    """Seeded inputs of a workload, uploaded, and a layer holding its weights."""
    import torch

    from combine_top_expert_amd.pipeline import LayerShape, MoELayer
    from workloads import make_workload

    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    wl = make_workload(cfg)
    shape = LayerShape(T=cfg.T, K=cfg.K, E=cfg.E, expert_begin=cfg.expert_begin, L=cfg.L, H=cfg.H,
                       I=cfg.I, R=cfg.R, act=cfg.act, wdt=cfg.wdt)

    def up(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).view(torch.bfloat16) if bf16 else t).to(dev)

    layer = MoELayer(shape, device=dev, fused=True)
    fp8 = cfg.wdt == "fp8"
    layer.set_weights(up(wl.w["w13"], cfg.wdt == "bf16"), up(wl.w["w2"], cfg.wdt == "bf16"),
                      up(wl.w["w13_scales"]) if fp8 else None, up(wl.w["w2_scales"]) if fp8 else None)
    x = up(wl.x, cfg.act == "bf16")
    ids = up(wl.ids)
    w = up(wl.weights)
    torch.cuda.synchronize()
    # each launch marshalled once: a step costs a few microseconds of host time
    bound = layer.bind_forward(x, ids, w)
    stages = [n for n, _ in bound]
    fns = [f for _, f in bound]
    return wl, layer, x, ids, w, stages, fns


def stage_pass(stages, fns, steps, stream):
    """Another ``steps`` whole steps with an event between stages: medians
    (and p10/p90) per stage, median step total."""
    import torch

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        ev[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(stages))]
                    for s in range(steps)]) * 1e3                       # us
    stage_us = {k: float(np.median(per[:, i])) for i, k in enumerate(stages)}
    p10_90 = {k: [float(np.percentile(per[:, i], 10)), float(np.percentile(per[:, i], 90))]
              for i, k in enumerate(stages)}
    return stage_us, p10_90, float(np.median(per.sum(axis=1)))


def roofline(work, prefix, us, peak_tf):
    """HBM or MFMA roofline of one GEMM call from its algorithmic bytes and
    flops and its measured duration: the bound is whichever resource takes
    longer at its peak."""
    b, f = work[prefix + "_bytes"], work[prefix + "_flops"]
    if b / (HBM_PEAK_GBS * 1e9) >= f / (peak_tf * 1e12):
        r = {"bound": "hbm", "achieved": b / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": f / (us * 1e-6) / 1e12, "peak": peak_tf, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["avg_us"] = us
    r["algorithmic_bytes"] = b
    r["algorithmic_flops"] = f
    r["mfma_frac"] = f / (us * 1e-6) / 1e12 / peak_tf
    r["hbm_frac"] = b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
    return r


def w2_combine_us(layer, topk_weights, steps, stream):
    """The down GEMM with the combine in its epilogue
    (moe_grouped_gemm_w2_combine: zero fill, GEMM with weighted atomic adds,
    rounding pass) timed like a stage: median of ``steps`` calls, each between
    two events, after the layer's forward has produced Z."""
    import torch

    import combine_top_expert_amd as ep

    s = layer.shape
    y_acc = torch.empty(s.T, s.H, dtype=torch.float32, device=layer.y.device)
    y = torch.empty_like(layer.y)
    f = ep.moe_grouped_gemm_w2_combine(layer.z, layer.z_scales, layer.w2, layer.w2_scales, layer.counts,
                                       layer.offsets, layer.row_src, topk_weights, y_acc, y, bind=True)
    for _ in range(3):
        f()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        f()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))


def workload_summary(cfg, layer, stages, fns, steps, stream, topk_weights=None):
    """Per-stage medians (a pass of whole steps with an event between
    stages) and the derived rates of one workload; with topk_weights, also
    the fused down GEMM + combine alternative against the two stages it
    replaces."""
    stage_us, p10_90, gpu_us = stage_pass(stages, fns, steps, stream)
    slot = layer.slot_of.cpu().numpy()
    counts = layer.counts.cpu().numpy()
    work = algorithmic_work(cfg, counts, int((slot >= 0).any(axis=1).sum()))
    loop = stage_us
    peak = MFMA_PEAK_TFLOPS[cfg.wdt]
    gemm_us = loop["gemm_w13"] + loop["gemm_w2"]
    return {
        "config": {"workload": cfg.name, "T": cfg.T, "K": cfg.K, "E": cfg.E, "L": cfg.L, "H": cfg.H,
                   "I": cfg.I, "R": cfg.R, "rows": work["rows"], "weights": cfg.wdt},
        "rows_per_s_stage_sum": work["rows"] / (gpu_us * 1e-6),
        "stage_us": stage_us, "stage_p10_p90_us": p10_90, "stage_sum_us": gpu_us,
        "gemm_tflops": work["gemm_flops"] / (gemm_us * 1e-6) / 1e12,
        "gemm_mfma_frac": work["gemm_flops"] / (gemm_us * 1e-6) / 1e12 / peak,
        "w13": roofline(work, "w13", loop["gemm_w13"], peak),
        "w2": roofline(work, "w2", loop["gemm_w2"], peak),
        "permute_gbs": work["permute_bytes"] / (loop["permute"] * 1e-6) / 1e9,
        "combine_gbs": work["combine_bytes"] / (loop["combine"] * 1e-6) / 1e9,
        "permute_bytes": work["permute_bytes"], "combine_bytes": work["combine_bytes"],
        **({"w2_combine_fused_us": w2_combine_us(layer, topk_weights, steps, stream),
            "w2_plus_combine_us": stage_us["gemm_w2"] + stage_us["combine"]}
           if topk_weights is not None else {}),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the MoE layer; --gpus {args.gpus} is not "
              "supported (the multi-GPU expert-parallel exchange is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_top_expert_amd  # noqa: F401  (fails loudly without the HIP library)
    from workloads import get_config

    cfg = get_config(args.workload)
    dev = torch.device("cuda:0")
    wl, layer, x, ids, w, stages, fns = build_layer(cfg, dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)       # one elementwise kernel: reads n bytes, writes n
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    # Timed region: exactly K whole steps.  The only events in it are the two
    # around each gate/up GEMM call (the roofline's kernel).  The launches are
    # pre-marshalled, so the host stays ahead of the device and each event
    # pair brackets the GEMM call alone.
    i13 = stages.index("gemm_w13")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        for i, f in enumerate(fns):
            if i == i13:
                ev[s_][0].record(stream)
                f()
                ev[s_][1].record(stream)
            else:
                f()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps                 # whole-job clock, host included
    w13_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    st = layer.dev_status.cpu().numpy()
    if st[0] != 0:
        raise RuntimeError(f"dispatch layout flagged {st}")

    # After the timed region: per-stage breakdown (events between stages).
    summ = workload_summary(cfg, layer, stages, fns, args.steps, stream, topk_weights=w)
    counts = layer.counts.cpu().numpy()
    work = algorithmic_work(cfg, counts)
    peak_tf = MFMA_PEAK_TFLOPS[cfg.wdt]
    roof = roofline(work, "w13", float(np.mean(w13_us)), peak_tf)
    roof["p10_p90_us"] = [float(np.percentile(w13_us, 10)), float(np.percentile(w13_us, 90))]
    roof["traffic"] = recorded_traffic(cfg.name)
    roof["kernel"] = ("grouped_gemm_kernel (moe_grouped_gemm_w13, fused SiLU*up, FP8 Z; the call's "
                      "K-split piece reduce included when it runs)")
    roof["timing"] = ("mean over the timed steps of HIP events recorded right before and after the "
                      "gate/up GEMM call on the kernels' stream")
    # in timed-step order: after a short warm-up the first steps run while the
    # shader clock is still rising, which shows here as a falling sequence
    roof["per_step_us"] = [round(v, 1) for v in w13_us]

    out = {
        "metric": METRIC,
        "value": work["rows"] / (step_ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "gpu_ms_per_step": summ["stage_sum_us"] * 1e-3,
        "stage_timing": "stage_us: medians of a second pass of the same number of steps with an "
                        "event between stages",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.wdt,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "K": cfg.K, "E": cfg.E, "L": cfg.L,
                   "H": cfg.H, "I": cfg.I, "R": cfg.R, "rows": work["rows"],
                   "act": cfg.act, "weights": cfg.wdt, "seed": cfg.seed},
        "gemm_tflops": summ["gemm_tflops"],
        "gemm_mfma_frac": summ["gemm_mfma_frac"],
        "stage_us": summ["stage_us"],
        "stage_p10_p90_us": summ["stage_p10_p90_us"],
        "stage_gbs": {"permute": summ["permute_gbs"], "combine": summ["combine_gbs"]},
        "roofline": roof,
        "roofline_w2": summ["w2"],
        "w2_combine_fused_us": summ["w2_combine_fused_us"],
        "w2_plus_combine_us": summ["w2_plus_combine_us"],
        "cpu_baseline": None,
    }

    out["next_rows"] = {}
    if cfg.routing == "softmax":
        out["next_rows"]["router_topk"] = router_timing(cfg, args.steps, dev)
    if cfg.wdt != "fp8" and not args.skip_backward:
        print("[bench] backward stages", file=sys.stderr, flush=True)
        out["next_rows"]["backward"] = backward_timing(cfg, layer, x, ids, w, min(args.steps, 20), dev)

    extra = [n for n in args.extra_workloads.split(",") if n and n != cfg.name]
    if extra:
        del layer, x, ids, w, fns
        torch.cuda.empty_cache()
        out["other_workloads"] = {}
        for name in extra:
            ecfg = get_config(name)
            ewl, elayer, ex, eids, ew, est, efns = build_layer(ecfg, dev)
            for _ in range(max(args.warmup, 5)):
                for f in efns:
                    f()
            torch.cuda.synchronize()
            print(f"[bench] {name}: stages and kernel loops", file=sys.stderr, flush=True)
            out["other_workloads"][name] = workload_summary(ecfg, elayer, est, efns, min(args.steps, 20),
                                                            stream, topk_weights=ew)
            del ewl, elayer, ex, eids, ew, efns
            torch.cuda.empty_cache()
        torch.cuda.synchronize()

    if not args.skip_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
