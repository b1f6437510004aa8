#!/usr/bin/env python3
"""Benchmark of the decode-step context-KV update (libdfkv) on one MI355X.

One step = dfkv_step on one batch of seeded synthetic inputs: fc over the
concatenated target layers, hidden_norm, the stacked K/V GEMM with k_norm and
RoPE fused into its epilogue, then the bookkeeping and the paged store into
every layer's pool.  Inputs are resident in HBM before timing starts.

Timing: the step is captured in HIP graphs, one per copy of the weights; the
timed loop rotates through 4 copies (4 x the weight bytes > the 256 MiB
Infinity Cache), so every step streams its weights from HBM.  A spin kernel is
queued first so the host runs ahead and the GPU executes the steps back to
back.  The dominant kernel (the projection) is timed the same way with one pair
of HIP events around each launch, on the stream it runs on.

Prints ONE JSON line.  --gpus N > 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per decode-step context-KV update at bs=1/64; accepted rows/s; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def algorithmic(wl, accepted_rows: int) -> dict:
    """Bytes and flops the method must move / compute per step (intermediates f, g, y excluded)."""
    g = wl.geom
    N, K, H, O = wl.n_rows, g.k_in, g.hidden, g.out_dim
    w_bytes = 2 * (H * K + H + O * H + g.n_layers * g.knorm_dim)
    x_bytes = 2 * N * K
    row_bytes = 2 * g.n_layers * g.slot_elems * (2 if g.kind == 0 else 1)
    flops = 2.0 * N * (K * H + H * O)
    return dict(weights=w_bytes, hidden=x_bytes, pool_writes=accepted_rows * row_bytes, kv_out=2 * N * O,
                step_bytes=w_bytes + x_bytes + accepted_rows * row_bytes,
                project_bytes=w_bytes + x_bytes + 2 * N * O, flops=flops)


def cpu_baseline(wl, seconds: float) -> dict:
    """The oracle, as it stands, running whole steps (projection of every row, bookkeeping, store into a
    host pool) on the host cores for about `seconds`."""
    import numpy as np
    import oracle
    orc = oracle.get()
    g = wl.geom
    cs = orc.rope_cache(wl.rope, wl.cache_len)
    P, pg = wl.num_pages, g.page_size
    per_layer_pool = P * pg * g.slot_elems
    pk = [np.zeros(per_layer_pool, np.uint16) for _ in range(g.n_layers)]
    pv = [np.zeros(per_layer_pool, np.uint16) for _ in range(g.n_layers)] if g.kind == 0 else None
    if g.kind == 0:
        sp, ss, sh = pg * g.n_kv_heads * g.head_dim, g.n_kv_heads * g.head_dim, g.head_dim
    else:
        sp, ss, sh = pg * g.slot_elems, g.slot_elems, 0
    steps, rows = 0, 0
    t0 = time.perf_counter()
    while True:
        res = orc.project(g, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs)
        bk = orc.bookkeeping(g, wl.n_reqs, wl.ctx_len, wl.n_acc, wl.alloc_limit, wl.is_dummy, wl.row_valid,
                             wl.block_table, wl.accepted_tokens, wl.acc_stride_req, wl.acc_stride_tok,
                             wl.mask_token_id, wl.num_pages)
        orc.store(g, res["kv"], bk["slot"], bk["write_mask"], pk, pv, sp, ss, sh)
        steps += 1
        rows += int(bk["write_mask"].sum())
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=rows / el, unit="accepted rows/s", cores=orc.threads(), kind="oracle",
                sample=f"{steps} whole steps of the same workload (all {wl.n_rows} rows projected, bookkeeping, "
                       f"store into a host pool) in {el:.1f} s; fp64 plain C, OpenMP",
                us_per_step=1e6 * el / steps)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload: 0 tiny, 1 dense bs=1, 2 dense bs=64, "
                                                           "3 MLA bs=1, 4 stress bs=256")
    ap.add_argument("--ctx", type=int, default=None, help="context length of the bs=1 workloads")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated through (cache defeat)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (for HBM counter scaling) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU; --gpus above 1 is not supported (the step shards by "
              "request with no exchange, so N GPUs each run this same single-GPU step)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0

    from dfkv_workloads import CTX_CHOICES, make_workload
    from store_dfkv_project_amd.step import DeviceStep

    ctx = args.ctx
    if ctx is None and args.config in CTX_CHOICES:
        ctx = CTX_CHOICES[args.config][-1] if args.config == 1 else CTX_CHOICES[args.config][0]
    wl = make_workload(args.config, ctx_choice=ctx)
    R = max(1, args.copies)
    ds = DeviceStep(wl, weight_copies=R)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    # capture: one graph per weight copy for the whole step, and for the projection alone
    step_graphs, proj_graphs = [], []
    with torch.cuda.stream(stream):
        for c in range(R):       # eager warm-up of every path before capture
            ds.step(copy=c)
    torch.cuda.synchronize()
    for c in range(R):
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs, stream=stream):
            ds.step(copy=c)
        step_graphs.append(gs)
        gp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp, stream=stream):
            ds.project(copy=c)
        proj_graphs.append(gp)
    torch.cuda.synchronize()
    accepted = int(ds.write_mask.sum().item())

    def timed(graphs, n, warm):
        with torch.cuda.stream(stream):
            for i in range(warm):
                graphs[i % R].replay()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            torch.cuda._sleep(50_000_000)          # let the host queue the loop ahead of the GPU
            t_all0 = torch.cuda.Event(enable_timing=True)
            t_all1 = torch.cuda.Event(enable_timing=True)
            t_all0.record(stream)
            for i in range(n):
                ev[i][0].record(stream)
                graphs[i % R].replay()
                ev[i][1].record(stream)
            t_all1.record(stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3   # us
        return per, t_all0.elapsed_time(t_all1) * 1e3 / n

    t_wall0 = time.perf_counter()
    step_us, step_avg_us = timed(step_graphs, args.steps, args.warmup)
    wall = time.perf_counter() - t_wall0
    proj_us, _ = timed(proj_graphs, args.steps, args.warmup)

    alg = algorithmic(wl, accepted)
    us_step = float(step_avg_us)
    proj_mean = float(proj_us.mean())
    bound = "hbm" if wl.n_rows <= 64 else "mfma"
    if bound == "hbm":
        achieved = alg["project_bytes"] / (proj_mean * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    else:
        achieved = alg["flops"] / (proj_mean * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_PEAK_TFLOPS, 4))
    roof.update(traffic=None, kernel="dfkv_project (fc + stacked K/V GEMM with fused k_norm/RoPE)",
                algorithmic_bytes_per_launch=alg["project_bytes"], algorithmic_flops_per_launch=alg["flops"],
                launch_us_mean=round(proj_mean, 2), launch_us_p10=round(float(np.percentile(proj_us, 10)), 2),
                launch_us_p90=round(float(np.percentile(proj_us, 90)), 2))

    out = {
        "metric": METRIC,
        "value": round(accepted / (us_step * 1e-6), 1),
        "unit": "accepted rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "us_per_step": round(us_step, 2),
        "us_per_step_p10": round(float(np.percentile(step_us, 10)), 2),
        "us_per_step_median": round(float(np.median(step_us)), 2),
        "us_per_step_p90": round(float(np.percentile(step_us, 90)), 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "config_id": args.config, "requests": wl.n_reqs, "rows": wl.n_rows,
                   "accepted_rows": accepted, "ctx_len": ctx, "k_in": wl.geom.k_in, "hidden": wl.geom.hidden,
                   "out_dim": wl.geom.out_dim, "layers": wl.geom.n_layers, "weight_copies": R,
                   "step_bytes": alg["step_bytes"], "step_flops": alg["flops"], "timing": "hipGraph replay, "
                   "HIP events on the replay stream"},
        "roofline": roof,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
