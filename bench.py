#!/usr/bin/env python3
"""Benchmark of the LiteAttention step on one MI355X.

A step is one denoising step of the whole hot path over the workload: one lite_attn_step
launch over every (batch, head, query tile) with the persistent skip mask, following the
workload's error-budget schedule (a generation of T steps starts from lite_attn_reset_mask).
Inputs for all T steps are generated on the GPU before timing and stay resident in HBM.

Prints ONE JSON line:
  value             dense-equivalent TFLOP/s over the timed steps: steps * 4*B*H*N^2*D / time
  skipped_tile_fraction  mean fraction of tiles skipped over the timed steps
  roofline          the attention kernel against the bf16 MFMA peak: algorithmic flops of the
                    computed tiles per launch / mean launch duration (HIP events on the launch
                    stream), plus HBM traffic per launch from rocprofv3 counters when they were
                    taken on the current kernel source
  cpu_baseline      the CPU oracle timed on this host on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dense-equiv attention TFLOP/s per denoising step; skipped-tile fraction"
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 flop/clk x 2.4 GHz
FP32_PEAK_TFLOPS = 157.3
DEFAULT_WORKLOAD = "wan14b_720p"
KERNEL_SOURCES = ["temporally_sparse_attention_amd/csrc/lite_attn_kernels.hip",
                  "temporally_sparse_attention_amd/csrc/lite_attn_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: one generation)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default: one generation)")
    ap.add_argument("--config", default=DEFAULT_WORKLOAD, help="workload name or id 1-5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    ap.add_argument("--per-step", action="store_true", help="add per-step times to the JSON")
    ap.add_argument("--schedule", action="store_true",
                    help="use lite_attn_step_scheduled (query tiles by visit count: heavy first, short "
                         "last; the "
                         "scheduling kernel is inside the timed step)")
    ap.add_argument("--refresh-delta", type=float, default=None,
                    help="use lite_attn_step_refresh with this divergence budget (mask rows whose "
                         "statistic moves by more are cleared)")
    ap.add_argument("--calibrate", default=None, metavar="LO,HI",
                    help="derive the log_eps schedule with lite_attn_calibrate (untimed, before the "
                         "warmup) from output-error budgets rising linearly from LO to HI (max "
                         "|out - dense|), and time that schedule instead of the workload's")
    ap.add_argument("--in-step-skip", action="store_true",
                    help="enable the in-step-skip option (tiles flagged in a step also leave that "
                         "step's output; their exponentials and PV are not computed)")
    ap.add_argument("--repeats", type=int, default=0, metavar="R",
                    help="also time every step of one generation R times, restoring the mask "
                         "(and tile statistics) from a saved copy before each repeat, outside the "
                         "timed events; reports the per-step medians and a fit over them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    return ap.parse_args()


def generate(cfg, dev):
    """Q_t, K_t for every step of the schedule and V, as bf16/fp32 [B, H, N, D] on `dev`."""
    import torch
    from workloads import Workload
    wl = Workload(cfg, dev)
    shape = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)
    qs = [torch.empty(shape, dtype=cfg.dtype, device=dev) for _ in range(cfg.steps)]
    ks = [torch.empty(shape, dtype=cfg.dtype, device=dev) for _ in range(cfg.steps)]
    v = torch.empty(shape, dtype=cfg.dtype, device=dev)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            for t in range(cfg.steps):
                qt, kt, vt = wl.head_inputs(t, b, h)
                qs[t][b, h].copy_(qt)
                ks[t][b, h].copy_(kt)
                if t == 0:
                    v[b, h].copy_(vt)
            wl._base_cache.pop((b, h), None)
    torch.cuda.synchronize()
    return qs, ks, v


def computed_work(mask, cfg, tiles_q, tiles_k):
    """Algorithmic work of one step given the mask at its start, over the tiles whose bit is
    clear (valid rows and columns only): flops 4 * rows * cols * D, K/V bytes requested
    2 * cols * D * sizeof(dtype), and the skipped-tile fraction."""
    import torch
    n, bq, bk = cfg.seq_len, cfg.tile_q, cfg.tile_k
    dev = mask.device
    j = torch.arange(tiles_k, device=dev)
    words = mask.view(torch.int32)[..., (j // 32)]
    bits = ((words >> (j % 32).to(torch.int32)) & 1).to(torch.float64)          # [B,H,Tq,Tk]
    rows = torch.clamp(n - torch.arange(tiles_q, device=dev) * bq, max=bq).to(torch.float64)
    cols = torch.clamp(n - j * bk, max=bk).to(torch.float64)
    keep = 1.0 - bits
    computed = (keep * rows[:, None] * cols[None, :]).sum().item()
    kv_cols = (keep * cols[None, :]).sum().item()
    elt = 2 if cfg.dtype == torch.bfloat16 else 4
    return 4.0 * computed * cfg.head_dim, 2.0 * kv_cols * cfg.head_dim * elt, bits.mean().item()


def linear_fit(xs, ys):
    """Least-squares y = a x + b; returns (a, b, r2)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    if n < 2 or sxx == 0.0:
        return None, None, None
    a = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    b = my - a * mx
    ss_tot = sum((y - my) ** 2 for y in ys)
    ss_res = sum((y - (a * x + b)) ** 2 for x, y in zip(xs, ys))
    return a, b, (1.0 - ss_res / ss_tot) if ss_tot > 0 else None


def per_step_medians(att, cfg, qs, ks, v, out, log_eps, stream, dev, args, workspace, tiles_q,
                     tiles_k):
    """Per-step timing protocol: along one generation from an empty mask, step t is launched R
    times, each time from the mask (and tile statistics) saved before its first launch; the
    restore is a device copy outside the timed events. Returns the median and spread of each
    step's launch time, the rates at the median, and the fit t = t_dense (1 - s) + t0 over the
    medians."""
    import statistics
    import torch
    R = args.repeats
    refresh = args.refresh_delta is not None
    mask = att.new_mask(dev)
    att.reset_mask(mask)
    stats = att.new_tile_stats(dev) if refresh else None
    if refresh:
        stats.fill_(float("nan"))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = []
    for t in range(cfg.steps):
        saved = mask.clone()
        saved_stats = stats.clone() if refresh else None
        f, kvb, sfrac = computed_work(mask, cfg, tiles_q, tiles_k)
        times = []
        for _ in range(R):
            mask.copy_(saved)
            if refresh:
                stats.copy_(saved_stats)
            e0.record(stream)
            if refresh:
                att.step(qs[t], ks[t], v, out, mask, log_eps[t], t, tile_stats=stats,
                         refresh_delta=args.refresh_delta)
            else:
                att.step(qs[t], ks[t], v, out, mask, log_eps[t], t, workspace=workspace)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        if args.in_step_skip:
            # tiles flagged during the step were scored but got no PV product
            f_after, _, _ = computed_work(mask, cfg, tiles_q, tiles_k)
            f = f_after + 0.5 * (f - f_after)
        med = statistics.median(times)
        rows.append({"t": t, "skipped": round(sfrac, 4), "kernel_ms_median": round(med, 4),
                     "kernel_ms_min": round(min(times), 4), "kernel_ms_max": round(max(times), 4),
                     "computed_tflops": round(f / (med * 1e-3) / 1e12, 2),
                     "kv_gbs_requested": round(kvb / (med * 1e-3) / 1e9, 1)})
    a, b0, r2 = linear_fit([1.0 - r["skipped"] for r in rows], [r["kernel_ms_median"] for r in rows])
    return {"repeats": R, "steps": rows,
            "time_fit": None if a is None else {"t_dense_ms": round(a, 3), "t0_ms": round(b0, 3),
                                                "r2": None if r2 is None else round(r2, 4)}}


def host_cpu() -> dict:
    """The host the CPU baseline ran on: logical CPUs and the processor model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "model": model}


def cpu_baseline(cfg, qs, ks, v, budget_s: float):
    """Time the CPU oracle on whole query tiles of step 0 until `budget_s` is spent."""
    import numpy as np
    import torch
    from oracle import lite_attn_step_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    bh = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    b, h = bh[int(rng.integers(len(bh)))]
    q = qs[0][b:b + 1, h:h + 1].cpu()
    k = ks[0][b:b + 1, h:h + 1].cpu()
    vv = v[b:b + 1, h:h + 1].cpu()
    tq = cfg.tiles_q
    w = -(-cfg.tiles_k // 32)
    mask = np.zeros((1, 1, tq, w), dtype=np.uint32)
    order = rng.permutation(tq)
    done, dense_flops = 0, 0.0
    t0 = time.perf_counter()
    while done < len(order):
        i = int(order[done])
        lite_attn_step_ref(q, k, vv, mask, tile_q=cfg.tile_q, tile_k=cfg.tile_k,
                           softmax_scale=cfg.softmax_scale, log_eps=cfg.log_eps[0], step=0,
                           order=cfg.order, dense_prefix=cfg.dense_prefix, rows=[(0, 0, i)])
        rows = min(cfg.tile_q, cfg.seq_len - i * cfg.tile_q)
        dense_flops += 4.0 * rows * cfg.seq_len * cfg.head_dim
        done += 1
        if time.perf_counter() - t0 >= budget_s and done >= 2:
            break
    dt = time.perf_counter() - t0
    return {
        "value": dense_flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "host": host_cpu(),
        "sample": f"{done} query tiles of step 0 of {cfg.name} (batch {b}, head {h}), float64 "
                  f"numpy oracle, {dt:.1f} s; dense-equivalent flops of those tiles / time",
    }


def traffic_per_launch(kernel_hash: str, workload: str):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3 counter
    summary, if it was taken on this kernel source and workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_hash") != kernel_hash:
        return None
    return entry.get("bytes_per_launch")


def copy_calibration(torch):
    """Plain kernels of known traffic: a fill writes 2^30 bytes, a copy reads and writes 2^30
    bytes, a sum reads 2^30 bytes (each three times)."""
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        src.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    total = 0.0
    for _ in range(3):
        total += float(src.sum())
    torch.cuda.synchronize()
    log(f"[bench] copy calibration done (checksum {total:.0f})")


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention of "
              "each (batch, head) is independent and would be sharded by head across GPUs, "
              "which this benchmark does not do.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import temporally_sparse_attention_amd as tsa
    from workloads import get_config

    cfg = get_config(args.config)
    steps = cfg.steps if args.steps is None else args.steps
    warmup = cfg.steps if args.warmup is None else args.warmup
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    log(f"[bench] generating {cfg.name}: B={cfg.batch} H={cfg.heads} N={cfg.seq_len} "
        f"D={cfg.head_dim} {cfg.dtype} x {cfg.steps} steps")
    t0 = time.perf_counter()
    qs, ks, v = generate(cfg, dev)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    dt_name = "bf16" if cfg.dtype == torch.bfloat16 else "fp32"
    att = tsa.LiteAttention(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, tile_q=cfg.tile_q,
                            tile_k=cfg.tile_k, dtype=dt_name, softmax_scale=cfg.softmax_scale,
                            order=cfg.order, dense_prefix=cfg.dense_prefix,
                            in_step_skip=args.in_step_skip)
    tiles_q, tiles_k = att.tiles
    out = torch.empty_like(qs[0])
    mask = att.new_mask(dev)
    stream = torch.cuda.current_stream(dev)
    log_eps = list(cfg.log_eps)
    calibration = None
    if args.calibrate:
        lo, hi = (float(x) for x in args.calibrate.split(","))
        n_st = cfg.steps
        budgets = [lo + (hi - lo) * t / max(1, n_st - 1) for t in range(n_st)]
        log(f"[bench] calibrating log_eps for budgets {lo} .. {hi}")
        res = att.calibrate(qs[:n_st], ks[:n_st], [v] * n_st, budgets)
        log_eps = list(res.log_eps)
        calibration = res.as_dict()
        calibration["log_eps"] = [None if math.isinf(x) else x for x in res.log_eps]
        log(f"[bench] calibrated log_eps {log_eps}")
    workspace = att.new_workspace(dev) if args.schedule else None
    refresh = args.refresh_delta is not None
    if refresh and args.schedule:
        sys.exit("--schedule and --refresh-delta do not combine")
    stats = att.new_tile_stats(dev) if refresh else None
    stats2 = att.new_tile_stats(dev) if refresh else None

    def run_step(k_idx, ev=None):
        t = k_idx % cfg.steps
        if t == 0:
            att.reset_mask(mask)
            if refresh:
                stats.fill_(float("nan"))
        if ev is not None:
            ev[0].record(stream)
        if refresh:
            att.step(qs[t], ks[t], v, out, mask, log_eps[t], t, tile_stats=stats,
                     refresh_delta=args.refresh_delta)
        else:
            att.step(qs[t], ks[t], v, out, mask, log_eps[t], t, workspace=workspace)
        if ev is not None:
            ev[1].record(stream)

    # warmup
    for k_idx in range(warmup):
        run_step(k_idx)
    torch.cuda.synchronize()

    # timed region
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for s in range(steps):
        run_step(warmup + s, events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kernel_ms = [a.elapsed_time(b) for a, b in events]

    # untimed replay of the same (deterministic) chain for per-step skipped fractions and
    # algorithmic flops of the computed tiles
    flops, kv_bytes, skipped = [], [], []
    mask2 = att.new_mask(dev)
    for k_idx in range(warmup + steps):
        t = k_idx % cfg.steps
        if t == 0:
            att.reset_mask(mask2)
            if refresh:
                stats2.fill_(float("nan"))
        if k_idx >= warmup:
            f, kvb, sfrac = computed_work(mask2, cfg, tiles_q, tiles_k)
        if refresh:
            att.step(qs[t], ks[t], v, out, mask2, log_eps[t], t, tile_stats=stats2,
                     refresh_delta=args.refresh_delta)
        else:
            att.step(qs[t], ks[t], v, out, mask2, log_eps[t], t)
        if k_idx >= warmup:
            if args.in_step_skip:
                # tiles flagged during this step were scored (QK) but got no PV product
                f_after, _, _ = computed_work(mask2, cfg, tiles_q, tiles_k)
                f = f_after + 0.5 * (f - f_after)
            flops.append(f)
            kv_bytes.append(kvb)
            skipped.append(sfrac)
    torch.cuda.synchronize()
    if not torch.equal(mask, mask2):
        log("[bench] warning: replayed mask chain differs from the timed chain")

    dense = cfg.dense_flops()
    value = steps * dense / wall / 1e12
    mean_ms = sum(kernel_ms) / len(kernel_ms)
    achieved = (sum(flops) / len(flops)) / (mean_ms * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if dt_name == "bf16" else FP32_PEAK_TFLOPS
    khash = kernel_source_hash()
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        # counters were taken on the plain step (no option) of the default schedule
        "traffic": (traffic_per_launch(khash, cfg.name)
                    if not (args.in_step_skip or args.schedule or refresh or args.calibrate)
                    else None),
        "kernel": f"lite_attn_fwd_{dt_name} (D={cfg.head_dim}, tile {cfg.tile_q}x{cfg.tile_k})",
        "kernel_ms_mean": round(mean_ms, 4),
        "flops_per_launch_mean": sum(flops) / len(flops),
        "kernel_source_hash": khash,
    }
    if args.repeats > 0:
        result_repeats = per_step_medians(att, cfg, qs, ks, v, out, log_eps, stream, dev, args,
                                          workspace, tiles_q, tiles_k)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(cfg, qs, ks, v, args.cpu_seconds)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "batch": cfg.batch, "heads": cfg.heads, "seq_len": cfg.seq_len,
            "head_dim": cfg.head_dim, "tile_q": cfg.tile_q, "tile_k": cfg.tile_k,
            "schedule_steps": cfg.steps, "softmax_scale": cfg.softmax_scale, "order": cfg.order,
            "dense_prefix": cfg.dense_prefix, "parallelism": "single GPU",
            "in_step_skip": bool(args.in_step_skip), "schedule": bool(args.schedule),
            "refresh_delta": args.refresh_delta,
            "log_eps": [None if math.isinf(x) else x for x in log_eps],   # None: -inf
        },
        "skipped_tile_fraction": round(sum(skipped) / len(skipped), 4),
        "dense_step_tflops_equiv_per_step": None,
        "computed_tflops_mean": round(achieved, 2),
        "kv_gbs_requested_mean": round(sum(kv_bytes) / (sum(kernel_ms) * 1e-3) / 1e9, 1),
        "time_fit": None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    # dense step (t = 0 of a generation) rate, if one was timed
    dense_steps = [kernel_ms[s] for s in range(steps) if (warmup + s) % cfg.steps == 0]
    if dense_steps:
        result["dense_step_tflops_equiv_per_step"] = round(dense / (min(dense_steps) * 1e-3) / 1e12, 2)
    # time_t ~= t_dense * (1 - s_t) + t0 over the timed steps
    a, b0, r2 = linear_fit([1.0 - x for x in skipped], kernel_ms)
    if a is not None:
        result["time_fit"] = {"t_dense_ms": round(a, 3), "t0_ms": round(b0, 3),
                              "r2": None if r2 is None else round(r2, 4)}
    if calibration is not None:
        result["calibration"] = calibration
    if args.repeats > 0:
        result["per_step_repeats"] = result_repeats
    if args.per_step:
        result["per_step"] = [
            {"t": (warmup + s) % cfg.steps, "kernel_ms": round(kernel_ms[s], 4),
             "skipped": round(skipped[s], 4),
             "computed_tflops": round(flops[s] / (kernel_ms[s] * 1e-3) / 1e12, 2),
             "kv_gbs_requested": round(kv_bytes[s] / (kernel_ms[s] * 1e-3) / 1e9, 1)}
            for s in range(steps)]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
