#!/usr/bin/env python3
"""Benchmark of the fused-MoE expert computation on one MI355X.

A step is one pass of the whole expert path over one batch of synthetic
inputs already resident in HBM: align/permute, W1 GEMM with SiLU-and-mul
(and, for MXFP8 weights, the activation quantisation), W2 GEMM with the
unpermute scatter, and the ordered top-k weighted reduce, launched through
the C ABI stage by stage on one stream (the same kernels moe_apply_contiguous
launches), with HIP events between the stages.

Default workload: the decode batch (M=4, K=4096, I=8192, E=64, top-8, bf16),
which is weight-bandwidth bound; ``--config`` picks another of the five.
Prints one JSON line: tokens/s for the whole job, the dominant kernel's
roofline (measured live from the events), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE layer tokens/s; TFLOP/s vs MFMA peak (prefill), GB/s vs HBM (decode)"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode",
                    help="tiny | decode | prefill | mxfp8 | batched (or a full workload name); "
                         "train_gu | train_dn: the training grouped GEMMs of one projection")
    ap.add_argument("--row-scales", action="store_true",
                    help="MXFP8: keep the weight scale arrays row-major instead of grouping them "
                         "(moe_pack_mxfp8_scales) where the tile kernels can read them grouped")
    ap.add_argument("--variant", default="auto", choices=["auto", "tile", "stream", "fused"],
                    help="kernel family (auto: the plan's choice); fused: one launch for align, "
                         "W1 and W2, then the reduce, timed as one stage")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens (or batched rows) the CPU oracle is timed on (0: per-workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until this much CPU time has been spent")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of this many MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter files of this "
                         "workload and of --copy-calibration into profiles/traffic_<workload>.json")
    return ap.parse_args()


def kernel_source_hash(files):
    """Hash of the kernels' sources with comments and whitespace removed, so
    that only a change to the code itself invalidates recorded counters."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixture_experts_expert_align_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(re.sub(r"\s+", "", src).encode())
    return h.hexdigest()[:16]


def traffic_record(cfg_name: str, kernel_files):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if there is none or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel_files):
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_LAUNCHES):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": COPY_LAUNCHES}))


def counter_values(path: str, counter: str, kernel_substr: str):
    """Per-dispatch values (KiB) of one counter for kernels whose name contains
    kernel_substr, from a rocprofv3 counter_collection.csv."""
    import csv
    vals = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter or kernel_substr not in row.get("Kernel_Name", ""):
                continue
            d = row.get("Dispatch_Id") or row.get("Correlation_Id")
            vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
    return list(vals.values())


def traffic_from(args):
    import numpy as np
    if args.config.startswith("train"):
        cfg_name = "_".join(args.config.split("_")[:2])
    else:
        cfg_name = args.config.split("_")[0] + ("" if args.variant == "auto" else "_" + args.variant)
    kerns = DOMINANT_KERNEL[cfg_name]
    # per kernel of the timed stage: the median over its dispatches; the
    # stage's traffic is the sum over its kernels
    fetch = [float(np.median(counter_values(args.traffic_from[0], "FETCH_SIZE", k))) for k in kerns]
    write = [float(np.median(counter_values(args.traffic_from[1], "WRITE_SIZE", k))) for k in kerns]
    # the calibration run makes COPY_LAUNCHES copies; the runtime may split a
    # copy over several dispatches, so compare per-copy sums
    cfetch = sum(counter_values(args.traffic_from[2], "FETCH_SIZE", "copy")) / COPY_LAUNCHES
    cwrite = sum(counter_values(args.traffic_from[3], "WRITE_SIZE", "copy")) / COPY_LAUNCHES
    copy_bytes = COPY_MIB << 20
    f_scale = copy_bytes / (cfetch * 1024)
    w_scale = copy_bytes / (cwrite * 1024)
    traffic = sum(fetch) * 1024 * f_scale + sum(write) * 1024 * w_scale
    rec = {"workload": cfg_name, "kernels": list(kerns),
           "kernel_source_hash": kernel_source_hash(KERNEL_FILES[cfg_name]),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "copy_calibration_bytes": copy_bytes,
           "copy_fetch_kib": float(cfetch), "copy_write_kib": float(cwrite),
           "fetch_scale": f_scale, "write_scale": w_scale,
           "traffic_bytes_per_launch": int(traffic)}
    out = os.path.join(ROOT, "profiles", f"traffic_{cfg_name}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


COPY_MIB = 1024
COPY_LAUNCHES = 3
# The kernels of each workload's timed dominant stage (name substrings in
# the profiler's kernel names) and the sources they are built from: the W1
# stage (gate_up_act) for the contiguous format (for MXFP8 weights it also
# quantises the gathered activation rows), both GEMMs (apply_batched) for
# the batched format.
# traffic records: keyed by workload, or workload_variant for a forced variant
FUSED_KERNELS = ["fused_stream_bf16_kernel", "reduce_contiguous_kernel"]
FUSED_FILES = ["fused.hip", "stream_bf16.h", "align_device.h", "reduce_codec.hip"]
DOMINANT_KERNEL = {"tiny": FUSED_KERNELS, "decode": ["gemm_stream_bf16_kernel<0,"],
                   "prefill": ["gemm_tile_split_bf16_kernel<0,"],
                   "mxfp8": ["quantize_gather_kernel", "gemm_tile_mxfp8_kernel<0"],
                   "mxfp8_stream": ["quantize_gather_kernel", "gemm_stream_mxfp8_kernel<0,"],
                   "batched": ["gemm_tile_split_bf16_kernel<0,", "gemm_tile_split_bf16_kernel<1,"],
                   "decode_fused": FUSED_KERNELS, "tiny_fused": FUSED_KERNELS,
                   "train_gu": ["train_wgrad_tile_kernel"], "train_dn": ["train_wgrad_tile_kernel"]}
KERNEL_FILES = {"tiny": FUSED_FILES, "decode": ["gemm_stream.hip", "stream_bf16.h"],
                "prefill": ["gemm_tile.hip", "tile_common.h"],
                "mxfp8": ["reduce_codec.hip", "gemm_mxfp8_tile.hip", "tile_common.h"],
                "mxfp8_stream": ["reduce_codec.hip", "gemm_mxfp8.hip"],
                "batched": ["gemm_tile.hip", "tile_common.h"], "decode_fused": FUSED_FILES, "tiny_fused": FUSED_FILES,
                "train_gu": ["train.hip", "gemm_tile.hip", "tile_common.h"],
                "train_dn": ["train.hip", "gemm_tile.hip", "tile_common.h"]}


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library runs on one GPU and has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.config.startswith("train"):
        main_train(args)
        return

    import numpy as np
    import torch

    import moe_inputs as mi
    import mixture_experts_expert_align_amd as moe

    cfg = mi.config(args.config)
    dev = "cuda"
    torch.cuda.init()
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = mi.make_inputs(cfg, device=dev, weights=True)
    w1_scale = w2_scale = None
    if cfg.w_dtype == "mxfp8":
        w1 = torch.empty(inp.w1.shape, dtype=torch.uint8, device=dev)
        w2 = torch.empty(inp.w2.shape, dtype=torch.uint8, device=dev)
        w1_scale = torch.empty((*inp.w1.shape[:-1], cfg.K // 32), dtype=torch.uint8, device=dev)
        w2_scale = torch.empty((*inp.w2.shape[:-1], cfg.I // 32), dtype=torch.uint8, device=dev)
        moe.moe_quantize_mxfp8(inp.w1, w1, w1_scale)
        moe.moe_quantize_mxfp8(inp.w2, w2, w2_scale)
        torch.cuda.synchronize()
        w_f32 = (inp.w1, inp.w2)
        inp.w1 = inp.w2 = None
    else:
        w1, w2 = inp.w1, inp.w2
        w_f32 = None

    contiguous = cfg.layout == "contiguous"
    # an expert-parallel share (the affine routing) is fed as an EP
    # implementation receives it: global ids, unmasked weights, the rank's map
    ep_share = contiguous and inp.global_ids is not None
    # MXFP8 on the tile kernels: the scale arrays grouped once, as weights are
    # loaded (outside the timed steps), where the shape allows it
    grouped = (cfg.w_dtype == "mxfp8" and not args.row_scales and args.variant in ("auto", "tile")
               and cfg.K % 512 == 0 and cfg.I % 512 == 0)
    if grouped:
        p1, p2 = torch.empty_like(w1_scale), torch.empty_like(w2_scale)
        moe.moe_pack_mxfp8_scales(w1_scale, p1)
        moe.moe_pack_mxfp8_scales(w2_scale, p2)
        torch.cuda.synchronize()
        w1_scale, w2_scale = p1, p2
    w_dtype = moe.W_BF16 if cfg.w_dtype == "bf16" else moe.W_MXFP8_GROUPED if grouped else moe.W_MXFP8
    prob = moe.make_problem(cfg.M, cfg.K, cfg.I, cfg.E, topk=cfg.topk, max_tokens=cfg.max_tokens,
                            layout=0 if contiguous else 1, w_dtype=w_dtype,
                            w1_order=0 if cfg.w1_order == "halves" else 1,
                            global_experts=cfg.global_experts if ep_share else 0,
                            variant={"auto": moe.VARIANT_AUTO, "tile": moe.VARIANT_TILE,
                                     "stream": moe.VARIANT_STREAM, "fused": moe.VARIANT_FUSED}[args.variant])
    plan = moe.moe_plan_init(prob)
    ws13, ws2 = moe.allocate_workspaces(plan)
    stream = torch.cuda.current_stream()

    if contiguous:
        emap = None
        if ep_share:
            ids = torch.from_numpy(inp.global_ids).to(dev)
            wts = torch.from_numpy(inp.global_weights).to(dev)
            emap = torch.from_numpy(mi.ep_expert_map(cfg.global_experts, cfg.E, rank=0)).to(dev)
        else:
            ids = torch.from_numpy(inp.topk_ids).to(dev)
            wts = torch.from_numpy(inp.topk_weights).to(dev)
        out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device=dev)
        R = cfg.M * cfg.topk
        valid = (inp.topk_ids >= 0) & (inp.topk_ids < cfg.E)
        n_routes = int(valid.sum())
        active = np.unique(inp.topk_ids[valid])
        n_tok_read = int(valid.any(axis=1).sum())
        stages = ["align", "gate_up_act", "down_unpermute", "reduce"]
        fused = plan.variant == moe.VARIANT_FUSED
        if fused:
            stages = ["apply"]

        def step(ev):
            if fused:   # the two launches of the single-launch variant, one stage
                ev[0].record(stream)
                moe.moe_apply_contiguous(plan, inp.x, ids, wts, w1, w2, out, ws13, ws2, w1_scale,
                                         w2_scale, stream, expert_map=emap)
                ev[1].record(stream)
                return
            ev[0].record(stream)
            moe.moe_align_permute(plan, ids, ws13, stream, expert_map=emap)
            ev[1].record(stream)
            moe.moe_gate_up_act(plan, inp.x, w1, w2, ws13, w1_scale, w2_scale, stream)
            ev[2].record(stream)
            moe.moe_down_unpermute(plan, w1, w2, ws13, ws2, w1_scale, w2_scale, stream)
            ev[3].record(stream)
            moe.moe_topk_reduce_contiguous(plan, ws2.view(torch.bfloat16), ids, wts, out, stream, expert_map=emap)
            ev[4].record(stream)
    else:
        counts = torch.from_numpy(inp.expert_num_tokens).to(dev)
        row_token = torch.from_numpy(inp.row_token).to(dev)
        row_weight = torch.from_numpy(inp.row_weight).to(dev)
        y = torch.empty((cfg.E, cfg.max_tokens, cfg.K), dtype=torch.bfloat16, device=dev)
        out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device=dev)
        wsr = torch.empty(moe.moe_naive_batched_ws_bytes(plan, cfg.M), dtype=torch.uint8, device=dev)
        n_routes = int(inp.expert_num_tokens.sum())
        active = np.flatnonzero(inp.expert_num_tokens > 0)
        stages = ["apply_batched", "reduce_naive_batched"]

        def step(ev):
            ev[0].record(stream)
            moe.moe_apply_batched(plan, inp.a, counts, w1, w2, y, ws13, stream)
            ev[1].record(stream)
            moe.moe_topk_reduce_naive_batched(plan, y, counts, row_token, row_weight, cfg.M, out,
                                              wsr, stream)
            ev[2].record(stream)

    elapsed, stage_ms, step_ev, cold_ev, aa_ev = time_steps(step, stages, args, dev)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = cfg.M
    value = tokens * args.steps / elapsed

    # ---- roofline of the dominant kernel (algorithmic work per launch)
    n_act = len(active)
    K, I = cfg.K, cfg.I
    if cfg.w_dtype == "mxfp8":
        wbytes = 1.0 + 1.0 / 32
        dtype_name = "bf16 activations, MXFP8 weights" + (" (scale arrays grouped)" if grouped else "")
        # both GEMMs multiply E4M3 codes with UE8M0 block scales (activations
        # and z quantised on the device), fp32 accumulate
        dtype = "mxfp8"
    else:
        wbytes = 2.0
        dtype_name = "bf16"
        dtype = "bf16"
    if contiguous and "apply" in stage_ms:
        # the whole layer in one stage: both weight sets, x rows read once,
        # out written once (intermediates are the implementation's overhead)
        dom = "apply"
        t_dom = stage_ms[dom] * 1e-3
        alg_bytes = n_act * 3 * I * K * wbytes + n_tok_read * K * 2 + cfg.M * K * 2
        alg_flops = 6.0 * n_routes * K * I
    elif contiguous:
        dom = "gate_up_act"
        t_dom = stage_ms[dom] * 1e-3
        w1_bytes = n_act * 2 * I * K * wbytes
        alg_bytes = w1_bytes + n_tok_read * K * 2 + n_routes * I * (2 if cfg.w_dtype == "bf16" else 1 + 1 / 32)
        alg_flops = 4.0 * n_routes * K * I
    else:
        dom = "apply_batched"
        t_dom = stage_ms[dom] * 1e-3
        alg_bytes = n_act * 3 * I * K * wbytes + 2 * n_routes * K * 2
        alg_flops = 6.0 * n_routes * K * I
    flops_per_byte = alg_flops / alg_bytes
    mfma_bound = flops_per_byte > (PEAK_TFLOPS["bf16"] * 1e12) / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = alg_flops / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4)}
    else:
        achieved = alg_bytes / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["kernel_ms"] = round(stage_ms[dom], 4)
    roof["algorithmic_per_launch"] = {"bytes": int(alg_bytes), "flops": int(alg_flops)}
    tkey = cfg.name.split("_")[0] + ("" if args.variant == "auto" else "_" + args.variant)
    roof["traffic"] = traffic_record(tkey, KERNEL_FILES[tkey]) if tkey in KERNEL_FILES else None

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, w1, w2, w_f32, args.cpu_sample, args.cpu_seconds)

    step_gbs = (n_act * 3 * I * K * wbytes) / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded counter-based generator; random-init expert weights)",
        "value_basis": "wall clock over the K steps, issued back to back (L2 and Infinity Cache as "
                       "the previous step left them); value_cache_flushed: tokens / p50 of K steps "
                       "each after a 512 MiB cache flush",
        "value_cache_flushed": round(tokens / (float(np.percentile(cold_ev, 50)) * 1e-3), 2),
        "config": {"workload": cfg.name, "M": cfg.M, "K": K, "I": I, "E": cfg.E, "topk": cfg.topk,
                   "max_tokens": cfg.max_tokens, "weights": dtype_name, "routes": n_routes,
                   "active_experts": n_act, "variant": plan.reason.decode(),
                   "global_experts": int(plan.prob.global_experts)},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "step_event_ms": pct(step_ev),
        "step_event_ms_cache_flushed": pct(cold_ev),
        "noise": noise(step_ev, aa_ev),
        "step_weight_GBps": round(step_gbs, 1),
        "step_TFLOPs": round(6.0 * n_routes * K * I / (ms_per_step * 1e-3) / 1e12, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def noise(step_ev, aa_ev):
    """Noise floor of the per-step event times: the 95% confidence interval
    of the mean step (normal approximation over the K steps) and an A/A
    rerun of the same K steps right after, as the measurement method of the
    deterministic grouped GEMM page does (A/A noise as the smallest
    detectable effect, 95% CI)."""
    import numpy as np
    a = np.asarray(step_ev, dtype=np.float64)
    b = np.asarray(aa_ev, dtype=np.float64)
    half = 1.96 * a.std(ddof=1) / np.sqrt(a.size) if a.size > 1 else 0.0
    return {"mean_ms": round(float(a.mean()), 4),
            "ci95_ms": [round(float(a.mean() - half), 4), round(float(a.mean() + half), 4)],
            "aa_mean_ms": round(float(b.mean()), 4),
            "aa_diff_pct": round(float(100.0 * (b.mean() - a.mean()) / a.mean()), 3)}


def pct(v):
    import numpy as np
    return {f"p{q}": round(float(np.percentile(v, q)), 4) for q in (10, 50, 90)}


def time_steps(step, stages, args, dev):
    """W untimed steps, then exactly K timed ones between two synchronisations
    (wall clock), with HIP events between the stages on the launch stream;
    then K more the same way (the A/A rerun); then K more, each after a
    512 MiB fill that flushes L2 and the Infinity Cache (outside each step's
    events and outside the wall-clock steps).  Returns (seconds for the K
    steps, mean ms per stage, per-step event ms, per-step event ms of the
    flushed steps, per-step event ms of the rerun)."""
    import numpy as np
    import torch
    nev = len(stages) + 1
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = {s: float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in events]))
                for i, s in enumerate(stages)}
    step_ev = [ev[0].elapsed_time(ev[-1]) for ev in events]
    aa = [mk() for _ in range(args.steps)]
    for k in range(args.steps):
        step(aa[k])
    torch.cuda.synchronize()
    aa_ev = [ev[0].elapsed_time(ev[-1]) for ev in aa]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = [mk() for _ in range(args.steps)]
    for k in range(args.steps):
        flush.fill_(k & 0xFF)
        step(cold[k])
    torch.cuda.synchronize()
    cold_ev = [ev[0].elapsed_time(ev[-1]) for ev in cold]
    del flush
    return elapsed, stage_ms, step_ev, cold_ev, aa_ev


TRAIN_METRIC = "training grouped GEMM rows/s (forward + dgrad + fp32 wgrad accumulate); TFLOP/s vs MFMA peak"


def main_train(args):
    """A training step of one MoE projection ([DET]): the ragged grouped
    forward, dgrad and wgrad with the fp32 accumulate into main_grad, through
    the C ABI on one stream."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import mixture_experts_expert_align_amd as moe

    cfg = mi.train_config(args.config)
    dev = "cuda"
    torch.cuda.init()
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    ti = mi.make_train_inputs(cfg, device=dev)
    off = torch.from_numpy(ti.offsets).to(dev)
    R = int(ti.offsets[-1])
    y = torch.empty((R, cfg.N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((R, cfg.K), dtype=torch.bfloat16, device=dev)
    main_grad = ti.main_grad
    stream = torch.cuda.current_stream()
    stages = ["forward", "dgrad", "wgrad_acc"]

    def step(ev):
        ev[0].record(stream)
        moe.moe_grouped_forward(ti.x, ti.w, off, y, stream)
        ev[1].record(stream)
        moe.moe_grouped_dgrad(ti.dy, ti.w, off, dx, stream)
        ev[2].record(stream)
        moe.moe_grouped_wgrad(ti.dy, ti.x, off, main_grad, accumulate=True, stream=stream)
        ev[3].record(stream)

    elapsed, stage_ms, step_ev, cold_ev, aa_ev = time_steps(step, stages, args, dev)
    ms_per_step = elapsed * 1e3 / args.steps
    flops = 2.0 * R * cfg.N * cfg.K           # per GEMM
    tf = {s: round(flops / (stage_ms[s] * 1e-3) / 1e12, 1) for s in stages}
    short = "_".join(cfg.name.split("_")[:2])
    # the accumulating wgrad: dy and x read once, main_grad read and written
    # in fp32; its bound is whichever roof is lower at this intensity
    dom = "wgrad_acc"
    t_dom = stage_ms[dom] * 1e-3
    alg_bytes = R * (cfg.N + cfg.K) * 2 + 2 * cfg.E * cfg.N * cfg.K * 4
    if flops / alg_bytes > (PEAK_TFLOPS["bf16"] * 1e12) / (PEAK_HBM_GBS * 1e9):
        achieved = flops / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS["bf16"], 4)}
    else:
        achieved = alg_bytes / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof.update({"kernel": dom, "kernel_ms": round(stage_ms[dom], 4),
                 "algorithmic_per_launch": {"flops": int(flops), "bytes": int(alg_bytes)},
                 "traffic": traffic_record(short, KERNEL_FILES[short]) if short in KERNEL_FILES else None})
    cpu = None if args.no_cpu_baseline else cpu_baseline_train(cfg, ti, args.cpu_seconds)
    rec = {
        "metric": TRAIN_METRIC, "value": round(R * args.steps / elapsed, 2), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; random-init expert weights)",
        "config": {"workload": cfg.name, "E": cfg.E, "N": cfg.N, "K": cfg.K, "rows": R,
                   "groups": cfg.balance, "accumulate": "fp32 main_grad, in the kernel"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_TFLOPs": tf,
        "step_event_ms": pct(step_ev), "step_event_ms_cache_flushed": pct(cold_ev),
        "noise": noise(step_ev, aa_ev),
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline_train(cfg, ti, min_seconds):
    """The oracle's forward, dgrad and wgrad on one group's rows (the
    lightest non-empty group), repeated to about ``min_seconds``: rows/s."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    sizes = np.diff(ti.offsets)
    e = int(np.argmin(np.where(sizes > 0, sizes, 1 << 30)))
    a, b = int(ti.offsets[e]), int(ti.offsets[e + 1])
    x = ti.x[a:b].float().cpu().numpy().astype(np.float64)
    dy = ti.dy[a:b].float().cpu().numpy().astype(np.float64)
    w = ti.w[e:e + 1].float().cpu().numpy().astype(np.float64)
    off = np.array([0, b - a])
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.grouped_forward(x, w, off)
        oracle.grouped_dgrad(dy, w, off)
        oracle.grouped_wgrad(dy, x, off)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round((b - a) * reps / dt, 4), "unit": "rows/s", "cores": int(blas_threads),
            "kind": "oracle", "sample": f"group {e} ({b - a} rows, N={cfg.N}, K={cfg.K}), {reps} passes",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_baseline(cfg, inp, w1, w2, w_f32, sample, min_seconds):
    """The oracle, as it stands, on a bounded sample, repeated until about
    ``min_seconds`` of CPU time: its rate in the same unit (tokens/s)."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    if cfg.layout == "contiguous":
        n = sample or {"tiny": 64, "decode": 4, "prefill": 2, "mxfp8": 4}.get(cfg.name.split("_")[0], 1)
        ids = inp.topk_ids
        valid = (ids >= 0) & (ids < cfg.E)
        cand = np.flatnonzero(valid.any(axis=1))
        tokens = cand[:n]
        experts = sorted({int(e) for e in ids[tokens][valid[tokens]]})
        # stage host copies of the inputs (not timed): raw bf16 bits or float32
        if w_f32 is not None:
            # the oracle's own codec encodes the float32 weights once, before
            # the timed loop (the GPU path too gets its weights encoded); the
            # timed oracle decodes them, as it decodes bf16 weights
            host = {e: (oracle.mxfp8_quantize(w_f32[0][e].cpu().numpy()),
                        oracle.mxfp8_quantize(w_f32[1][e].cpu().numpy())) for e in experts}
            dec = lambda cs: oracle.mxfp8_dequantize(*cs)
        else:
            host = {e: (mi.bf16_bits(inp.w1[e]), mi.bf16_bits(inp.w2[e])) for e in experts}
            dec = oracle.bf16_to_f64
        x = mi.bf16_bits(inp.x[torch.from_numpy(tokens).cuda()])
        reps = 0
        t0 = time.perf_counter()
        while True:
            xr = oracle.bf16_to_f64(x)
            oracle.moe_contiguous(xr, tokens, ids, inp.topk_weights, cfg.E, lambda e: dec(host[e][0]),
                                  lambda e: dec(host[e][1]), cfg.w1_order)
            reps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
        what = (f"{len(tokens)} tokens ({int(valid[tokens].sum())} routes over {len(experts)} experts), "
                f"{reps} passes")
        units = len(tokens) * reps
    else:
        counts = inp.expert_num_tokens
        n = sample or 2
        es = [int(e) for e in np.argsort(counts)[:n] if counts[e] > 0]   # the lightest experts
        host = {e: (mi.bf16_bits(inp.w1[e]), mi.bf16_bits(inp.w2[e]),
                    mi.bf16_bits(inp.a[e][: counts[e]])) for e in es}
        t0 = time.perf_counter()
        rows = 0
        while True:
            for e in es:
                oracle.expert_ffn(oracle.bf16_to_f64(host[e][2]), oracle.bf16_to_f64(host[e][0]),
                                  oracle.bf16_to_f64(host[e][1]))
                rows += int(counts[e])
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
        what = f"{rows} batched rows of experts {es} (out tokens/s scaled by 512 tokens / V rows)"
        units = rows * cfg.M / max(1, int(counts.sum()))
    return {"value": round(units / dt, 4), "unit": "tokens/s", "cores": int(blas_threads),
            "kind": "oracle", "sample": what, "seconds": round(dt, 2),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
