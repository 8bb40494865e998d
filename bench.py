#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload deepseek_v3_bf16]

One step = one moe_forward call over the whole batch (router linear, top-k,
dispatch, gate_up + SwiGLU grouped GEMM, down grouped GEMM, shared expert,
combine) with inputs and weights already resident in HBM.  Before every step
(warm-up and timed) an untimed 512 MiB scratch write evicts the last-level cache;
each step is bracketed by HIP events on the library's stream and the median
step is reported.  Prints one JSON line: tokens/s for the workload, the roofline
of the dominant kernel (its launches timed live between the events that
moe_forward_staged records around the very launches moe_forward makes), the
routed and shared phases against their own rooflines, and the CPU oracle timed
on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "MoE-layer fwd tokens/sec on 1 MI355X; % of MFMA bf16 / HBM peak"
# sources of the grouped-GEMM kernels: counter records are used only while these are unchanged
GEMM_SOURCES = ["sparse_mixture_experts_level_amd/csrc/gemm_stream.hip",
                "sparse_mixture_experts_level_amd/csrc/gemm_big.hip",
                "sparse_mixture_experts_level_amd/csrc/common.hpp"]
# the largest configuration that fits one GPU
DEFAULT_WORKLOAD = "deepseek_v3_bf16"
CPU_SAMPLE = {"tiny_f32": 64, "switch_bf16": 8192, "mixtral_bf16": 64, "gptoss_decode_bf16": 16,
              "deepseek_v3_bf16": 16}


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--flush-mib", type=int, default=512,
                   help="untimed scratch write before every step, in MiB (0: none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=0, help="tokens in the oracle's sample (0: pick by workload)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="after the run, copy a buffer of this many MiB three times (a kernel of known traffic for "
                        "scaling hardware byte counters)")
    p.add_argument("--backward", action="store_true",
                   help="time the layer's backward pass (moe_backward, routing from one forward) instead of the "
                        "forward")
    p.add_argument("--tiled", choices=("auto", "on", "off"), default="auto",
                   help="tile-major copies of the routed (shared) expert weights, prepared once before timing "
                        "(auto: when the routed experts (the shared expert) take the large-tile regime)")
    p.add_argument("--zero-expert-weights", action="store_true",
                   help="diagnostic: the routed and shared expert weights all zero (routing unchanged, every kernel "
                        "still runs on the same shapes), to show how the matrix cores' clock depends on operand "
                        "values; not a throughput figure")
    p.add_argument("--ep-shards", type=int, default=1, metavar="N",
                   help="time one expert-parallel rank's share instead of the whole layer: experts split in N "
                        "contiguous ranges, every range timed on this GPU, the slowest one reported")
    return p.parse_args(argv)


def device_info(torch) -> dict:
    """The GPU the line was measured on, as the runtime reports it (and rocminfo's maximum
    engine clock of the first gfx950 agent, when rocminfo is there)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "max_clock_mhz": None}
    try:
        import subprocess
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        agent = txt[txt.index("gfx950"):] if "gfx950" in txt else ""
        for line in agent.splitlines():
            if "Max Clock Freq" in line:
                info["max_clock_mhz"] = int(line.split(":")[1].split()[0])
                break
    except Exception:  # the clock is context only
        pass
    return info


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def weight_layout(args):
    which = [n for n, on in (("routed", args.use_tiles), ("shared", args.use_shared_tiles)) if on]
    if not which:
        return "row-major"
    return f"row-major plus tile-major copies of the {' and '.join(which)} expert weights, prepared once before timing"


def big_regime(rows_max, groups, group_rows_max):
    """The library's regime rule: groups averaging >= 256 rows that can reach 256 rows run on
    the large-tile kernel, the others on the streaming one."""
    return groups > 0 and rows_max // groups >= 256 and group_rows_max >= 256


def tail_rows(rows, n_out_min):
    """Rows the large-tile launch leaves to its tail launch: a group's last partial 256-row tile
    of at most 128 rows, when the tail launch (groups x 64-column tiles) reaches 512 workgroups."""
    if len(rows) * ((n_out_min + 63) // 64) < 512:
        return 0
    return int(sum(r % 256 for r in rows if 0 < r % 256 <= 128))


def stage_work(w, R, E_t, kept, T, s_bytes, cap, rmax):
    """Algorithmic bytes and FLOP of the main launch of each GEMM stage (what the method must
    move and compute: touched weights once, activation rows read once, outputs written once)."""
    d, f, fs, E = w.d_model, w.d_ff, w.d_ff_shared, w.num_experts
    grm = T if cap is None else min(T, cap)
    work = {}
    routed_big = w.dtype == "bf16" and big_regime(rmax, E, grm)
    Rm = R - (tail_rows(kept, min(d, f)) if routed_big else 0)
    work["gate_up"] = {"bytes": s_bytes * (E_t * 2 * f * d + Rm * d + Rm * f), "flop": 4.0 * Rm * d * f,
                       "kernel": "grouped_gemm_big_kernel (gate_up + SwiGLU)" if routed_big
                       else "grouped_gemm_stream_kernel (gate_up + SwiGLU)"}
    work["down"] = {"bytes": s_bytes * (E_t * d * f + Rm * f + Rm * d), "flop": 2.0 * Rm * d * f,
                    "kernel": "grouped_gemm_big_kernel (down)" if routed_big else "grouped_gemm_stream_kernel (down)"}
    if fs:
        sh_big = w.dtype == "bf16" and big_regime(T, 1, T)
        Ts = T - (tail_rows([T], min(d, fs)) if sh_big else 0)
        kind = "grouped_gemm_big_kernel" if sh_big else "grouped_gemm_stream_kernel"
        work["shared_gate_up"] = {"bytes": s_bytes * (2 * fs * d + Ts * d + Ts * fs), "flop": 4.0 * Ts * d * fs,
                                  "kernel": f"{kind} (shared expert gate_up + SwiGLU)"}
        work["shared_down"] = {"bytes": s_bytes * (d * fs + Ts * fs + Ts * d), "flop": 2.0 * Ts * d * fs,
                               "kernel": f"{kind} (shared expert down)"}
    return work


def roofline_of(work, dur_us, s_bytes):
    """Bound by the kernel's own intensity against the ridge (peak FLOP/s / peak bytes/s)."""
    peak_flops = (MFMA_BF16_PEAK_TFLOPS if s_bytes == 2 else MFMA_F32_PEAK_TFLOPS) * 1e12
    ridge = peak_flops / (HBM_PEAK_GBS * 1e9)
    if work["flop"] / work["bytes"] < ridge:
        achieved = work["bytes"] / (dur_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = work["flop"] / (dur_us * 1e-6) / 1e12
    peak = peak_flops / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4)}


def counter_traffic(workload, stage):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE record of this
    kernel on this workload, while the GEMM sources are those the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        tj = json.load(fh)
    if tj.get("source_hash") != source_hash(GEMM_SOURCES):
        return None
    return tj.get("hbm_bytes_per_launch")


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this build runs the layer on a "
              f"single MI355X and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_mixture_experts_level_amd.ops as ops
    from sparse_mixture_experts_level_amd import workloads as wl

    dev = "cuda"
    w = wl.get_workload(args.workload)
    print(f"[bench] {w.name}: drawing inputs", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, seed=args.seed, device=dev)
    if args.zero_expert_weights:
        for t in (inp.w_gate_up, inp.w_down, inp.w_shared_gate_up, inp.w_shared_down):
            if t is not None:
                t.zero_()
    cap = ops.moe_capacity(w.num_tokens, w.num_experts, w.capacity_factor)
    T, d, E, k, f, fs = w.num_tokens, w.d_model, w.num_experts, w.top_k, w.d_ff, w.d_ff_shared
    desc = ops.make_desc(T, d, f, E, k, cap, fs, w.torch_dtype)
    rmax = ops.moe_max_rows(desc)
    large_tiles = big_regime(rmax, E, T if cap is None else min(T, cap))
    args.use_tiles = w.dtype == "bf16" and (args.tiled == "on" or (args.tiled == "auto" and large_tiles))
    # the shared expert, one group of all T tokens, takes the large-tile regime from 256 tokens
    args.use_shared_tiles = w.dtype == "bf16" and fs > 0 and (args.tiled == "on" or (args.tiled == "auto" and T >= 256))
    layer = ops.MoELayer(inp, cap, device=dev, tiled=args.use_tiles, shared_tiled=args.use_shared_tiles)
    s_bytes = 2 if w.dtype == "bf16" else 4
    if args.ep_shards > 1:
        return ep_share_bench(args, w, inp, cap, layer, s_bytes)
    if args.backward:
        return backward_bench(args, w, inp, cap, layer, s_bytes)

    scratch = torch.empty(max(args.flush_mib, 1) << 20, dtype=torch.uint8, device=dev)

    def flush(i):
        if args.flush_mib:
            scratch.fill_(i & 0xFF)  # untimed: evicts x and the weights from the last-level cache

    # ---------------------------------------------------------------- whole-layer timing
    for i in range(args.warmup):
        flush(i)
        layer.forward(with_routing=False)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: timing {args.steps} steps", file=sys.stderr, flush=True)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(marks):
        flush(i)
        a.record()
        layer.forward(with_routing=False)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in marks]
    ms_per_step = statistics.median(step_ms)
    tokens_per_s = T / (ms_per_step * 1e-3)

    # ---------------------------------------------------------------- routing facts of this batch
    layer.forward(with_routing=True)
    torch.cuda.synchronize()
    off = layer.routing["expert_offsets"].cpu().numpy().astype(np.int64)
    kept = np.diff(off)
    R = int(off[-1])
    E_t = int((kept > 0).sum())

    # ---------------------------------------------------------------- per-stage timing of moe_forward's own launches
    evsets = [ops.stage_events() for _ in range(args.steps)]
    for i, evs in enumerate(evsets):
        flush(i)
        layer.forward_staged(evs)
    torch.cuda.synchronize()
    per_stage = {s: [] for s in ops.STAGES}
    for evs in evsets:
        for i, s in enumerate(ops.STAGES):
            per_stage[s].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)  # us
    stage_us = {s: statistics.median(v) for s, v in per_stage.items()}

    # ---------------------------------------------------------------- roofline of the dominant kernel
    work = stage_work(w, R, E_t, kept.tolist(), T, s_bytes, cap, rmax)
    dom = max(work, key=lambda s: stage_us[s])
    roofline = roofline_of(work[dom], stage_us[dom], s_bytes)
    roofline.update({"kernel": work[dom]["kernel"], "stage": dom, "avg_launch_us": round(stage_us[dom], 2),
                     "launch_us_statistic": "median over the timed steps",
                     "algorithmic_bytes": int(work[dom]["bytes"]), "algorithmic_flop": int(work[dom]["flop"]),
                     "traffic": counter_traffic(w.name, dom)})
    kernels = {}
    for s, wk in work.items():
        if stage_us[s] > 0:
            r = roofline_of(wk, stage_us[s], s_bytes)
            kernels[s] = {"us": round(stage_us[s], 2), "bound": r["bound"], "achieved": r["achieved"],
                          "unit": r["unit"], "frac": r["frac"]}

    # ---------------------------------------------------------------- whole layer and its phases
    def rt(flop, nbytes):
        return max(flop / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)) * 1e3  # ms

    flop = 2.0 * T * d * E + 6.0 * R * d * f + 6.0 * T * d * fs
    layer_bytes = s_bytes * (T * d + E * d + E_t * 3 * d * f + 3 * d * fs + T * d)
    layer_rt = rt(flop, layer_bytes)
    layer_roofline = {"algorithmic_flop": flop, "algorithmic_bytes": layer_bytes, "roofline_ms": round(layer_rt, 4),
                      "frac_of_roofline": round(layer_rt / ms_per_step, 4),
                      "hbm_frac": round(layer_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                      "mfma_frac": round(flop / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)}
    phases = None
    if fs:
        shared_st = [s for s in ops.STAGES if s.startswith("shared_")]
        routed_st = [s for s in ops.STAGES if s not in shared_st]
        r_flop, r_bytes = 2.0 * T * d * E + 6.0 * R * d * f, s_bytes * (T * d + E * d + E_t * 3 * d * f + T * d)
        s_flop, s_bytes_ = 6.0 * T * d * fs, s_bytes * 3 * d * fs
        r_ms = sum(stage_us[s] for s in routed_st) / 1e3
        s_ms = sum(stage_us[s] for s in shared_st) / 1e3
        r_rt, s_rt = rt(r_flop, r_bytes), rt(s_flop, s_bytes_)
        phases = {
            "routed": {"stages": routed_st, "ms": round(r_ms, 4), "bound": "hbm" if r_flop / r_bytes < 312.5 else "mfma",
                       "roofline_ms": round(r_rt, 4), "frac_of_roofline": round(r_rt / r_ms, 4),
                       "algorithmic_bytes": r_bytes, "algorithmic_flop": r_flop},
            "shared": {"stages": shared_st, "ms": round(s_ms, 4), "bound": "hbm" if s_flop / s_bytes_ < 312.5 else "mfma",
                       "roofline_ms": round(s_rt, 4), "frac_of_roofline": round(s_rt / s_ms, 4),
                       "algorithmic_bytes": s_bytes_, "algorithmic_flop": s_flop},
            "phase_sum_roofline_ms": round(r_rt + s_rt, 4), "overlapped_roofline_ms": round(layer_rt, 4),
            "step_frac_of_phase_sum_roofline": round((r_rt + s_rt) / ms_per_step, 4),
        }

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] {w.name}: CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, cap, args.cpu_sample)

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic, expert weights all zero (diagnostic, not a throughput figure)" if args.zero_expert_weights
                else "synthetic",
        "config": {"workload": w.name, "description": w.description, "num_tokens": T, "d_model": d,
                   "num_experts": E, "top_k": k, "d_ff": f, "d_ff_shared": fs, "capacity": cap,
                   "kept_rows": R, "experts_touched": E_t, "drops": int(T * k - R),
                   "weight_layout": weight_layout(args)},
        "timing": {"statistic": "median", "step_ms_min": round(min(step_ms), 4), "step_ms_max": round(max(step_ms), 4),
                   "step_ms_mean": round(statistics.mean(step_ms), 4),
                   "wall_ms_per_step_with_flush": round(wall * 1e3 / args.steps, 4),
                   "method": f"HIP events around each moe_forward on the library's stream; an untimed "
                             f"{args.flush_mib} MiB scratch write before every step"},
        "roofline": roofline,
        "kernels": kernels,
        "layer_roofline": layer_roofline,
        "phases": phases,
        "stage_us": {s: round(v, 2) for s, v in stage_us.items()},
        "cpu_baseline": cpu,
        "device": device_info(torch),
    }
    print(json.dumps(line), flush=True)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


def ep_share_bench(args, w, inp, cap, layer, s_bytes):
    """One rank's share of expert parallelism at the layer's real shapes: every rank runs the
    router, top-k and dispatch for all T tokens and the FFN of its E/N experts (rank 0 also the
    shared expert), writing a partial output that an all-reduce would sum.  Each rank's share is
    timed here in turn on the one GPU; a step of N ranks takes as long as the slowest share plus
    the all-reduce, which is not part of this measurement."""
    import numpy as np
    import torch

    import sparse_mixture_experts_level_amd.ops as ops

    T, d, E, f, fs = w.num_tokens, w.d_model, w.num_experts, w.d_ff, w.d_ff_shared
    N = args.ep_shards
    if E % N:
        print(f"--ep-shards {N} does not divide the {E} experts", file=sys.stderr)
        sys.exit(2)
    per = E // N
    part = torch.empty_like(inp.x)
    layer.forward(with_routing=True)
    torch.cuda.synchronize()
    kept = np.diff(layer.routing["expert_offsets"].cpu().numpy().astype(np.int64))

    # each rank's tile-major copies of its own experts, prepared once
    tiles = [ops.tiled_weights(layer.desc, inp.w_gate_up[r * per:(r + 1) * per], inp.w_down[r * per:(r + 1) * per])
             if args.use_tiles else None for r in range(N)]

    def share(r):
        b, e = r * per, (r + 1) * per
        ops.moe_forward_expert_shard(layer.desc, inp.w_router, inp.w_gate_up[b:e], inp.w_down[b:e], b, e, r == 0,
                                     inp.x, inp.logit_offset, part, layer.ws, w_shared_gate_up=inp.w_shared_gate_up,
                                     w_shared_down=inp.w_shared_down, tiled=tiles[r],
                                     shared_tiled=layer.shared_tiled if r == 0 else None)

    ranks = []
    for r in range(N):
        for _ in range(args.warmup):
            share(r)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            share(r)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        loc = kept[r * per:(r + 1) * per]
        R_r, Et_r = int(loc.sum()), int((loc > 0).sum())
        fs_r = fs if r == 0 else 0
        flop = 2.0 * T * d * E + 6.0 * R_r * d * f + 6.0 * T * d * fs_r
        nbytes = s_bytes * (T * d + E * d + Et_r * 3 * d * f + 3 * d * fs_r + T * d)
        rt = max(flop / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9))
        ranks.append({"rank": r, "experts": [r * per, (r + 1) * per], "ms": round(ms, 4), "kept_rows": R_r,
                      "experts_touched": Et_r, "shared": bool(fs_r), "roofline_ms": round(rt * 1e3, 4),
                      "frac_of_roofline": round(rt * 1e3 / ms, 4)})
    slow = max(ranks, key=lambda x: x["ms"])
    line = {
        "metric": METRIC,
        "value": round(T / (slow["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": slow["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}, one rank's share of {N}-way expert parallelism (slowest rank)",
                   "num_tokens": T, "d_model": d, "num_experts": E, "top_k": w.top_k, "d_ff": f, "d_ff_shared": fs,
                   "capacity": cap, "ep_shards": N, "experts_per_rank": per,
                   "weight_layout": weight_layout(args)},
        "ranks": ranks,
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def backward_bench(args, w, inp, cap, layer, s_bytes):
    """The backward pass alone: gradients of sum(dy * out) with respect to x and every
    weight, for the routing of one forward pass of the same batch."""
    import numpy as np
    import torch

    import sparse_mixture_experts_level_amd.ops as ops

    dev = "cuda"
    T, d, E, k, f, fs = w.num_tokens, w.d_model, w.num_experts, w.top_k, w.d_ff, w.d_ff_shared
    if w.dtype != "bf16":
        print("the backward pass is implemented for bf16 layers", file=sys.stderr)
        sys.exit(2)
    layer.forward(with_routing=True)
    torch.cuda.synchronize()
    kept = np.diff(layer.routing["expert_offsets"].cpu().numpy().astype(np.int64))
    R, E_t = int(kept.sum()), int((kept > 0).sum())
    g = torch.Generator(device=dev).manual_seed(args.seed + 1)
    dy = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    dx = torch.empty_like(dy)
    grads = {"dw_router": torch.empty((E, d), dtype=torch.float32, device=dev),
             "dw_gate_up": torch.empty((E, 2 * f, d), dtype=torch.bfloat16, device=dev),
             "dw_down": torch.empty((E, d, f), dtype=torch.bfloat16, device=dev)}
    if fs:
        grads["dw_shared_gate_up"] = torch.empty((2 * fs, d), dtype=torch.bfloat16, device=dev)
        grads["dw_shared_down"] = torch.empty((d, fs), dtype=torch.bfloat16, device=dev)
    ws = ops.workspace(ops.moe_backward_workspace_size(layer.desc), dev)

    def step():
        ops.moe_backward(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, layer.routing, dy, dx, grads, ws,
                         w_shared_gate_up=inp.w_shared_gate_up, w_shared_down=inp.w_shared_down, tiled=layer.tiled,
                         shared_tiled=layer.shared_tiled)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # algorithmic work: recompute of G|U, dH', dx rows, dW_gate_up, dW_down (16 R d f), the
    # router (4 T E d) and the shared expert (16 T d f_s); bytes: touched experts' weights read
    # once, every weight gradient written once, x, dy read and dx written
    flop = 16.0 * R * d * f + 4.0 * T * E * d + 16.0 * T * d * fs
    nbytes = s_bytes * (E_t * 3 * d * f + E * 3 * d * f + 6 * d * fs + 3 * T * d) + E * d * (s_bytes + 4)
    rt = max(flop / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9))
    line = {
        "metric": "MoE-layer backward tokens/sec on 1 MI355X",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}, backward pass", "num_tokens": T, "d_model": d, "num_experts": E,
                   "top_k": k, "d_ff": f, "d_ff_shared": fs, "capacity": cap, "kept_rows": R,
                   "experts_touched": E_t, "weight_layout": weight_layout(args)},
        "layer_roofline": {"algorithmic_flop": flop, "algorithmic_bytes": nbytes, "roofline_ms": round(rt * 1e3, 4),
                           "frac_of_roofline": round(rt * 1e3 / ms, 4)},
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(inp, cap, sample, min_seconds=10.0):
    """The CPU oracle as it stands, on a bounded sample: routing over the whole batch,
    expert FFN and combine for `sample` tokens.  Expert weights are copied to the host
    before the clock starts; their float64 conversion inside the oracle is timed."""
    import numpy as np
    import torch

    import oracle

    w = inp.workload
    sample = sample or CPU_SAMPLE.get(w.name, 64)
    sample = min(sample, w.num_tokens)
    h = lambda t: None if t is None else t.float().cpu().numpy()
    x, wr, off = h(inp.x), h(inp.w_router), h(inp.logit_offset)
    tokens = np.sort(np.random.default_rng(0).choice(w.num_tokens, sample, replace=False))
    # experts the sample can reach (host copies, untimed)
    ids = oracle.topk_select(oracle.router_logits(x, wr, off), w.top_k)
    need = sorted(set(ids[tokens].reshape(-1).tolist()))
    gu = {e: h(inp.w_gate_up[e]) for e in need}
    dn = {e: h(inp.w_down[e]) for e in need}
    sgu, sd = h(inp.w_shared_gate_up), h(inp.w_shared_down)
    torch.cuda.synchronize()
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    reps, done = 0, 0
    t0 = time.perf_counter()
    while True:  # whole passes over the sample until at least `min_seconds` of CPU work
        oracle.moe_forward(x, wr, gu, dn, w.top_k, cap, off, w_shared_gate_up=sgu, w_shared_down=sd, tokens=tokens)
        reps += 1
        done += sample
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} pass(es) over {sample} of {w.num_tokens} tokens (routing and capacity fill over all "
                      f"{w.num_tokens}; expert FFN and combine for the sample), {dt:.1f} s, NumPy float64",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
