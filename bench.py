#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload switch_bf16]

One step = one moe_forward call over the whole batch (router linear, top-k,
dispatch, gate_up + SwiGLU grouped GEMM, down grouped GEMM, combine) with inputs
and weights already resident in HBM.  Prints one JSON line: tokens/s for the
workload, the roofline of the dominant kernel (timed live with HIP events on the
library's stream), and the CPU oracle timed on a bounded sample on this host.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "MoE-layer fwd tokens/sec on 1 MI355X; % of MFMA bf16 / HBM peak"
DOMINANT_SOURCES = ["sparse_mixture_experts_level_amd/csrc/gemm_stream.hip",
                    "sparse_mixture_experts_level_amd/csrc/common.hpp"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="switch_bf16")
    p.add_argument("--seed", type=int, default=0)
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
    p.add_argument("--ep-shards", type=int, default=1, metavar="N",
                   help="time one expert-parallel rank's share instead of the whole layer: experts split in N "
                        "contiguous ranges, every range timed on this GPU, the slowest one reported")
    return p.parse_args()


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


def main():
    args = parse()
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
    inp = wl.make_inputs(w, seed=args.seed, device=dev)
    cap = ops.moe_capacity(w.num_tokens, w.num_experts, w.capacity_factor)
    T, d, E, k, f, fs = w.num_tokens, w.d_model, w.num_experts, w.top_k, w.d_ff, w.d_ff_shared
    # The library's regime rule: groups averaging >= 256 rows (R_max / E) that can reach 256
    # rows (min(T, C)) run on the large-tile kernel, which reads tile-major copies when given.
    desc = ops.make_desc(T, d, f, E, k, cap, fs, w.torch_dtype)
    large_tiles = ops.moe_max_rows(desc) // E >= 256 and (T if cap is None else min(T, cap)) >= 256
    args.use_tiles = w.dtype == "bf16" and (args.tiled == "on" or (args.tiled == "auto" and large_tiles))
    # the shared expert, one group of all T tokens, takes the large-tile regime from 256 tokens
    args.use_shared_tiles = w.dtype == "bf16" and fs > 0 and (args.tiled == "on" or (args.tiled == "auto" and T >= 256))
    layer = ops.MoELayer(inp, cap, device=dev, tiled=args.use_tiles, shared_tiled=args.use_shared_tiles)
    s_bytes = 2 if w.dtype == "bf16" else 4
    if args.ep_shards > 1:
        return ep_share_bench(args, w, inp, cap, layer, s_bytes)
    if args.backward:
        return backward_bench(args, w, inp, cap, layer, s_bytes)

    # ---------------------------------------------------------------- whole-path timing
    for _ in range(args.warmup):
        layer.forward(with_routing=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(with_routing=False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = T * args.steps / (t1 - t0)

    # ---------------------------------------------------------------- routing facts of this batch
    layer.forward(with_routing=True)
    torch.cuda.synchronize()
    off = layer.routing["expert_offsets"].cpu().numpy().astype(np.int64)
    kept = np.diff(off)
    R = int(off[-1])
    E_t = int((kept > 0).sum())

    # ---------------------------------------------------------------- per-stage HIP-event timing
    # The same kernels as moe_forward, called stage by stage through the C ABI, with events on
    # the stream the library launches on (torch's current stream).  As in moe_forward, the
    # gate_up projection gathers token rows from x through row_token (no x_perm).
    r = layer.routing
    desc = layer.desc
    Rmax = ops.moe_max_rows(desc)
    hid = torch.empty((max(Rmax, 1), f), dtype=inp.x.dtype, device=dev)
    y_perm = torch.empty((max(Rmax, 1), d), dtype=inp.x.dtype, device=dev)
    out = torch.empty_like(inp.x)
    grm = max(1, min(T, cap) if cap is not None else T)
    stages = ["router_logits", "router_topk", "dispatch_permute", "gate_up_swiglu", "down", "combine"]
    ev = {s: [] for s in stages}

    def staged_step(record):
        marks = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                marks.append(e)

        mark()
        ops.moe_router_logits(desc, inp.x, inp.w_router, inp.logit_offset, r["logits"])
        mark()
        ops.moe_router_topk(desc, r["logits"], r["topk_ids"], r["topk_gates"])
        mark()
        ops.moe_dispatch_permute(desc, r["topk_ids"], None, r["expert_counts"], r["expert_offsets"], r["slot"],
                                 r["row_token"], None, layer.ws)
        mark()
        ops.moe_grouped_gate_up_swiglu(E, Rmax, grm, d, f, inp.x.dtype, inp.x, r["expert_offsets"], inp.w_gate_up,
                                       hid, row_index=r["row_token"])
        mark()
        ops.moe_grouped_down(E, Rmax, grm, d, f, inp.x.dtype, hid, r["expert_offsets"], inp.w_down, y_perm)
        mark()
        ops.moe_combine_unpermute(desc, y_perm, r["topk_ids"], r["topk_gates"], r["slot"], r["expert_offsets"], None,
                                  out)
        mark()
        return marks

    if fs:
        # the shared expert: the same grouped GEMMs with one group of all T tokens
        stages += ["shared_gate_up", "shared_down"]
        ev.update({"shared_gate_up": [], "shared_down": []})
        sh_off = torch.tensor([0, T], dtype=torch.int32, device=dev)
        sh_hid = torch.empty((T, fs), dtype=inp.x.dtype, device=dev)
        sh_out = torch.empty_like(inp.x)

    def staged_shared(marks, record):
        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                marks.append(e)
        ops.moe_grouped_gate_up_swiglu(1, T, T, d, fs, inp.x.dtype, inp.x, sh_off, inp.w_shared_gate_up, sh_hid)
        mark()
        ops.moe_grouped_down(1, T, T, d, fs, inp.x.dtype, sh_hid, sh_off, inp.w_shared_down, sh_out)
        mark()

    for _ in range(args.warmup):
        m = staged_step(False)
        if fs:
            staged_shared(m, False)
    all_marks = []
    for _ in range(args.steps):
        m = staged_step(True)
        if fs:
            staged_shared(m, True)
        all_marks.append(m)
    torch.cuda.synchronize()
    for marks in all_marks:
        for i, s in enumerate(stages):
            ev[s].append(marks[i].elapsed_time(marks[i + 1]) * 1e3)  # us
    stage_us = {s: float(np.mean(v)) for s, v in ev.items()}

    # ---------------------------------------------------------------- roofline of the dominant kernel
    gate_up_bytes = E_t * 2 * f * d * s_bytes + R * d * s_bytes + R * f * s_bytes
    gate_up_flop = 2.0 * R * d * 2 * f
    down_bytes = E_t * d * f * s_bytes + R * f * s_bytes + R * d * s_bytes
    dom = "gate_up_swiglu"
    dur = stage_us.get(dom)
    roofline = None
    if dur:
        intensity = gate_up_flop / gate_up_bytes
        peak_flops = (MFMA_BF16_PEAK_TFLOPS if s_bytes == 2 else MFMA_F32_PEAK_TFLOPS) * 1e12
        ridge = peak_flops / (HBM_PEAK_GBS * 1e9)
        if intensity < ridge:
            achieved = gate_up_bytes / (dur * 1e-6) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4)}
        else:
            achieved = gate_up_flop / (dur * 1e-6) / 1e12
            peak = peak_flops / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(achieved / peak, 4)}
        roofline["kernel"] = "grouped_gemm_stream_kernel (gate_up + SwiGLU)" if grm <= 512 else "grouped gate_up GEMM"
        roofline["avg_launch_us"] = round(dur, 2)
        roofline["algorithmic_bytes"] = int(gate_up_bytes)
        roofline["algorithmic_flop"] = int(gate_up_flop)
        traffic = None
        tfile = os.path.join(ROOT, "profiles", f"traffic_gate_up_{args.workload}.json")
        if os.path.exists(tfile):
            with open(tfile) as fh:
                tj = json.load(fh)
            if tj.get("source_hash") == source_hash(DOMINANT_SOURCES):
                traffic = tj.get("hbm_bytes_per_launch")
        roofline["traffic"] = traffic

    # whole-layer algorithmic work (for context next to the kernel roofline)
    flop = 2.0 * T * d * E + 6.0 * R * d * f + 6.0 * T * d * fs
    layer_bytes = s_bytes * (T * d + E * d + E_t * 3 * d * f + 3 * d * fs + T * d)
    rt = max(flop / (MFMA_BF16_PEAK_TFLOPS * 1e12), layer_bytes / (HBM_PEAK_GBS * 1e9))
    layer_roofline = {"algorithmic_flop": flop, "algorithmic_bytes": layer_bytes, "roofline_ms": round(rt * 1e3, 4),
                      "frac_of_roofline": round(rt * 1e3 / ms_per_step, 4),
                      "hbm_frac": round(layer_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                      "mfma_frac": round(flop / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)}

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
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
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "num_tokens": T, "d_model": d,
                   "num_experts": E, "top_k": k, "d_ff": f, "d_ff_shared": fs, "capacity": cap,
                   "kept_rows": R, "experts_touched": E_t, "drops": int(T * k - R),
                   "weight_layout": weight_layout(args)},
        "roofline": roofline,
        "layer_roofline": layer_roofline,
        "stage_us": {s: round(v, 2) for s, v in stage_us.items()},
        "cpu_baseline": cpu,
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
    sample = sample or {"switch_bf16": w.num_tokens, "tiny_f32": w.num_tokens}.get(w.name, 64)
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
