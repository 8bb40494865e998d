"""GPU parity of moe_backward against the oracle's chain-rule backward (float64), through
the C ABI.  The forward runs on the GPU; the oracle then differentiates the same layer
with the GPU's routing (ids), so near-tie routing differences cannot enter.

Tolerance: row-normalised max relative error 2e-2 (bf16 layers, as for the forward) on
dx and on every weight-gradient matrix (rows of dW_gate_up, dW_down, dW_router); rows
whose reference is exactly zero (experts without kept rows, k = 1 router) must be
exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_mixture_experts_level_amd import workloads as wl
from tests.moe_testlib import HostExperts, row_rel_err, say, to_np

pytestmark = pytest.mark.gpu
ops = pytest.importorskip("sparse_mixture_experts_level_amd.ops")
DEV = "cuda"
TOL = 2e-2


def _run(w, seed=4, overflow="drop", fill_order="token", dy_scale=1.0):
    inp = wl.make_inputs(w, seed=seed, device=DEV)
    cap = ops.moe_capacity(w.num_tokens, w.num_experts, w.capacity_factor)
    layer = ops.MoELayer(inp, cap, fill_order=fill_order, overflow=overflow)
    layer.forward()
    T, d, E, f, fs = w.num_tokens, w.d_model, w.num_experts, w.d_ff, w.d_ff_shared
    g = torch.Generator(device=DEV).manual_seed(seed + 99)
    dy = (torch.randn((T, d), generator=g, device=DEV) * dy_scale).to(torch.bfloat16)
    dx = torch.full((T, d), 7.0, dtype=torch.bfloat16, device=DEV)
    grads = {
        "dw_router": torch.full((E, d), 7.0, dtype=torch.float32, device=DEV),
        "dw_gate_up": torch.full((E, 2 * f, d), 7.0, dtype=torch.bfloat16, device=DEV),
        "dw_down": torch.full((E, d, f), 7.0, dtype=torch.bfloat16, device=DEV),
    }
    if fs:
        grads["dw_shared_gate_up"] = torch.full((2 * fs, d), 7.0, dtype=torch.bfloat16, device=DEV)
        grads["dw_shared_down"] = torch.full((d, fs), 7.0, dtype=torch.bfloat16, device=DEV)
    ws = ops.workspace(ops.moe_backward_workspace_size(layer.desc))
    ops.moe_backward(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, layer.routing, dy, dx, grads, ws,
                     w_shared_gate_up=inp.w_shared_gate_up, w_shared_down=inp.w_shared_down)
    torch.cuda.synchronize()
    return inp, cap, layer, dy, dx, grads, ws


def _reference(w, inp, cap, layer, dy, overflow="drop", fill_order="token"):
    x = to_np(inp.x).astype(np.float64)
    wr = to_np(inp.w_router).astype(np.float64)
    off = None if inp.logit_offset is None else to_np(inp.logit_offset)
    ids = to_np(layer.routing["topk_ids"]).astype(np.int64)
    sgu = sd = None
    if w.d_ff_shared:
        sgu = to_np(inp.w_shared_gate_up).astype(np.float64)
        sd = to_np(inp.w_shared_down).astype(np.float64)
    o = "slot" if fill_order == "rank" else "token"
    return oracle.moe_backward(x, wr, HostExperts(inp.w_gate_up), HostExperts(inp.w_down), w.top_k, cap,
                               to_np(dy).astype(np.float64), off, w_shared_gate_up=sgu, w_shared_down=sd, ids=ids,
                               fill_order=o, overflow=overflow)


def _compare(w, ref, dx, grads):
    E = w.num_experts
    errs = {"dx": row_rel_err(to_np(dx), ref["dx"])}
    gu, dn = to_np(grads["dw_gate_up"]), to_np(grads["dw_down"])
    errs["dw_gate_up"] = max(row_rel_err(gu[e], ref["dw_gate_up"][e]) for e in range(E))
    errs["dw_down"] = max(row_rel_err(dn[e], ref["dw_down"][e]) for e in range(E))
    errs["dw_router"] = row_rel_err(to_np(grads["dw_router"]), ref["dw_router"])
    if w.d_ff_shared:
        errs["dw_shared_gate_up"] = row_rel_err(to_np(grads["dw_shared_gate_up"]), ref["dw_shared_gate_up"])
        errs["dw_shared_down"] = row_rel_err(to_np(grads["dw_shared_down"]), ref["dw_shared_down"])
    for name, e in errs.items():
        assert e <= TOL, (name, e, errs)
    return errs


@pytest.mark.parametrize("T,d,E,k,f,cf,fs,offset", [
    (300, 256, 8, 2, 192, 1.25, 0, "boost4"),
    (513, 128, 16, 4, 128, None, 64, None),
    (257, 64, 4, 1, 64, 0.75, 0, None),        # top-1: the router gets exactly zero gradient
    (200, 128, 32, 8, 64, 1.0, 128, "boost4"),
    (64, 64, 8, 2, 64, 0.1, 0, None),          # most assignments dropped, idle experts
    (1024, 256, 4, 2, 320, None, 0, None),     # hundreds of rows per expert: the large-tile kernels
    (1024, 768, 4, 2, 256, None, 0, None),     # ... with d >= 2 f: [dG dU] transposed instead of x
    (600, 256, 6, 2, 128, None, 256, "boost4"),  # shared expert on the large-tile kernels, ragged tiles
    (600, 512, 6, 2, 128, None, 256, None),      # ... with f_s < d and d >= 2 f_s: the other transposes
])
def test_backward_small_layers(T, d, E, k, f, cf, fs, offset):
    w = wl.Workload("bwd", T, d, E, k, f, cf, "bf16", d_ff_shared=fs, offset=offset)
    say(f"backward T={T} d={d} E={E} k={k} f={f} cf={cf} shared={fs}")
    inp, cap, layer, dy, dx, grads, _ = _run(w)
    ref = _reference(w, inp, cap, layer, dy)
    _compare(w, ref, dx, grads)
    if k == 1:
        assert torch.all(grads["dw_router"] == 0)


@pytest.mark.parametrize("order,overflow", [("rank", "drop"), ("token", "reroute"), ("rank", "reroute")])
def test_backward_dispatch_variants(order, overflow):
    w = wl.Workload("bwd-variant", 300, 128, 8, 2, 128, 1.0, "bf16", offset="boost4")
    say(f"backward variant order={order} overflow={overflow}")
    inp, cap, layer, dy, dx, grads, _ = _run(w, overflow=overflow, fill_order=order)
    ref = _reference(w, inp, cap, layer, dy, overflow=overflow, fill_order=order)
    _compare(w, ref, dx, grads)


def test_backward_is_deterministic():
    w = wl.Workload("bwd-det", 400, 128, 16, 2, 128, 1.25, "bf16", d_ff_shared=64, offset="boost4")
    say("backward determinism")
    inp, cap, layer, dy, dx, grads, ws = _run(w)
    dx2 = torch.empty_like(dx)
    grads2 = {n: torch.empty_like(v) for n, v in grads.items()}
    ops.moe_backward(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, layer.routing, dy, dx2, grads2, ws,
                     w_shared_gate_up=inp.w_shared_gate_up, w_shared_down=inp.w_shared_down)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2)
    for n in grads:
        assert torch.equal(grads[n], grads2[n]), n


def test_backward_with_tile_major_weights():
    """~512 rows per expert (large tiles): the gate_up recompute reading the tile-major copy
    gives the same gradients, bit for bit."""
    w = wl.Workload("bwd-tiled", 1024, 768, 4, 2, 256, None, "bf16", offset="boost4")
    say("backward with tile-major weights")
    inp, cap, layer, dy, dx, grads, ws = _run(w)
    dx2 = torch.empty_like(dx)
    grads2 = {n: torch.empty_like(v) for n, v in grads.items()}
    ops.moe_backward(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, layer.routing, dy, dx2, grads2, ws,
                     tiled=ops.tiled_weights(layer.desc, inp.w_gate_up, inp.w_down))
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    for n in grads:
        assert torch.equal(grads[n], grads2[n]), n


def test_backward_with_tile_major_shared_weights():
    """400 tokens: the shared expert's recompute takes the large-tile regime; reading its
    weights' tile-major copy gives the same gradients, bit for bit."""
    w = wl.Workload("bwd-tiled-shared", 400, 128, 16, 2, 128, 1.25, "bf16", d_ff_shared=320, offset="boost4")
    say("backward with tile-major shared weights")
    inp, cap, layer, dy, dx, grads, ws = _run(w)
    dx2 = torch.empty_like(dx)
    grads2 = {n: torch.empty_like(v) for n, v in grads.items()}
    ops.moe_backward(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, layer.routing, dy, dx2, grads2, ws,
                     w_shared_gate_up=inp.w_shared_gate_up, w_shared_down=inp.w_shared_down,
                     shared_tiled=ops.tiled_shared_weights(layer.desc, inp.w_shared_gate_up, inp.w_shared_down))
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    for n in grads:
        assert torch.equal(grads[n], grads2[n]), n


def test_backward_replays_from_a_captured_graph():
    """moe_backward captured into a HIP graph: every replay equals the eager gradients bit
    for bit (the library clears its buffers with kernels, never with memsets)."""
    w = wl.Workload("bwd-graph", 400, 128, 16, 2, 128, 1.25, "bf16", d_ff_shared=64, offset="boost4")
    say("backward graph capture")
    inp, cap, layer, dy, dx, grads, ws = _run(w)
    want_dx = dx.clone()
    want = {n: v.clone() for n, v in grads.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.moe_backward(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, layer.routing, dy, dx, grads, ws,
                         w_shared_gate_up=inp.w_shared_gate_up, w_shared_down=inp.w_shared_down)
    for i in range(3):
        dx.fill_(3.0)
        for v in grads.values():
            v.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx, want_dx), i
        for n in grads:
            assert torch.equal(grads[n], want[n]), (i, n)


def test_backward_switch_workload_full_size():
    """The Switch-style workload at full size (T = 8192, 64 experts, C = 128)."""
    w = wl.get_workload("switch_bf16")
    say("backward switch_bf16 full size")
    inp, cap, layer, dy, dx, grads, _ = _run(w, seed=0)
    ref = _reference(w, inp, cap, layer, dy)
    errs = _compare(w, ref, dx, grads)
    say(f"errors {errs}")


def _unit_grads(x64, dy64, w_gate_up, w_down, toks, scale, units):
    """The weight gradients of single hidden units of one SwiGLU FFN: the units of a
    SwiGLU FFN are independent (y = sum over u of W_d[:, u] H_u), so the oracle's FFN
    backward on the sub-FFN of unit u (gate row u, up row f + u, down column u) gives
    exactly rows u and f + u of dW_gate_up and column u of dW_down."""
    f = w_down.shape[-1]
    out = {}
    for u in units:
        wgu = np.stack([to_np(w_gate_up[u]), to_np(w_gate_up[f + u])]).astype(np.float64)
        wd = to_np(w_down[:, u:u + 1]).astype(np.float64)
        b = oracle.swiglu_ffn_backward(x64[toks], wgu, wd, dy64[toks], scale=scale)
        out[u] = (b["dw_gate_up"], b["dw_down"][:, 0])
    return out


def _vec_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got))
    m = np.abs(ref).max()
    if m == 0:
        assert np.all(got == 0)
        return 0.0
    return float(np.abs(got - ref).max() / m)


@pytest.mark.parametrize("name,ntok", [("mixtral_bf16", 8), ("deepseek_v3_bf16", 6), ("gptoss_decode_bf16", 16)])
def test_backward_full_size_sampled(name, ntok):
    """Full-size workloads (the bench's configuration) on sampled outputs the oracle computes
    one by one: dx of sampled tokens (their kept assignments' FFN backward, the router term
    and the shared expert, from the oracle's pieces), and single hidden units of the weight
    gradients of the most, a middle and the least loaded expert and of the shared expert."""
    w = wl.get_workload(name)
    say(f"backward {name} full size, sampled")
    inp, cap, layer, dy, dx, grads, _ = _run(w, seed=0)
    T, d, E, k, f, fs = w.num_tokens, w.d_model, w.num_experts, w.top_k, w.d_ff, w.d_ff_shared
    r = {kk: to_np(v) for kk, v in layer.routing.items()}
    ids, slot, gates = r["topk_ids"].astype(np.int64), r["slot"], r["topk_gates"].astype(np.float64)
    serving = ids
    x64 = to_np(inp.x).astype(np.float64)
    dy64 = to_np(dy).astype(np.float64)
    wr = to_np(inp.w_router).astype(np.float64)
    off = None if inp.logit_offset is None else to_np(inp.logit_offset)
    gu, dn = HostExperts(inp.w_gate_up), HostExperts(inp.w_down)
    sgu = sd = None
    if fs:
        sgu = to_np(inp.w_shared_gate_up).astype(np.float64)
        sd = to_np(inp.w_shared_down).astype(np.float64)

    # dx of sampled tokens
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([rng.choice(T, max(ntok - 2, 1), replace=False), [T - 2, T - 1]]))[:ntok]
    got = to_np(dx)[toks]
    ref = np.zeros((toks.size, d))
    for n, t in enumerate(toks):
        dg = np.zeros((1, k))
        for j in range(k):
            if slot[t, j] >= 0:
                e = int(serving[t, j])
                b = oracle.swiglu_ffn_backward(x64[t:t + 1], gu[e], dn[e], dy64[t:t + 1], scale=gates[t, j:j + 1])
                ref[n] += b["dx"][0]
                dg[0, j] = b["dscale"][0]
        lt = oracle.router_logits(x64[t:t + 1], wr, off)
        ref[n] += (oracle.topk_gates_backward(lt, ids[t:t + 1], dg) @ wr)[0]
        if fs:
            ref[n] += oracle.swiglu_ffn_backward(x64[t:t + 1], sgu, sd, dy64[t:t + 1])["dx"][0]
    errs = {"dx": row_rel_err(got, ref)}

    # single units of the weight gradients of three experts
    counts = np.diff(r["expert_offsets"].astype(np.int64))
    nz = np.flatnonzero(counts)
    order = nz[np.argsort(counts[nz], kind="stable")]
    experts = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    units = sorted({0, f - 1, int(rng.integers(1, f - 1))})
    dgu_all, ddn_all = grads["dw_gate_up"], grads["dw_down"]
    for e in experts:
        tt, jj = np.nonzero((slot >= 0) & (serving == e))  # the expert's kept rows
        etoks, scale = tt, gates[tt, jj]
        ref_u = _unit_grads(x64, dy64, inp.w_gate_up[e], inp.w_down[e], etoks, scale, units)
        for u, (rgu, rdn) in ref_u.items():
            g_gu = to_np(dgu_all[e, [u, f + u]])
            errs[f"dw_gate_up[{e}][{u}]"] = max(row_rel_err(g_gu[0:1], rgu[0:1]), row_rel_err(g_gu[1:2], rgu[1:2]))
            errs[f"dw_down[{e}][:,{u}]"] = _vec_rel_err(to_np(ddn_all[e, :, u]), rdn)
    empty = np.flatnonzero(counts == 0)
    if empty.size:
        e0 = int(empty[0])
        assert torch.all(dgu_all[e0] == 0) and torch.all(ddn_all[e0] == 0)
    if fs:
        allt = np.arange(T)
        su = sorted({0, fs - 1, int(rng.integers(1, fs - 1))})
        ref_u = _unit_grads(x64, dy64, inp.w_shared_gate_up, inp.w_shared_down, allt, None, su)
        for u, (rgu, rdn) in ref_u.items():
            g_gu = to_np(grads["dw_shared_gate_up"][[u, fs + u]])
            errs[f"dw_shared_gate_up[{u}]"] = max(row_rel_err(g_gu[0:1], rgu[0:1]), row_rel_err(g_gu[1:2], rgu[1:2]))
            errs[f"dw_shared_down[:,{u}]"] = _vec_rel_err(to_np(grads["dw_shared_down"][:, u]), rdn)
    worst = max(errs.values())
    say(f"  worst sampled error {worst:.3e} over {len(errs)} checks (experts {experts}, units {units})")
    assert worst <= TOL, errs
