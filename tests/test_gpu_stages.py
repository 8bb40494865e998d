"""GPU parity of each hot-path stage against the CPU oracle, called through the C ABI.

Sizes span several tiles and ragged tails while the oracle still finishes in seconds.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.demo_inputs import demo2_fixture, demo2_router_logits
from tests.moe_testlib import (GATE_TOL, HostExperts, check_dispatch_exact, row_rel_err, say, to_np, tol_for)

pytestmark = pytest.mark.gpu
ops = pytest.importorskip("sparse_mixture_experts_level_amd.ops")
DEV = "cuda"


def _desc(T, E, k, cap=None, d=64, f=64, fs=0, dtype=torch.float32, fill_order="token", overflow="drop"):
    return ops.make_desc(T, d, f, E, k, cap, fs, dtype, fill_order=fill_order, overflow=overflow)


# ------------------------------------------------------------------------------------- top-k

def _topk_case(logits_np, k):
    T, E = logits_np.shape
    say(f"topk T={T} E={E} k={k}")
    lg = torch.from_numpy(logits_np.astype(np.float32)).to(DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ops.moe_router_topk(_desc(T, E, k), lg, ids, gates)
    torch.cuda.synchronize()
    ref_l = logits_np.astype(np.float32).astype(np.float64)
    ref_ids = oracle.topk_select(ref_l, k)
    ref_g = oracle.topk_gates(ref_l, ref_ids)
    assert np.array_equal(to_np(ids), ref_ids)
    assert np.abs(to_np(gates) - ref_g).max() <= GATE_TOL


@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (257, 64, 1), (100, 32, 4), (130, 256, 8), (33, 5, 5),
                                   (40, 1024, 70), (17, 130, 3), (1, 1, 1)])
def test_topk_bitexact_random(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    _topk_case(rng.normal(size=(T, E)) * 2.0, k)


def test_topk_ties_signed_zero_and_neg_inf():
    rng = np.random.default_rng(11)
    l = rng.integers(-2, 3, size=(200, 12)).astype(np.float64)
    l[0] = 0.0
    l[1, :6] = -0.0
    l[2] = -np.inf
    l[2, 7] = 1.0
    l[3, ::2] = -np.inf
    for k in (1, 3, 6, 12):
        _topk_case(l, k)


# ------------------------------------------------------------------------------------- dispatch

def _dispatch_case(ids_np, E, cap, d=64, dtype=torch.bfloat16, tag=""):
    T, k = ids_np.shape
    say(f"dispatch {tag} T={T} E={E} k={k} cap={cap}")
    desc = _desc(T, E, k, cap, d=d, f=64, dtype=dtype)
    R = ops.moe_max_rows(desc)
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
    x = torch.randn((T, d), device=DEV).to(dtype)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    row_token = torch.full((max(R, 1),), -7, dtype=torch.int32, device=DEV)
    x_perm = torch.zeros((max(R, 1), d), dtype=dtype, device=DEV)
    ws = ops.workspace(ops.moe_workspace_size(desc))
    ops.moe_dispatch_permute(desc, ids, x, counts, offsets, slot, row_token, x_perm, ws)
    torch.cuda.synchronize()
    ref = check_dispatch_exact(ids_np, E, cap, to_np(counts), to_np(offsets), to_np(slot), to_np(row_token))
    Rk = int(ref["offsets"][-1])
    assert torch.equal(x_perm[:Rk], x[torch.from_numpy(ref["row_token"]).long().to(DEV)])
    return ref


def _ids(rng, T, E, k, skew=0.0):
    p = np.exp(-skew * np.log(np.arange(1, E + 1)))
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,cap,skew", [
    (300, 8, 2, 10, 0.0), (300, 8, 2, None, 1.0), (5000, 64, 1, 78, 1.1), (3000, 256, 8, 40, 1.1),
    (777, 1024, 3, 2, 0.5), (64, 8, 2, 0, 0.0), (1, 4, 4, 1, 0.0), (4100, 32, 4, None, 0.0),
])
def test_dispatch_bitexact(T, E, k, cap, skew):
    rng = np.random.default_rng(T + E + k)
    _dispatch_case(_ids(rng, T, E, k, skew), E, cap)


def _ids_with_strays(seed, T=700, E=16, k=2):
    """Routing ids with one entry outside [0, E) in about 5% of the tokens; also the same ids
    with every stray entry replaced by a phantom expert E, ordered after all real ones, and the
    valid ids the strays replaced."""
    rng = np.random.default_rng(seed)
    ids = _ids(rng, T, E, k, 0.5)
    toks = np.nonzero(rng.random(T) < 0.05)[0]
    js = rng.integers(0, k, size=toks.size)
    bad = ids.copy()
    bad[toks, js] = rng.choice([-1, -5, E, E + 3, 1 << 20, -(1 << 30)], size=toks.size)
    phantom = ids.copy()
    phantom[toks, js] = E
    return bad, phantom, (toks, js), ids


def test_dispatch_ids_outside_the_range_are_dropped():
    """An id outside [0, E) (a broken precondition) is no expert: slot -1, not counted, no row.
    The expected tables are the oracle's fill with such ids sent to a phantom expert E placed
    after every real one (its rows come last, so no real expert's slots or offsets move)."""
    T, E, k, cap = 700, 16, 2, 60
    bad, phantom, stray, _ = _ids_with_strays(5, T, E, k)
    say(f"dispatch with stray ids T={T} E={E} k={k} cap={cap}")
    desc = _desc(T, E, k, cap, dtype=torch.bfloat16)
    R = ops.moe_max_rows(desc)
    ids = torch.from_numpy(bad).to(DEV)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    row_token = torch.full((max(R, 1),), -7, dtype=torch.int32, device=DEV)
    ws = ops.workspace(ops.moe_workspace_size(desc))
    ops.moe_dispatch_permute(desc, ids, None, counts, offsets, slot, row_token, None, ws)
    torch.cuda.synchronize()
    ref = oracle.capacity_fill(phantom, E + 1, cap)
    want_slot = ref["slot"].copy()
    want_slot[stray] = -1
    assert np.array_equal(to_np(counts), ref["counts"][:E])
    assert np.array_equal(to_np(offsets), ref["offsets"][:E + 1])
    assert np.array_equal(to_np(slot), want_slot)
    Rk = int(ref["offsets"][E])
    assert np.array_equal(to_np(row_token)[:Rk], ref["row_token"][:Rk])

    # the combine adds nothing for an id outside [0, E), even with a slot >= 0 beside it
    d = 64
    y_perm = torch.randn((max(R, 1), d), device=DEV).to(torch.bfloat16)
    gates = torch.rand((T, k), device=DEV)
    slot_good = slot.clone()
    toks, js = stray
    good_ids = torch.from_numpy(np.where(phantom == E, 0, phantom).astype(np.int32)).to(DEV)
    slot_good[torch.from_numpy(toks).long().to(DEV), torch.from_numpy(js).long().to(DEV)] = 0
    out_bad = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    out_ref = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    ops.moe_combine_unpermute(desc, y_perm, ids, gates, slot_good, offsets, None, out_bad)
    ops.moe_combine_unpermute(desc, y_perm, good_ids, gates, slot, offsets, None, out_ref)
    torch.cuda.synchronize()
    assert torch.equal(out_bad, out_ref)


def test_debug_library_rejects_ids_outside_the_range():
    """libmoe_debug.so checks the ids precondition on the host before any launch: a stray id
    gives MOE_ERR_INVALID and leaves every output untouched; valid ids give the release
    library's tables."""
    T, E, k, cap = 700, 16, 2, 60
    bad, _, stray, good = _ids_with_strays(6, T, E, k)
    D = ops.debug_lib()
    desc = _desc(T, E, k, cap, dtype=torch.bfloat16)
    R = ops.moe_max_rows(desc)
    ws = ops.workspace(ops.moe_workspace_size(desc))

    def run(ids_np, L):
        tabs = [torch.full(n, -7, dtype=torch.int32, device=DEV) for n in ((E,), (E + 1,), (T, k), (max(R, 1),))]
        ops.moe_dispatch_permute(desc, torch.from_numpy(ids_np).to(DEV), None, *tabs, None, ws, L=L)
        torch.cuda.synchronize()
        return [to_np(t) for t in tabs]

    say("debug library: stray id rejected")
    with pytest.raises(ops.MoEError) as ei:
        run(bad, D)
    assert ei.value.status == ops.MOE_ERR_INVALID
    t0, j0 = int(stray[0][0]), int(stray[1][0])
    assert f"topk_ids[{t0}][{j0}]" in str(ei.value)
    say("debug library: valid ids accepted, same tables as the release library")
    got, want = run(good, D), run(good, ops.lib())
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
    y_perm = torch.zeros((max(R, 1), 64), dtype=torch.bfloat16, device=DEV)
    out = torch.full((T, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.MoEError):
        ops.moe_combine_unpermute(desc, y_perm, torch.from_numpy(bad).to(DEV), torch.ones((T, k), device=DEV),
                                  torch.zeros((T, k), dtype=torch.int32, device=DEV),
                                  torch.zeros(E + 1, dtype=torch.int32, device=DEV), None, out, L=D)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def _variant_case(logits_np, k, cap, order, reroute, tag=""):
    """Rank-major fill and/or redirection of overflow on the GPU vs the oracle, bit-exact.  The
    ids come from the GPU's top-k of float32 logits, and the oracle takes the same float32
    logits, so the routing is identical and every integer output must match."""
    T, E = logits_np.shape
    say(f"dispatch variant {tag} T={T} E={E} k={k} cap={cap} order={order} reroute={reroute}")
    desc = _desc(T, E, k, cap, fill_order=order, overflow="reroute" if reroute else "drop")
    R = ops.moe_max_rows(desc)
    lg32 = logits_np.astype(np.float32)
    lg = torch.from_numpy(lg32).to(DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ops.moe_router_topk(desc, lg, ids, gates)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    assigned = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    row_token = torch.full((max(R, 1),), -7, dtype=torch.int32, device=DEV)
    ws = ops.workspace(ops.moe_workspace_size(desc))
    if reroute:
        ops.moe_dispatch_reroute(desc, lg, ids, counts, offsets, slot, assigned, row_token, ws)
    else:
        ops.moe_dispatch_permute(desc, ids, None, counts, offsets, slot, row_token, None, ws)
    torch.cuda.synchronize()
    ids_np = to_np(ids)
    assert np.array_equal(ids_np, oracle.topk_select(lg32.astype(np.float64), k))
    order_o = "slot" if order == "rank" else "token"
    return check_dispatch_exact(ids_np, E, cap, to_np(counts), to_np(offsets), to_np(slot), to_np(row_token),
                                order=order_o, logits=lg32.astype(np.float64) if reroute else None,
                                assigned=to_np(assigned) if reroute else None)


@pytest.mark.parametrize("T,E,k,cap,skew,reroutes", [
    (300, 8, 2, 10, 0.0, False), (5000, 64, 1, 78, 2.0, True), (3000, 256, 8, 40, 1.5, True),
    (777, 1024, 3, 2, 0.5, True), (64, 8, 2, 0, 0.0, False), (1, 4, 4, 1, 0.0, False), (4100, 32, 4, 600, 1.0, True),
    (1000, 6, 3, 700, 0.0, False),
])
@pytest.mark.parametrize("order,reroute", [("rank", False), ("token", True), ("rank", True)])
def test_dispatch_variants_bitexact(T, E, k, cap, skew, reroutes, order, reroute):
    rng = np.random.default_rng(T + 3 * E + k)
    logits = rng.normal(size=(T, E)) - skew * np.log(np.arange(1, E + 1))[None, :]
    ref = _variant_case(logits, k, cap, order, reroute)
    if reroute and reroutes:  # cases chosen so that hot experts overflow while cold ones keep room
        assert ref["rerouted"] > 0


def test_dispatch_reroute_without_capacity_is_the_plain_dispatch():
    rng = np.random.default_rng(9)
    _variant_case(rng.normal(size=(400, 16)), 4, None, "token", True)


def test_dispatch_float_rows_and_everyone_on_one_expert():
    ids = np.zeros((500, 1), dtype=np.int32)
    ref = _dispatch_case(ids, 8, 17, d=24, dtype=torch.float32, tag="collapse")
    assert ref["drops"] == 500 - 17


def test_demo_worked_example_on_gpu():
    """The page's demo: drops 8/5 (balanced) and 11/9 (collapsed) at C = 4/5."""
    g = demo2_fixture()
    logits = demo2_router_logits()
    for name, lg in logits.items():
        say(f"demo {name}")
        lg = torch.from_numpy(lg.astype(np.float32)).to(DEV)
        ids = torch.empty((32, 1), dtype=torch.int32, device=DEV)
        gates = torch.empty((32, 1), dtype=torch.float32, device=DEV)
        ops.moe_router_topk(_desc(32, 8, 1), lg, ids, gates)
        for i, cf in enumerate(g["capacity_factors"]):
            cap = ops.moe_capacity(32, 8, cf)
            assert cap == g[name]["capacity"][i]
            desc = _desc(32, 8, 1, cap)
            counts = torch.empty(8, dtype=torch.int32, device=DEV)
            offsets = torch.empty(9, dtype=torch.int32, device=DEV)
            slot = torch.empty((32, 1), dtype=torch.int32, device=DEV)
            row_token = torch.empty(32, dtype=torch.int32, device=DEV)
            ops.moe_dispatch_permute(desc, ids, None, counts, offsets, slot, row_token, None,
                                     ops.workspace(ops.moe_workspace_size(desc)))
            torch.cuda.synchronize()
            assert int((slot < 0).sum()) == g[name]["dropped"][i]
            if "counts" in g[name]:
                assert to_np(counts).tolist() == g[name]["counts"]
        assert torch.all(gates == 1.0)


# ------------------------------------------------------------------------------------- router logits

@pytest.mark.parametrize("T,d,E,dtype", [(300, 256, 8, torch.bfloat16), (129, 128, 64, torch.bfloat16),
                                         (70, 192, 256, torch.bfloat16), (65, 64, 300, torch.bfloat16),
                                         (77, 100, 9, torch.float32)])
def test_router_logits(T, d, E, dtype):
    say(f"router_logits T={T} d={d} E={E} {dtype}")
    g = torch.Generator(device=DEV).manual_seed(T + d + E)
    x = torch.randn((T, d), generator=g, device=DEV).to(dtype)
    w = (torch.randn((E, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    off = torch.randn((E,), generator=g, device=DEV)
    logits = torch.full((T, E), float("nan"), device=DEV)
    ops.moe_router_logits(_desc(T, E, 1, d=d, f=64, dtype=dtype), x, w, off, logits)
    torch.cuda.synchronize()
    xn, wn = to_np(x).astype(np.float64), to_np(w).astype(np.float64)
    ref = oracle.router_logits(xn, wn, to_np(off))
    bound = np.abs(xn) @ np.abs(wn).T
    err = np.abs(to_np(logits) - ref)
    assert np.all(err <= 4e-6 * bound + 1e-6), err.max()


# ------------------------------------------------------------------------------------- grouped GEMM

def _gemm_case(sizes, d, f, dtype, hint, seed=0, x_scale=1.0):
    G = len(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offs[-1]) + 5  # spare rows beyond the last group stay untouched
    say(f"grouped_gemm G={G} sizes={sizes} d={d} f={f} {dtype} hint={hint} x_scale={x_scale}")
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = (torch.randn((R, d), generator=g, device=DEV) * x_scale).to(dtype)
    wgu = (torch.randn((G, 2 * f, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    wd = (torch.randn((G, d, f), generator=g, device=DEV) / math.sqrt(f)).to(dtype)
    y = torch.full((R, d), 3.0, dtype=dtype, device=DEV)
    go = torch.from_numpy(offs).to(DEV)
    ws = ops.workspace(ops.moe_grouped_gemm_workspace_size(G, R, f, dtype))
    ops.moe_grouped_swiglu_gemm(G, R, hint, d, f, dtype, x, go, wgu, wd, y, ws)
    torch.cuda.synchronize()
    xn, yn = to_np(x).astype(np.float64), to_np(y)
    W1, W2 = HostExperts(wgu), HostExperts(wd)
    worst = 0.0
    for e in range(G):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo:
            ref = oracle.swiglu_ffn(xn[lo:hi], W1[e], W2[e])
            worst = max(worst, row_rel_err(yn[lo:hi], ref))
    assert np.all(yn[offs[-1]:] == 3.0), "rows outside every group were written"
    assert worst <= tol_for(dtype), worst
    return worst


@pytest.mark.parametrize("sizes,hint", [
    ([0, 1, 17, 130, 5, 0, 64, 33], 128), ([16, 3, 0, 9], 16), ([40, 31, 64], 64),
    ([300, 2], 16),  # groups larger than the tiling hint are still computed
    ([7], 7),
])
def test_grouped_gemm_bf16(sizes, hint):
    _gemm_case(sizes, 256, 192, torch.bfloat16, hint)


def test_grouped_gemm_bf16_wide():
    _gemm_case([33, 0, 129], 1024, 320, torch.bfloat16, 129, seed=3)


@pytest.mark.parametrize("sizes,d,f", [
    ([600, 0, 300, 1000], 256, 192),  # ragged row tiles, an empty group, a column tail (192 = 1.5 x 128)
    ([2000], 512, 384),
    ([257, 511, 1, 256], 320, 256),   # K = 320 (five 64-wide steps)
    # eight groups x 4096 columns: gate_up leaves last tiles of <= 128 rows to a streaming
    # launch (44, 88 and 8 rows; a 40-row group entirely), keeps 188- and 130-row ones
    ([300, 600, 40, 520, 700, 256, 130, 0], 256, 4096),
    # 72 groups (the tail launch maps workgroups to tail groups only up to 64 groups): in
    # every eight, tails of 44, 4, 34, 1 and 14 rows and a 144-row last tile kept
    ([300, 260, 256, 400, 290, 0, 513, 270] * 9, 128, 512),
])
def test_grouped_gemm_bf16_large_groups(sizes, d, f):
    """Average group of >= 256 rows: the 256 x 256 MFMA tile kernel."""
    _gemm_case(sizes, d, f, torch.bfloat16, max(sizes), seed=len(sizes))


@pytest.mark.parametrize("sizes,hint", [([40, 3, 100], 128), ([600, 0, 300], 600)])
def test_grouped_gemm_bf16_large_preactivations(sizes, hint):
    """Gate pre-activations in the hundreds (x scaled by 100): silu saturates to -0 for very
    negative ones (exp overflows to inf) and to the identity for very positive ones, in the
    streaming and the large-tile kernels' SwiGLU epilogues."""
    _gemm_case(sizes, 256, 192, torch.bfloat16, hint, seed=3, x_scale=100.0)


@pytest.mark.parametrize("sizes,d,f", [([0, 1, 17, 70, 5], 100, 72), ([10], 128, 256), ([3, 4], 7, 5)])
def test_grouped_gemm_f32(sizes, d, f):
    _gemm_case(sizes, d, f, torch.float32, max(sizes))


@pytest.mark.parametrize("sizes,d,f,dtype,hint", [
    ([0, 1, 17, 130, 5, 0, 64, 33], 256, 192, torch.bfloat16, 130),  # streaming kernel
    ([600, 0, 300, 1000], 256, 192, torch.bfloat16, 1000),           # large-tile kernel
    ([0, 3, 40, 9], 100, 72, torch.float32, 40),
])
def test_gate_up_row_gather(sizes, d, f, dtype, hint):
    """gate_up with row_index: rows are read from an unpermuted activation matrix."""
    G = len(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offs[-1])
    T = max(1, R // 2 + 7)
    say(f"gate_up gather G={G} sizes={sizes} T={T} {dtype}")
    rng = np.random.default_rng(G)
    idx = rng.integers(0, T, size=R).astype(np.int32)
    g = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randn((T, d), generator=g, device=DEV).to(dtype)
    wgu = (torch.randn((G, 2 * f, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    h = torch.full((R + 3, f), 5.0, dtype=dtype, device=DEV)
    go = torch.from_numpy(offs).to(DEV)
    ops.moe_grouped_gate_up_swiglu(G, R + 3, hint, d, f, dtype, x, go, wgu, h,
                                   row_index=torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    xn, hn = to_np(x).astype(np.float64), to_np(h)
    W1 = HostExperts(wgu)
    worst = 0.0
    for e in range(G):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo:
            Wg = W1[e]
            X = xn[idx[lo:hi]]
            ref = oracle.silu(X @ Wg[:f].T) * (X @ Wg[f:].T)
            worst = max(worst, row_rel_err(hn[lo:hi], ref))
    assert np.all(hn[R:] == 5.0)
    assert worst <= (1e-2 if dtype == torch.bfloat16 else 1e-5), worst


# ------------------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,E,k,cap,d,dtype,shared", [
    (300, 8, 2, 40, 256, torch.bfloat16, False), (300, 8, 2, 40, 256, torch.bfloat16, True),
    (100, 64, 1, 2, 1024, torch.bfloat16, False), (50, 32, 8, None, 64, torch.float32, True),
    (10, 4, 4, 1, 30, torch.float32, False),
    # enough tokens for two 16-byte vectors per lane: rows fetched two at a time, one at a
    # time (k = 1), and a last column segment only partly filled (130 vectors of 128 + 2)
    (4096, 16, 2, 600, 1024, torch.bfloat16, True), (4200, 8, 1, None, 512, torch.float32, False),
    (4096, 8, 3, None, 520, torch.float32, True),
    # more than 64 assignments per token: the wave reads a second group of slots
    (40, 96, 70, 8, 128, torch.bfloat16, True), (30, 80, 66, None, 64, torch.float32, False),
])
def test_combine(T, E, k, cap, d, dtype, shared):
    say(f"combine T={T} E={E} k={k} cap={cap} d={d} {dtype} shared={shared}")
    rng = np.random.default_rng(T + k)
    ids_np = _ids(rng, T, E, k)
    fill = oracle.capacity_fill(ids_np, E, cap)
    R = max(int(fill["offsets"][-1]), 1)
    gates_np = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    g = torch.Generator(device=DEV).manual_seed(5)
    y = torch.randn((R, d), generator=g, device=DEV).to(dtype)
    sh = torch.randn((T, d), generator=g, device=DEV).to(dtype) if shared else None
    out = torch.full((T, d), 7.0, dtype=dtype, device=DEV)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    ops.moe_combine_unpermute(_desc(T, E, k, cap, d=d, dtype=dtype), y, t(ids_np.astype(np.int32)), t(gates_np),
                              t(fill["slot"]), t(fill["offsets"].astype(np.int32)), sh, out)
    torch.cuda.synchronize()
    yn = to_np(y).astype(np.float64)
    rows = lambda tt, j: yn[fill["offsets"][ids_np[tt, j]] + fill["slot"][tt, j]]
    ref = oracle.combine(T, d, ids_np, gates_np.astype(np.float64), fill["slot"], rows,
                         shared=to_np(sh).astype(np.float64) if shared else None)
    assert row_rel_err(to_np(out), ref) <= (2 ** -8 if dtype == torch.bfloat16 else 1e-6)


# ------------------------------------------------------------------------------------- aux loss

def _aux_gpu(logits_np, k, alpha=0.01, cap=None):
    T, E = logits_np.shape
    desc = _desc(T, E, k, cap)
    lg = torch.from_numpy(logits_np.astype(np.float32)).to(DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, k), dtype=torch.float32, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    slot = torch.empty((T, k), dtype=torch.int32, device=DEV)
    row_token = torch.empty(max(ops.moe_max_rows(desc), 1), dtype=torch.int32, device=DEV)
    ws = ops.workspace(ops.moe_workspace_size(desc))
    loss = torch.full((1,), float("nan"), device=DEV)
    ops.moe_router_topk(desc, lg, ids, gates)
    ops.moe_dispatch_permute(desc, ids, None, counts, offsets, slot, row_token, None, ws)
    ops.moe_router_aux_loss(desc, lg, counts, alpha, loss, ws)
    torch.cuda.synchronize()
    return float(loss.item()), to_np(ids)


def test_aux_loss_reproduces_the_demo():
    """The page's demo prints 0.010505 (balanced router) and 0.019086 (collapsed)."""
    g = demo2_fixture()
    logits = demo2_router_logits()
    for name, lg in logits.items():
        say(f"aux loss demo {name}")
        loss, _ = _aux_gpu(lg.astype(np.float64), 1, cap=ops.moe_capacity(32, 8, 1.0))
        assert round(loss, 6) == g[name]["aux_loss"]


@pytest.mark.parametrize("T,E,k", [(1000, 64, 2), (300, 8, 1), (777, 256, 8), (50, 1024, 3)])
def test_aux_loss_matches_oracle(T, E, k):
    say(f"aux loss T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E)
    lg = rng.normal(size=(T, E)) * 2 + np.linspace(0, 3, E)[None, :]
    loss, ids = _aux_gpu(lg, k, alpha=0.01)
    ref = oracle.aux_load_balancing_loss(ids, oracle.softmax(lg.astype(np.float32).astype(np.float64)), E, 0.01)
    assert loss == pytest.approx(ref, rel=2e-5)


def test_aux_loss_uniform_is_alpha():
    E, T = 16, 512
    lg = np.zeros((T, E))
    lg[np.arange(T), np.arange(T) % E] = 1e-3  # round-robin choice, nearly uniform probabilities
    loss, _ = _aux_gpu(lg, 1, alpha=0.02)
    assert loss == pytest.approx(0.02, rel=1e-3)


def _tiled_reference(w, rows_per_tile_gate, n_rows, K, swiglu):
    """The tile-major layout as include/moe.h documents it, built with NumPy from row-major
    weights w [E, rows, K] (uint16 view): per expert, tile nt and K step kt a block of 256 rows
    x 32 values, 16-byte chunk c of row r stored at chunk position c ^ ((r >> 2) & 3), rows past
    the matrix zero; gate_up tiles hold 128 gate rows then the matching up rows (n_rows apart)."""
    E = w.shape[0]
    ntiles = -(-n_rows // rows_per_tile_gate)
    out = np.zeros((E, ntiles, K // 32, 256, 4, 8), dtype=np.uint16)
    for e in range(E):
        for nt in range(ntiles):
            for r in range(256):
                if swiglu:
                    col = nt * 128 + (r & 127)
                    if col >= n_rows:
                        continue
                    src = col if r < 128 else n_rows + col
                else:
                    src = nt * 256 + r
                    if src >= n_rows:
                        continue
                chunks = w[e, src].reshape(K // 32, 4, 8)
                for c in range(4):
                    out[e, nt, :, r, c ^ ((r >> 2) & 3), :] = chunks[:, c, :]
    return out.reshape(-1)


def test_tile_major_weights_layout_is_the_documented_one():
    """moe_tile_expert_weights writes exactly the layout its declaration describes (ragged
    tiles: f = 192 is 1.5 gate_up tiles of 128, d = 64 is a quarter of a down tile)."""
    E, d, f = 3, 64, 192
    say("tile-major weight layout, E=3 d=64 f=192")
    g = torch.Generator(device=DEV).manual_seed(21)
    w_gu = torch.randn((E, 2 * f, d), generator=g, device=DEV).to(torch.bfloat16)
    w_dn = torch.randn((E, d, f), generator=g, device=DEV).to(torch.bfloat16)
    desc = ops.make_desc(64, d, f, E, 1, None, 0, torch.bfloat16)
    gu_t, dn_t = ops.tiled_weights(desc, w_gu, w_dn)
    torch.cuda.synchronize()
    got_gu = gu_t.cpu().numpy().view(np.uint16)
    got_dn = dn_t.cpu().numpy().view(np.uint16)
    want_gu = _tiled_reference(w_gu.cpu().view(torch.int16).numpy().view(np.uint16), 128, f, d, True)
    want_dn = _tiled_reference(w_dn.cpu().view(torch.int16).numpy().view(np.uint16), 256, d, f, False)
    assert got_gu.shape == want_gu.shape and got_dn.shape == want_dn.shape
    assert np.array_equal(got_gu, want_gu)
    assert np.array_equal(got_dn, want_dn)
