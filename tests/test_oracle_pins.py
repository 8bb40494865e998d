"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: each check uses values printed on
the pages (tests/golden/), closed forms at special points, brute-force
enumeration on tiny inputs, invariants, or an independent library routine.
CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests.demo_inputs import demo2_router_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# --------------------------------------------------------------------------------------------
# Worked example printed on the page (demo 2): capacity, drops, per-expert counts, aux loss.
# --------------------------------------------------------------------------------------------

def _demo2_logits():
    lg = demo2_router_logits()
    return lg["balanced"], lg["collapsed"]


def test_demo2_capacity_drops_counts_aux():
    g = _load("demo2_capacity_dropping.json")
    lb, lc = _demo2_logits()
    for name, logits in (("balanced", lb), ("collapsed", lc)):
        want = g[name]
        ids = oracle.topk_select(logits, 1)
        for i, cf in enumerate(g["capacity_factors"]):
            cap = oracle.capacity(32, 8, cf)
            assert cap == want["capacity"][i]
            fill = oracle.capacity_fill(ids, 8, cap)
            assert fill["drops"] == want["dropped"][i]
            assert int(np.sum(fill["slot"] < 0)) == want["dropped"][i]
            if "counts" in want:
                assert fill["counts"].tolist() == want["counts"]
        aux = oracle.aux_load_balancing_loss(ids, oracle.softmax(logits), 8, alpha=0.01)
        assert round(aux, 6) == want["aux_loss"]


def test_demo2_drops_closed_form_from_printed_counts():
    """For k = 1 the sequential fill drops sum_e max(0, n_e - C); the printed collapsed
    counts give the printed 11 and 9 drops whatever the token order."""
    g = _load("demo2_capacity_dropping.json")
    counts = g["collapsed"]["counts"]
    rng = np.random.default_rng(7)
    ids = np.repeat(np.arange(8), counts)
    for trial in range(3):
        perm = rng.permutation(ids).reshape(-1, 1).astype(np.int32)
        for i, cap in enumerate(g["collapsed"]["capacity"]):
            fill = oracle.capacity_fill(perm, 8, cap)
            assert fill["drops"] == g["collapsed"]["dropped"][i]
            assert fill["drops"] == sum(max(0, n - cap) for n in counts)
            assert fill["counts"].tolist() == counts


def test_demo1_active_parameter_counts():
    g = _load("demo1_active_params.json")
    L = g["layer"]
    for k, key in ((1, "top1"), (2, "top2")):
        r = oracle.active_params(L["d_model"], L["hidden"], L["num_experts"], k, ffn="relu_bias")
        assert r["active"] == g[key]["active"]
        assert r["total"] == g[key]["total"]
        assert round(100 * r["active"] / r["total"], 1) == g[key]["percent"]


# --------------------------------------------------------------------------------------------
# Capacity
# --------------------------------------------------------------------------------------------

def test_capacity_values_and_evaluation_order():
    assert oracle.capacity(64, 8, 1.25) == 10
    assert oracle.capacity(8192, 64, 1.0) == 128
    assert oracle.capacity(16384, 256, 1.25) == 80
    assert oracle.capacity(32, 8, 1.0) == 4 and oracle.capacity(32, 8, 1.25) == 5
    assert oracle.capacity(100, 8, None) is None and oracle.capacity(100, 8, 0.0) is None
    # ceil(cf * T / E) in that order, in double: 1.1 * 50 / 5 is 11.000000000000002 and
    # rounds up to 12, while 1.1 * (50 / 5) is exactly 11.
    assert 1.1 * 50 / 5 > 11.0 and 1.1 * (50 / 5) == 11.0
    assert oracle.capacity(50, 5, 1.1) == 12


# --------------------------------------------------------------------------------------------
# Top-k selection: brute force over all k-subsets on tiny inputs with many exact ties.
# --------------------------------------------------------------------------------------------

def _brute_topk(row, k):
    E = len(row)
    hits = []
    for S in itertools.combinations(range(E), k):
        ok = all((row[e] > row[o]) or (row[e] == row[o] and e < o)
                 for e in S for o in range(E) if o not in S)
        if ok:
            hits.append(S)
    assert len(hits) == 1
    S = hits[0]
    # descending logit; equal logits by ascending index
    return sorted(S, key=lambda e: (-row[e], e))


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(0)
    for E in (1, 2, 3, 5, 6):
        for k in range(1, E + 1):
            logits = rng.integers(-2, 3, size=(40, E)).astype(np.float64)
            logits[0] = 0.0
            logits[1] = -np.inf
            logits[1, E - 1] = 0.0
            ids = oracle.topk_select(logits, k)
            for t in range(logits.shape[0]):
                assert ids[t].tolist() == _brute_topk(logits[t].tolist(), k)


def test_topk_signed_zero_is_a_tie():
    ids = oracle.topk_select(np.array([[-0.0, 0.0, -1.0]]), 1)
    assert ids.tolist() == [[0]]


# --------------------------------------------------------------------------------------------
# Gates
# --------------------------------------------------------------------------------------------

def test_gates_sum_to_one_and_equal_softmax_of_selected_logits():
    rng = np.random.default_rng(1)
    logits = rng.normal(size=(50, 12)) * 3
    for k in (1, 2, 4, 12):
        ids = oracle.topk_select(logits, k)
        g = oracle.topk_gates(logits, ids)
        assert np.allclose(g.sum(axis=1), 1.0, atol=1e-12, rtol=0)
        if k == 1:
            assert np.all(g == 1.0)
        for t in range(logits.shape[0]):
            sel = [logits[t, e] for e in ids[t]]
            m = max(sel)
            z = [math.exp(v - m) for v in sel]
            want = [v / math.fsum(z) for v in z]
            assert np.allclose(g[t], want, rtol=1e-13, atol=0)
            assert np.all(np.diff(g[t]) <= 0)  # descending order of the chosen experts


# --------------------------------------------------------------------------------------------
# Capacity fill: brute-force count definition and invariants.
# --------------------------------------------------------------------------------------------

def _random_ids(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def test_fill_matches_bruteforce_count():
    rng = np.random.default_rng(2)
    for T, E, k in ((1, 1, 1), (7, 3, 1), (30, 4, 2), (25, 5, 3), (40, 6, 6)):
        ids = _random_ids(rng, T, E, k)
        for cap in (None, 1, 2, 5, T * k):
            fill = oracle.capacity_fill(ids, E, cap)
            for t in range(T):
                for j in range(k):
                    e = ids[t, j]
                    before = sum(1 for u in range(t) if e in ids[u])
                    want = before if (cap is None or before < cap) else -1
                    assert fill["slot"][t, j] == want
            for e in range(E):
                kept_tokens = [t for t in range(T) if e in ids[t]]
                if cap is not None:
                    kept_tokens = kept_tokens[:cap]
                lo, hi = fill["offsets"][e], fill["offsets"][e + 1]
                assert fill["row_token"][lo:hi].tolist() == kept_tokens


def test_fill_invariants():
    rng = np.random.default_rng(3)
    T, E, k = 3000, 16, 2
    # skewed demand: a few experts are popular
    p = np.array([8.0] * 3 + [1.0] * (E - 3))
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    for cap in (None, 50, 375, 400):
        fill = oracle.capacity_fill(ids, E, cap)
        n = np.bincount(ids.reshape(-1), minlength=E)
        assert fill["counts"].tolist() == n.tolist()
        c = np.inf if cap is None else cap
        assert np.all(fill["kept"] == np.minimum(n, c))
        assert fill["kept"].sum() == T * k - fill["drops"]
        assert np.all(fill["kept"] <= c)
        assert fill["offsets"][0] == 0 and np.all(np.diff(fill["offsets"]) == fill["kept"])
        # every slot of an expert appears exactly once
        for e in range(E):
            s = np.sort(fill["slot"][ids == e])
            s = s[s >= 0]
            assert s.tolist() == list(range(int(fill["kept"][e])))
        # late tokens drop more often than early ones under a tight capacity
        if cap == 50:
            dropped = (fill["slot"] < 0).any(axis=1)
            assert dropped[: T // 2].sum() < dropped[T // 2:].sum()


# --------------------------------------------------------------------------------------------
# Expert FFN (SwiGLU): closed forms at special points and an independent library routine.
# --------------------------------------------------------------------------------------------

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    got = oracle.silu(np.array([0.0, ln3, -ln3, 800.0, -800.0]))
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly
    assert got[0] == 0.0
    assert got[1] == pytest.approx(0.75 * ln3, rel=1e-15)
    assert got[2] == pytest.approx(-0.25 * ln3, rel=1e-15)
    assert got[3] == 800.0 and abs(got[4]) < 1e-300


def test_swiglu_hand_worked_example():
    """d = 3, f = 2, hand-computed: gate pre-activations (ln 3, 0), up (2, ln 3),
    h = (2 * 0.75 ln 3, 0), y = W_d h."""
    ln3 = math.log(3.0)
    x = np.array([[ln3, 1.0, 0.5]])
    w_gate = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    w_up = np.array([[0.0, 2.0, 0.0], [1.0, 0.0, 0.0]])
    w_down = np.array([[1.0, 5.0], [3.0, 7.0], [-2.0, 4.0]])  # [d, f]
    y = oracle.swiglu_ffn(x, np.concatenate([w_gate, w_up]), w_down)
    h0 = 2 * 0.75 * ln3
    assert y.shape == (1, 3)
    assert np.allclose(y[0], [h0 * 1.0, h0 * 3.0, h0 * -2.0], rtol=1e-14, atol=0)


def test_swiglu_against_torch_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    d, f, n = 48, 80, 9
    x = rng.normal(size=(n, d))
    wgu = rng.normal(size=(2 * f, d)) / math.sqrt(d)
    wd = rng.normal(size=(d, f)) / math.sqrt(f)
    y = oracle.swiglu_ffn(x, wgu, wd)
    tx, tgu, td = (torch.from_numpy(a) for a in (x, wgu, wd))
    g, u = torch.nn.functional.linear(tx, tgu).chunk(2, dim=-1)
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, td).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------------
# Whole layer: reductions to known cases and symmetries.
# --------------------------------------------------------------------------------------------

def _layer(rng, T, d, E, f, fs=0):
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d)) / math.sqrt(d)
    wgu = rng.normal(size=(E, 2 * f, d)) / math.sqrt(d)
    wd = rng.normal(size=(E, d, f)) / math.sqrt(f)
    sgu = rng.normal(size=(2 * fs, d)) / math.sqrt(d) if fs else None
    sd = rng.normal(size=(d, fs)) / math.sqrt(fs) if fs else None
    return x, wr, wgu, wd, sgu, sd


def test_k_equals_E_without_capacity_is_the_dense_mixture():
    rng = np.random.default_rng(5)
    T, d, E, f = 12, 16, 5, 24
    x, wr, wgu, wd, _, _ = _layer(rng, T, d, E, f)
    out = oracle.moe_forward(x, wr, wgu, wd, top_k=E, cap=None)["out"]
    # dense MoE: every expert processes every token, weighted by its router probability
    logits = x @ wr.T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dense = np.zeros((T, d))
    for e in range(E):
        dense += p[:, e:e + 1] * oracle.swiglu_ffn(x, wgu[e], wd[e])
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-13)


def test_single_expert_reduces_to_one_ffn():
    rng = np.random.default_rng(6)
    T, d, f = 10, 16, 8
    x, wr, wgu, wd, _, _ = _layer(rng, T, d, 1, f)
    torch = pytest.importorskip("torch")
    out = oracle.moe_forward(x, wr, wgu, wd, top_k=1, cap=None)["out"]
    g, u = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(wgu[0])).chunk(2, dim=-1)
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, torch.from_numpy(wd[0])).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_dropped_tokens_get_exactly_zero_or_the_shared_expert():
    rng = np.random.default_rng(8)
    T, d, E, f = 6, 8, 2, 8
    x, wr, wgu, wd, sgu, sd = _layer(rng, T, d, E, f, fs=8)
    off = np.array([50.0, 0.0])  # everyone picks expert 0 first
    r = oracle.moe_forward(x, wr, wgu, wd, top_k=1, cap=2, logit_offset=off)
    assert r["ids"][:, 0].tolist() == [0] * T
    assert r["slot"][:, 0].tolist() == [0, 1, -1, -1, -1, -1]
    assert np.all(r["out"][2:] == 0.0)
    assert np.all(r["out"][:2] != 0.0)
    rs = oracle.moe_forward(x, wr, wgu, wd, top_k=1, cap=2, logit_offset=off, w_shared_gate_up=sgu, w_shared_down=sd)
    sh = oracle.swiglu_ffn(x, sgu, sd)
    assert np.array_equal(rs["out"][2:], sh[2:])
    # k = 2: the token keeps its second assignment when the first is dropped
    r2 = oracle.moe_forward(x, wr, wgu, wd, top_k=2, cap=2, logit_offset=off)
    assert r2["slot"][:, 1].tolist() == [0, 1, -1, -1, -1, -1]


def test_expert_relabelling_leaves_output_unchanged():
    rng = np.random.default_rng(9)
    T, d, E, f = 40, 16, 6, 8
    x, wr, wgu, wd, _, _ = _layer(rng, T, d, E, f)
    perm = rng.permutation(E)
    for k, cap in ((1, 5), (2, 9), (3, None)):
        a = oracle.moe_forward(x, wr, wgu, wd, top_k=k, cap=cap)["out"]
        b = oracle.moe_forward(x, wr[perm], wgu[perm], wd[perm], top_k=k, cap=cap)["out"]
        assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


def test_token_subset_matches_full_batch():
    rng = np.random.default_rng(10)
    T, d, E, f = 30, 8, 4, 8
    x, wr, wgu, wd, sgu, sd = _layer(rng, T, d, E, f, fs=4)
    full = oracle.moe_forward(x, wr, wgu, wd, top_k=2, cap=9, w_shared_gate_up=sgu, w_shared_down=sd)
    sub = [29, 3, 17, 0]
    part = oracle.moe_forward(x, wr, wgu, wd, top_k=2, cap=9, w_shared_gate_up=sgu, w_shared_down=sd, tokens=sub)
    assert np.allclose(part["out"], full["out"][sub], rtol=1e-14, atol=1e-15)


def test_aux_loss_uniform_routing_gives_alpha():
    E, T = 8, 64
    logits = np.zeros((T, E))
    ids = (np.arange(T) % E).reshape(-1, 1)
    assert oracle.aux_load_balancing_loss(ids, oracle.softmax(logits), E, alpha=0.01) == pytest.approx(0.01, rel=1e-15)
    # all tokens on one expert with a one-hot router: f = P = e_0, loss = alpha * E
    onehot = np.full((T, E), -1e4)
    onehot[:, 0] = 0.0
    ids0 = np.zeros((T, 1), dtype=np.int64)
    assert oracle.aux_load_balancing_loss(ids0, oracle.softmax(onehot), E, alpha=0.01) == pytest.approx(0.08, rel=1e-12)
