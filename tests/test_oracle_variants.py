"""Pins of the oracle's capacity-fill variants: capacity with a top-k factor, the
rank-major ("slot") fill order, and redirection of overflowing assignments to the
token's next most suitable expert.

As for the base path, nothing here compares the oracle with itself: hand-worked
tiny cases, closed forms, brute-force counts written in a different form, and
invariants the readings imply.  CPU only.
"""
import numpy as np
import pytest

import oracle


# --------------------------------------------------------------------------------------------
# Capacity with a top-k factor
# --------------------------------------------------------------------------------------------

def test_capacity_topk_closed_forms():
    assert oracle.capacity_topk(8, 4, 2, 1.0) == 4
    assert oracle.capacity_topk(32, 8, 2, 1.0) == 8
    assert oracle.capacity_topk(32, 8, 2, 1.25) == 10
    assert oracle.capacity_topk(16384, 256, 8, 1.25) == 640
    assert oracle.capacity_topk(64, 8, 2, 1.25) == 20
    assert oracle.capacity_topk(5, 3, 2, 1.0) == 4   # 10 / 3 rounds up
    assert oracle.capacity_topk(10, 4, 2, None) is None
    assert oracle.capacity_topk(10, 4, 2, 0.0) is None


def test_capacity_topk_with_k1_is_the_base_formula():
    rng = np.random.default_rng(3)
    for _ in range(200):
        T, E = int(rng.integers(1, 5000)), int(rng.integers(1, 300))
        cf = float(rng.uniform(0.05, 3.0))
        assert oracle.capacity_topk(T, E, 1, cf) == oracle.capacity(T, E, cf)


# --------------------------------------------------------------------------------------------
# Rank-major fill order
# --------------------------------------------------------------------------------------------

def test_slot_major_hand_worked():
    ids = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    # visit order (t, j): (0,0) e0, (1,0) e1, (2,0) e0, (0,1) e1, (1,1) e0, (2,1) e1; C = 2
    f = oracle.capacity_fill(ids, 2, 2, order="slot")
    assert f["slot"].tolist() == [[0, 1], [0, -1], [1, -1]]
    assert f["row_token"].tolist() == [0, 2, 1, 0]
    assert f["kept"].tolist() == [2, 2] and f["drops"] == 2
    g = oracle.capacity_fill(ids, 2, 2, order="token")
    assert g["slot"].tolist() == [[0, 0], [1, 1], [-1, -1]]


def _random_ids(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def test_slot_major_equals_token_major_for_top1():
    rng = np.random.default_rng(0)
    for _ in range(20):
        T, E = int(rng.integers(1, 60)), int(rng.integers(1, 9))
        ids = rng.integers(0, E, (T, 1)).astype(np.int32)
        cap = int(rng.integers(1, 10))
        a = oracle.capacity_fill(ids, E, cap, order="token")
        b = oracle.capacity_fill(ids, E, cap, order="slot")
        for key in ("counts", "kept", "offsets", "slot", "row_token"):
            np.testing.assert_array_equal(a[key], b[key])


def test_slot_major_matches_vectorised_count():
    """slot(t, j) = #{(t', j') with the same expert and (j' < j, or j' = j and t' < t)},
    kept iff below C -- counted with array operations instead of a walk."""
    rng = np.random.default_rng(1)
    for _ in range(30):
        T, E = int(rng.integers(1, 40)), int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        ids = _random_ids(rng, T, E, k)
        cap = int(rng.integers(1, 12))
        f = oracle.capacity_fill(ids, E, cap, order="slot")
        tt, jj = np.meshgrid(np.arange(T), np.arange(k), indexing="ij")
        for t in range(T):
            for j in range(k):
                earlier = (ids == ids[t, j]) & ((jj < j) | ((jj == j) & (tt < t)))
                n = int(earlier.sum())
                assert f["slot"][t, j] == (n if n < cap else -1)


def test_slot_major_protects_first_choices():
    """Under the rank-major order an expert keeps a second-or-later choice only after it
    has kept every first choice made for it."""
    rng = np.random.default_rng(2)
    for _ in range(30):
        T, E, k = int(rng.integers(5, 50)), int(rng.integers(2, 9)), 2
        k = min(k, E)
        ids = _random_ids(rng, T, E, k)
        cap = int(rng.integers(1, 8))
        f = oracle.capacity_fill(ids, E, cap, order="slot")
        for e in range(E):
            first = f["slot"][:, 0][ids[:, 0] == e]
            later_kept = (f["slot"][:, 1:][ids[:, 1:] == e] >= 0).any()
            if later_kept:
                assert (first >= 0).all()


# --------------------------------------------------------------------------------------------
# Redirection of overflowing assignments
# --------------------------------------------------------------------------------------------

def test_reroute_hand_worked_two_passes():
    logits = np.array([[3.0, 2.0, 1.0],
                       [3.0, 1.0, 2.0],
                       [3.0, 2.0, 1.0],
                       [1.0, 3.0, 2.0]])
    ids = oracle.topk_select(logits, 1)
    assert ids[:, 0].tolist() == [0, 0, 0, 1]
    f = oracle.capacity_fill_reroute(ids, logits, 3, 1)
    # pass 1: t0 -> e0, t3 -> e1, t1 and t2 overflow; pass 2: t1 offered e2 (room), t2
    # offered e1 (filled by t3 in pass 1) -> dropped
    assert f["slot"][:, 0].tolist() == [0, 0, -1, 0]
    assert f["assigned"][:, 0].tolist() == [0, 2, 0, 1]
    assert f["kept"].tolist() == [1, 1, 1]
    assert f["offsets"].tolist() == [0, 1, 2, 3]
    assert f["row_token"].tolist() == [0, 3, 1]
    assert f["counts"].tolist() == [3, 1, 0]
    assert f["drops"] == 1 and f["rerouted"] == 1


def test_reroute_second_overflow_takes_the_next_rank():
    # one token, k = 2, E = 4, both chosen experts full (C = 1 taken by earlier tokens)
    logits = np.array([[5.0, 4.0, 0.0, 0.0],     # t0 takes e0 and e1
                       [5.0, 4.0, 3.0, 2.0]])    # t1 overflows twice -> e2, then e3
    ids = oracle.topk_select(logits, 2)
    f = oracle.capacity_fill_reroute(ids, logits, 4, 1)
    assert f["slot"].tolist() == [[0, 0], [0, 0]]
    assert f["assigned"].tolist() == [[0, 1], [2, 3]]
    assert f["row_token"].tolist() == [0, 0, 1, 1]


def test_reroute_without_a_spare_expert_drops():
    logits = np.array([[2.0, 1.0], [2.0, 1.0], [2.0, 1.0]])
    ids = oracle.topk_select(logits, 2)             # k = E: no expert left to offer
    f = oracle.capacity_fill_reroute(ids, logits, 2, 1)
    g = oracle.capacity_fill(ids, 2, 1)
    np.testing.assert_array_equal(f["slot"], g["slot"])
    assert f["rerouted"] == 0


def _ranked(rng, T, E):
    # distinct logits per row so that the router order is unique
    return np.stack([rng.permutation(E) + rng.uniform(0, 0.5, E) for _ in range(T)])


@pytest.mark.parametrize("order", ["token", "slot"])
def test_reroute_invariants(order):
    rng = np.random.default_rng(4)
    for _ in range(40):
        T, E = int(rng.integers(1, 50)), int(rng.integers(2, 10))
        k = int(rng.integers(1, E + 1))
        logits = _ranked(rng, T, E)
        ids = oracle.topk_select(logits, k)
        cap = int(rng.integers(1, 10))
        drop = oracle.capacity_fill(ids, E, cap, order)
        f = oracle.capacity_fill_reroute(ids, logits, E, cap, order)
        ranking = np.argsort(-logits, axis=1)
        # the first pass is the drop policy, untouched
        first = drop["slot"] >= 0
        np.testing.assert_array_equal(f["slot"][first], drop["slot"][first])
        np.testing.assert_array_equal(f["assigned"][first], ids[first])
        assert (f["kept"] <= cap).all()
        assert (f["kept"] >= drop["kept"]).all()
        assert f["kept"].sum() == drop["kept"].sum() + f["rerouted"]
        np.testing.assert_array_equal(f["counts"], drop["counts"])
        for t in range(T):
            over = [j for j in range(k) if not first[t, j]]
            for i, j in enumerate(over):
                if f["slot"][t, j] >= 0:
                    assert f["assigned"][t, j] == ranking[t, k + i]
                    assert f["slot"][t, j] >= drop["kept"][f["assigned"][t, j]]
                else:
                    assert f["assigned"][t, j] == ids[t, j]
            kept_experts = [int(f["assigned"][t, j]) for j in range(k) if f["slot"][t, j] >= 0]
            assert len(kept_experts) == len(set(kept_experts))
        # rows: every kept assignment appears once, at its expert's offset plus its slot
        seen = np.zeros(len(f["row_token"]), dtype=int)
        for t in range(T):
            for j in range(k):
                if f["slot"][t, j] >= 0:
                    r = f["offsets"][f["assigned"][t, j]] + f["slot"][t, j]
                    assert f["row_token"][r] == t
                    seen[r] += 1
        assert (seen == 1).all()


def test_reroute_second_pass_keeps_the_first_offers_in_fill_order():
    """Per expert, the redirected assignments kept are the first (C - kept after pass 1)
    offered to it in fill order -- counted with a sort instead of a walk."""
    rng = np.random.default_rng(5)
    for _ in range(30):
        T, E, k = int(rng.integers(2, 60)), int(rng.integers(3, 10)), 2
        logits = _ranked(rng, T, E)
        ids = oracle.topk_select(logits, k)
        cap = int(rng.integers(1, 8))
        drop = oracle.capacity_fill(ids, E, cap)
        f = oracle.capacity_fill_reroute(ids, logits, E, cap)
        ranking = np.argsort(-logits, axis=1)
        over = drop["slot"] < 0
        nth = np.cumsum(over, axis=1) - 1
        rank = k + np.maximum(nth, 0)
        offered = np.where(over & (rank < E), ranking[np.arange(T)[:, None], np.minimum(rank, E - 1)], -1)
        for e in range(E):
            pos = np.flatnonzero(offered.reshape(-1) == e)       # token-major positions, in order
            room = cap - int(drop["kept"][e])
            keep = pos[:room]
            got = np.flatnonzero(((f["assigned"] == e) & ~(drop["slot"] >= 0) & (f["slot"] >= 0)).reshape(-1))
            np.testing.assert_array_equal(np.sort(got), keep)


def test_reroute_with_ample_capacity_is_the_drop_policy():
    rng = np.random.default_rng(6)
    T, E, k = 40, 6, 2
    logits = _ranked(rng, T, E)
    ids = oracle.topk_select(logits, k)
    for cap in (None, T):
        f = oracle.capacity_fill_reroute(ids, logits, E, cap)
        g = oracle.capacity_fill(ids, E, cap)
        for key in ("counts", "kept", "offsets", "slot", "row_token"):
            np.testing.assert_array_equal(f[key], g[key])
        np.testing.assert_array_equal(f["assigned"], ids)


def test_forward_with_reroute_uses_the_serving_expert():
    """k = 1 (gate 1): each token's output is the FFN of the expert that served it, which
    for redirected tokens is their second-ranked expert."""
    rng = np.random.default_rng(7)
    T, d, E, f_ = 6, 8, 4, 4
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((E, d))
    off = np.array([10.0, 0.0, 0.0, 0.0])       # every token picks expert 0
    gu = rng.standard_normal((E, 2 * f_, d))
    dn = rng.standard_normal((E, d, f_))
    res = oracle.moe_forward(x, w_r, gu, dn, 1, 2, logit_offset=off, overflow="reroute")
    logits = x @ w_r.T + off
    second = np.argsort(-logits, axis=1)[:, 1]
    fill_second = {}
    for t in range(T):
        if t < 2:
            want = oracle.swiglu_ffn(x[t:t + 1], gu[0], dn[0])[0]
        else:
            e = int(second[t])
            n = fill_second.get(e, 0)
            if n < 2:
                fill_second[e] = n + 1
                want = oracle.swiglu_ffn(x[t:t + 1], gu[e], dn[e])[0]
            else:
                want = np.zeros(d)
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-12, atol=1e-12)


def test_forward_slot_major_k1_equals_token_major():
    rng = np.random.default_rng(8)
    T, d, E, f_ = 12, 8, 3, 4
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((E, d))
    gu = rng.standard_normal((E, 2 * f_, d))
    dn = rng.standard_normal((E, d, f_))
    a = oracle.moe_forward(x, w_r, gu, dn, 1, 2)
    b = oracle.moe_forward(x, w_r, gu, dn, 1, 2, fill_order="slot")
    np.testing.assert_array_equal(a["out"], b["out"])
