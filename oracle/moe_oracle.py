"""CPU oracle for the forward pass of a sparse Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library and never
imports it.  It is deliberately plain and slow: NumPy in float64, one stage per
function, a per-token sequential capacity fill, one matmul per expert.

Sources (web pages; cited by title and section):
  [SMoE]  "Sparse Mixture-of-Experts", bigdataschool.ru wiki
          (sections "Роутер и top-k gating", "Expert capacity и capacity factor",
          "Маршрутизация токена и auxiliary loss", "Top-1 routing в Switch
          Transformer против top-2 в GShard", "Подводные камни collapse экспертов
          и token dropping", "Демо top-k router на PyTorch").
  [HF-MoE] "Что такое Mixture of Experts (MoE) в трансформерах: архитектура и
          параллелизм", aglamov.biz (sections "Рефакторинг загрузки весов",
          "Бэкенд для экспертов (Expert Backend)").
  [GW]    "Архитектура MoE в больших языковых моделях — кто такие «эксперты»?",
          gerwin.io (sections "Как работает MoE: принцип маршрутизации",
          "Обратная сторона медали: недостатки и сложности MoE").

The backward pass (``moe_backward``) is the plain chain-rule derivative of these
steps with the routing held fixed.

The steps, in order:
  1. router logits  l_t = W_r x_t (+ optional per-expert offset)   [SMoE, router]
  2. softmax over experts, in float64                               [SMoE, router]
  3. top-k: the k experts with the largest probability; equal values go to
     the lower expert index                                          [SMoE, router]
  4. gates: the selected probabilities renormalised to sum to one    [SMoE, router]
  5. capacity C = ceil(capacity_factor * T / E)                      [SMoE, capacity]
  6. first-come capacity fill in token order; overflow assignments
     are dropped and contribute nothing                              [SMoE, capacity; collapse]
  7. expert FFN, bias-free SwiGLU with the gate half first in the
     packed gate_up weight                                           [HF-MoE, weight loading]
  8. gate-weighted sum of the kept expert outputs (plus an always-on
     shared expert when one is given)                                [SMoE, router; GW, drawbacks item 5]

Readings where the pages are silent or garbled are listed in the repository's
design notes; each one is also stated next to the code that takes it.

Parity status: every function below is pinned by CPU tests against values the
pages print, closed forms, brute force or an independent library routine,
except `moe_forward` at large sizes, whose end-to-end numbers the pages never
print (there it is checked only through its pinned stages).
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

__all__ = [
    "capacity",
    "capacity_topk",
    "router_logits",
    "softmax",
    "topk_select",
    "topk_gates",
    "capacity_fill",
    "capacity_fill_reroute",
    "silu",
    "swiglu_ffn",
    "combine",
    "moe_forward",
    "aux_load_balancing_loss",
    "active_params",
    "silu_grad",
    "swiglu_ffn_backward",
    "topk_gates_backward",
    "moe_backward",
]


def capacity(num_tokens: int, num_experts: int, capacity_factor: Optional[float]) -> Optional[int]:
    """Expert capacity: capacity_factor times tokens in the batch, divided by the
    number of experts, rounded up ([SMoE], "Expert capacity и capacity factor";
    the demo evaluates exactly ``ceil(cf * T / E)`` in double precision, in that
    order).  ``None`` (or a factor <= 0) means no capacity limit.

    Reading: the formula carries no top-k factor, also for k > 1.
    """
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.ceil(capacity_factor * num_tokens / num_experts))


def capacity_topk(num_tokens: int, num_experts: int, top_k: int, capacity_factor: Optional[float]) -> Optional[int]:
    """Capacity variant with a top-k factor: the same rounded-up quotient with the
    batch counted in assignments (k per token) instead of tokens,
    ``ceil(cf * (k * T) / E)`` in double precision ([SMoE], "Expert capacity и
    capacity factor" gives the formula for a batch of tokens; with k > 1 each token
    brings k assignments).  ``None`` (or a factor <= 0) means no capacity limit.
    """
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.ceil(capacity_factor * (top_k * num_tokens) / num_experts))


def router_logits(x, w_router, logit_offset=None) -> np.ndarray:
    """Bias-free linear router: logits[t, e] = sum_i W_r[e, i] * x[t, i]
    ([SMoE], "Роутер и top-k gating"; the demo's gate is a Linear with no bias).

    ``logit_offset`` [E] is a synthetic per-expert shift used only to create
    skewed load in test workloads; it is added to every token's logits.
    Computed in float64 from the exact input values.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_router, dtype=np.float64)
    logits = x64 @ w64.T
    if logit_offset is not None:
        logits = logits + np.asarray(logit_offset, dtype=np.float64)[None, :]
    return logits


def softmax(logits) -> np.ndarray:
    """Row softmax in float64 ([SMoE], "Роутер и top-k gating")."""
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l, axis=-1, keepdims=True)
    z = np.exp(l - m)
    return z / np.sum(z, axis=-1, keepdims=True)


def topk_select(logits, k: int) -> np.ndarray:
    """Indices of the k experts with the highest router probability per token,
    in descending order ([SMoE], "Роутер и top-k gating").

    Softmax is strictly increasing in the logit, so ranking logits ranks
    probabilities; ranking the logits also keeps distinct logits distinct.
    Reading: equal logits go to the lower expert index (a stable sort of the
    negated logits).  Returns int32 [T, k].
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-l, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def topk_gates(logits, ids) -> np.ndarray:
    """Renormalised gate weights: the selected softmax probabilities divided by
    their sum so they add up to one ([SMoE], "Роутер и top-k gating").

    Reading: gates are fixed before capacity is applied; a dropped assignment
    keeps its gate but contributes nothing.  For k = 1 every gate is 1.
    """
    p = softmax(logits)
    ids = np.asarray(ids)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / np.sum(sel, axis=1, keepdims=True)


def fill_sequence(num_tokens: int, top_k: int, order: str = "token"):
    """The assignments (t, j) in the order the capacity fill visits them.

    ``"token"``: token-major, token t before token t+1 and, within a token, its
    experts in rank order ([SMoE], "Подводные камни collapse экспертов и token
    dropping": buffers fill in batch order, so late tokens are dropped).
    ``"slot"``: rank-major, every token's first choice before any second choice
    (a priority variant in which a token's top choice never loses its place to
    another token's lower-ranked choice).
    """
    if order == "token":
        return [(t, j) for t in range(num_tokens) for j in range(top_k)]
    if order == "slot":
        return [(t, j) for j in range(top_k) for t in range(num_tokens)]
    raise ValueError("order must be 'token' or 'slot'")


def _rows_by_expert(ids, slot, num_experts: int, kept) -> tuple:
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_token = np.full(int(offsets[-1]), -1, dtype=np.int32)
    T, k = slot.shape
    for t in range(T):
        for j in range(k):
            if slot[t, j] >= 0:
                row_token[offsets[int(ids[t, j])] + slot[t, j]] = t
    return offsets, row_token


def capacity_fill(ids, num_experts: int, cap: Optional[int], order: str = "token") -> dict:
    """Sequential first-come capacity fill ([SMoE], "Expert capacity и capacity
    factor": tokens reaching a full expert are not processed; "Подводные камни
    collapse экспертов и token dropping": tokens late in the batch are dropped more
    often; the demo walks tokens in batch order and gives each one the next free
    slot of its expert while slots remain).

    Readings: for k > 1 the walk is token-major over the [T, k] assignment table
    (``order="token"``, the default; ``"slot"`` is the rank-major variant, see
    ``fill_sequence``); dropping is per (token, expert) assignment.

    Returns a dict with
      counts   [E] int64  demand per expert (all assignments, kept or not)
      kept     [E] int64  kept assignments per expert = min(counts, cap)
      offsets  [E+1] int64 exclusive prefix sum of ``kept``
      slot     [T, k] int32 position inside the expert's buffer, -1 if dropped
      row_token [R] int32  token of each kept row, rows ordered by (expert, slot),
                          i.e. by expert and then in fill order
      drops    int        number of dropped assignments
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    fill = [0] * num_experts
    counts = [0] * num_experts
    slot = np.full((T, k), -1, dtype=np.int32)
    drops = 0
    for t, j in fill_sequence(T, k, order):
        e = int(ids[t, j])
        counts[e] += 1
        if cap is None or fill[e] < cap:
            slot[t, j] = fill[e]
            fill[e] += 1
        else:
            drops += 1
    kept = np.array(fill, dtype=np.int64)
    offsets, row_token = _rows_by_expert(ids, slot, num_experts, kept)
    return {
        "counts": np.array(counts, dtype=np.int64),
        "kept": kept,
        "offsets": offsets,
        "slot": slot,
        "row_token": row_token,
        "drops": drops,
    }


def capacity_fill_reroute(ids, logits, num_experts: int, cap: Optional[int], order: str = "token") -> dict:
    """Capacity fill in which an overflowing assignment is redirected to the token's
    next most suitable expert instead of being dropped outright ([GW], "Как работает
    MoE: принцип маршрутизации", load-balancing item 4: exceeding an expert's capacity
    leads to dropping the token or sending it on to the next best expert).

    Readings (the page names the option and nothing more):
      * Two passes.  The first is the plain fill of ``capacity_fill``; no token's
        own top-k choice is ever displaced by a redirected one, so the assignments
        kept by the first pass are exactly those of the drop policy.
      * The token's i-th overflowing assignment (i = 0, 1, ... in rank order j) is
        offered to the expert ranked k + i in the token's router order (descending
        logit, equal logits to the lower index), which the token does not use yet;
        if k + i >= E there is none and the assignment is dropped.
      * The second pass visits the offered assignments in the same fill order and
        gives each the next free slot of its new expert while the expert has room
        left after the first pass; otherwise it is dropped.  Rows of an expert: its
        first-pass rows, then its redirected rows.
      * An assignment keeps its gate (gates are fixed before capacity applies).
    Returns the ``capacity_fill`` keys (``counts`` stays the router's demand) plus
      assigned [T, k] int32  expert that serves each assignment (the router's
                             choice unless redirected)
      rerouted int           number of assignments kept by the second pass
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    first = capacity_fill(ids, num_experts, cap, order)
    assigned = ids.astype(np.int32).copy()
    slot = first["slot"].copy()
    if cap is None:
        return {**first, "assigned": assigned, "rerouted": 0}
    ranking = np.argsort(-np.asarray(logits, dtype=np.float64), axis=1, kind="stable")
    offered = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        i = 0
        for j in range(k):
            if slot[t, j] < 0:
                if k + i < num_experts:
                    offered[t, j] = ranking[t, k + i]
                i += 1
    fill = [int(v) for v in first["kept"]]
    rerouted = 0
    for t, j in fill_sequence(T, k, order):
        e = int(offered[t, j])
        if e >= 0 and fill[e] < cap:
            slot[t, j] = fill[e]
            fill[e] += 1
            assigned[t, j] = e
            rerouted += 1
    kept = np.array(fill, dtype=np.int64)
    offsets, row_token = _rows_by_expert(assigned, slot, num_experts, kept)
    return {
        "counts": first["counts"],
        "kept": kept,
        "offsets": offsets,
        "slot": slot,
        "row_token": row_token,
        "drops": int((slot < 0).sum()),
        "assigned": assigned,
        "rerouted": rerouted,
    }


def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(x_rows, w_gate_up, w_down) -> np.ndarray:
    """One expert's bias-free SwiGLU FFN in float64.

    Packed layout ([HF-MoE], "Рефакторинг загрузки весов": per-expert w1 and w3
    are concatenated into ``gate_up_proj``, w1 listed first; w2 is
    ``down_proj``):
      w_gate_up [2f, d]: rows 0..f-1 are the gate projection, rows f..2f-1 the up
      projection; w_down [d, f].
      y = (silu(x W_g^T) * (x W_u^T)) W_d^T
    """
    X = np.asarray(x_rows, dtype=np.float64)
    Wgu = np.asarray(w_gate_up, dtype=np.float64)
    Wd = np.asarray(w_down, dtype=np.float64)
    f = Wd.shape[1]
    if Wgu.shape[0] != 2 * f:
        raise ValueError("w_gate_up must have 2*d_ff rows")
    g = X @ Wgu[:f].T
    u = X @ Wgu[f:].T
    h = silu(g) * u
    return h @ Wd.T


def combine(num_tokens: int, d_model: int, ids, gates, slot, expert_rows: Callable[[int, int], np.ndarray],
            shared=None, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Gate-weighted sum of the kept expert outputs per token ([SMoE],
    "Роутер и top-k gating": the layer output is the weighted sum of the chosen
    experts' outputs; "Expert capacity и capacity factor": a dropped token gets
    nothing from the MoE sublayer).

    ``expert_rows(t, j)`` returns the expert output row for assignment (t, j).
    ``shared`` [T, d] is an always-on shared expert output added with weight 1
    ([GW], drawbacks item 5, shared-expert isolation).  Terms are summed in
    rank order j = 0..k-1.  ``tokens`` restricts the computation to a subset;
    the result then has one row per listed token.
    """
    toks = range(num_tokens) if tokens is None else list(tokens)
    out = np.zeros((len(toks), d_model), dtype=np.float64)
    for r, t in enumerate(toks):
        if shared is not None:
            out[r] += np.asarray(shared[t], dtype=np.float64)
        for j in range(ids.shape[1]):
            if slot[t, j] >= 0:
                out[r] += gates[t, j] * expert_rows(t, j)
    return out


def _expert(w, e) -> np.ndarray:
    return np.asarray(w[e], dtype=np.float64)


def moe_forward(x, w_router, w_gate_up, w_down, top_k: int, cap: Optional[int], logit_offset=None,
                w_shared_gate_up=None, w_shared_down=None, tokens: Optional[Sequence[int]] = None,
                ids=None, fill_order: str = "token", overflow: str = "drop") -> dict:
    """The whole layer: route, fill, expert FFNs, combine.

    ``w_gate_up`` / ``w_down`` may be any object whose ``[e]`` item converts to
    a float64 array (so a caller can hand over experts lazily).  ``tokens``
    limits the FFN and combine to a subset of tokens; routing and the capacity
    fill always run over the whole batch, since a token's slot depends on every
    earlier token.  ``ids`` overrides the top-k choice (the gates are still the
    renormalised probabilities of the given experts); it lets a comparison
    absorb near-tie routing differences.  ``fill_order`` ("token" or "slot") and
    ``overflow`` ("drop" or "reroute") select the capacity-fill variant
    (``capacity_fill`` / ``capacity_fill_reroute``).
    """
    x64 = np.asarray(x, dtype=np.float64)
    T, d = x64.shape
    E = np.asarray(w_router).shape[0]
    logits = router_logits(x64, w_router, logit_offset)
    if ids is None:
        ids = topk_select(logits, top_k)
    ids = np.asarray(ids, dtype=np.int32)
    gates = topk_gates(logits, ids)
    if overflow == "drop":
        fill = capacity_fill(ids, E, cap, fill_order)
        serving = ids
    elif overflow == "reroute":
        fill = capacity_fill_reroute(ids, logits, E, cap, fill_order)
        serving = fill["assigned"]
    else:
        raise ValueError("overflow must be 'drop' or 'reroute'")
    slot = fill["slot"]
    toks = list(range(T)) if tokens is None else [int(t) for t in tokens]

    # Expert outputs for the assignments of the requested tokens, one expert at a time.
    need = {}
    for t in toks:
        for j in range(top_k):
            if slot[t, j] >= 0:
                need.setdefault(int(serving[t, j]), []).append((t, j))
    rows = {}
    for e in sorted(need):
        X = x64[[t for t, _ in need[e]]]
        Y = swiglu_ffn(X, _expert(w_gate_up, e), _expert(w_down, e))
        for r, tj in enumerate(need[e]):
            rows[tj] = Y[r]

    shared = None
    if w_shared_gate_up is not None:
        sh = swiglu_ffn(x64[toks], w_shared_gate_up, w_shared_down)
        shared = {t: sh[r] for r, t in enumerate(toks)}

    out = combine(T, d, ids, gates, slot, lambda t, j: rows[(t, j)], shared=shared, tokens=toks)
    return {
        "out": out,
        "tokens": np.array(toks, dtype=np.int64),
        "logits": logits,
        "ids": ids,
        "gates": gates,
        **fill,
    }


def aux_load_balancing_loss(ids, probs, num_experts: int, alpha: float = 1e-2) -> float:
    """Switch-style auxiliary load-balancing loss alpha * N * sum_i f_i * P_i
    ([SMoE], "Маршрутизация токена и auxiliary loss"): f_i is the fraction of
    the batch's assignments routed to expert i (by router choice, before
    capacity, as in the demo), P_i the router probability of expert i averaged
    over the batch.

    Reading for k > 1: f_i divides by the T*k assignments so that sum_i f_i = 1;
    for k = 1 this is the page's formula exactly.
    """
    ids = np.asarray(ids)
    p = np.asarray(probs, dtype=np.float64)
    T = p.shape[0]
    f = np.bincount(ids.reshape(-1), minlength=num_experts).astype(np.float64) / ids.size
    P = p.mean(axis=0)
    return float(alpha * num_experts * np.sum(f * P)) if T else 0.0


def silu_grad(z) -> np.ndarray:
    """d/dz silu(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z))), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def swiglu_ffn_backward(x_rows, w_gate_up, w_down, dy_rows, scale=None) -> dict:
    """Gradient of one expert's SwiGLU FFN (``swiglu_ffn``) summed over its rows,
    each row's output weighted by ``scale`` (its gate; 1 when omitted):
        out_r = scale_r * y_r,  y = (silu(X W_g^T) * (X W_u^T)) W_d^T.
    Returns dx [n, d], dw_gate_up [2f, d], dw_down [d, f] and dscale [n] (= dy_r . y_r),
    by the chain rule, float64.  The training setting is the pages' ([HF-MoE],
    "Обучение MoE с помощью Transformers": the expert projections run as grouped
    GEMMs in training as well); the gradient itself is the plain derivative.
    """
    X = np.asarray(x_rows, dtype=np.float64)
    Wgu = np.asarray(w_gate_up, dtype=np.float64)
    Wd = np.asarray(w_down, dtype=np.float64)
    dY = np.asarray(dy_rows, dtype=np.float64)
    n, f = X.shape[0], Wd.shape[1]
    c = np.ones(n) if scale is None else np.asarray(scale, dtype=np.float64)
    G = X @ Wgu[:f].T
    U = X @ Wgu[f:].T
    H = silu(G) * U
    Y = H @ Wd.T
    dscale = np.sum(dY * Y, axis=1)
    dYs = dY * c[:, None]                 # gradient reaching y_r
    dH = dYs @ Wd                         # [n, f]
    dG = dH * U * silu_grad(G)
    dU = dH * silu(G)
    dx = dG @ Wgu[:f] + dU @ Wgu[f:]
    dw_gate_up = np.concatenate([dG.T @ X, dU.T @ X], axis=0)
    dw_down = dYs.T @ H
    return {"dx": dx, "dw_gate_up": dw_gate_up, "dw_down": dw_down, "dscale": dscale}


def topk_gates_backward(logits, ids, dgates) -> np.ndarray:
    """Gradient of the renormalised top-k gates with respect to the router logits.
    The gates are a softmax over the selected logits (``topk_gates``), so for the
    selected experts dl_j = g_j * (dg_j - sum_j' g_j' dg_j') and dl = 0 for the
    others (the selection itself is piecewise constant).  Returns dlogits [T, E]."""
    l = np.asarray(logits, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    g = topk_gates(l, ids)
    dg = np.asarray(dgates, dtype=np.float64)
    dsel = g * (dg - np.sum(g * dg, axis=1, keepdims=True))
    dl = np.zeros_like(l)
    np.put_along_axis(dl, ids, dsel, axis=1)
    return dl


def moe_backward(x, w_router, w_gate_up, w_down, top_k: int, cap: Optional[int], dy, logit_offset=None,
                 w_shared_gate_up=None, w_shared_down=None, ids=None, fill_order: str = "token",
                 overflow: str = "drop") -> dict:
    """Gradient of ``moe_forward``'s output, contracted with ``dy`` [T, d], with respect
    to x, the router weight and every expert weight, float64.

    Routing (top-k choice, capacity slots, drops, redirection) is piecewise constant
    and taken as fixed; gradients flow through the gates, the expert FFNs and the shared
    expert.  A dropped assignment contributes nothing, so its gate receives no
    gradient from it (its gate still enters the renormalisation of the others); an
    expert with no kept rows gets zero weight gradients.  ``ids`` overrides the top-k
    choice as in ``moe_forward``.  Returns dx, dw_router, dw_gate_up, dw_down (and
    dw_shared_gate_up / dw_shared_down when a shared expert is given), plus dlogits and
    dgates.
    """
    x64 = np.asarray(x, dtype=np.float64)
    dy64 = np.asarray(dy, dtype=np.float64)
    T, d = x64.shape
    wr = np.asarray(w_router, dtype=np.float64)
    E = wr.shape[0]
    logits = router_logits(x64, wr, logit_offset)
    if ids is None:
        ids = topk_select(logits, top_k)
    ids = np.asarray(ids, dtype=np.int32)
    gates = topk_gates(logits, ids)
    if overflow == "drop":
        fill = capacity_fill(ids, E, cap, fill_order)
        serving = ids
    elif overflow == "reroute":
        fill = capacity_fill_reroute(ids, logits, E, cap, fill_order)
        serving = fill["assigned"]
    else:
        raise ValueError("overflow must be 'drop' or 'reroute'")
    slot = fill["slot"]
    dx = np.zeros((T, d))
    dgates = np.zeros((T, top_k))
    dw_gate_up, dw_down = {}, {}
    rows = {}
    for t in range(T):
        for j in range(top_k):
            if slot[t, j] >= 0:
                rows.setdefault(int(serving[t, j]), []).append((t, j))
    for e in range(E):
        Wgu = _expert(w_gate_up, e)
        Wd = _expert(w_down, e)
        if e not in rows:
            dw_gate_up[e] = np.zeros_like(Wgu)
            dw_down[e] = np.zeros_like(Wd)
            continue
        tj = rows[e]
        toks = [t for t, _ in tj]
        g = np.array([gates[t, j] for t, j in tj])
        b = swiglu_ffn_backward(x64[toks], Wgu, Wd, dy64[toks], scale=g)
        for r, (t, j) in enumerate(tj):
            dx[t] += b["dx"][r]
            dgates[t, j] = b["dscale"][r]
        dw_gate_up[e] = b["dw_gate_up"]
        dw_down[e] = b["dw_down"]
    dlogits = topk_gates_backward(logits, ids, dgates)
    dx += dlogits @ wr
    out = {
        "dx": dx,
        "dw_router": dlogits.T @ x64,
        "dw_gate_up": np.stack([dw_gate_up[e] for e in range(E)]),
        "dw_down": np.stack([dw_down[e] for e in range(E)]),
        "dlogits": dlogits,
        "dgates": dgates,
        "ids": ids,
        "slot": slot,
    }
    if w_shared_gate_up is not None:
        b = swiglu_ffn_backward(x64, w_shared_gate_up, w_shared_down, dy64)
        out["dx"] = out["dx"] + b["dx"]
        out["dw_shared_gate_up"] = b["dw_gate_up"]
        out["dw_shared_down"] = b["dw_down"]
    return out


def active_params(d_model: int, hidden: int, num_experts: int, top_k: int, ffn: str = "swiglu") -> dict:
    """Parameters touched per token: the router plus k experts; total = router
    plus all experts ([SMoE], "Top-1 routing в Switch Transformer против top-2
    в GShard").  ``ffn="relu_bias"`` is the demo's two-layer FFN with biases,
    ``"swiglu"`` the bias-free gate/up/down expert used here."""
    router = num_experts * d_model
    if ffn == "relu_bias":
        expert = d_model * hidden + hidden + hidden * d_model + d_model
    elif ffn == "swiglu":
        expert = 3 * d_model * hidden
    else:
        raise ValueError(ffn)
    return {"active": router + top_k * expert, "total": router + num_experts * expert, "expert": expert}
