"""Strength of the oracle's pins: each plausible mistake planted in the oracle (on the
CPU, via monkeypatch) must make at least one pin in test_oracle_pins.py fail."""
import math

import numpy as np
import pytest

import oracle
import oracle.moe_oracle as M
import tests.test_oracle_pins as pins

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _mut_swap_gate_up(x_rows, w_gate_up, w_down):
    Wgu = np.asarray(w_gate_up, dtype=np.float64)
    f = np.asarray(w_down).shape[1]
    return M.__dict__["_orig_swiglu"](x_rows, np.concatenate([Wgu[f:], Wgu[:f]]), w_down)


def _mut_silu_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _mut_tie_high_index(logits, k):
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[1]
    order = np.argsort(-l[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _mut_no_renorm(logits, ids):
    p = M.softmax(logits)
    return np.take_along_axis(p, np.asarray(ids).astype(np.int64), axis=1)


def _mut_fill_le(ids, num_experts, cap):
    return M.__dict__["_orig_fill"](ids, num_experts, None if cap is None else cap + 1)


def _mut_fill_reverse(ids, num_experts, cap):
    ids = np.asarray(ids)
    r = M.__dict__["_orig_fill"](ids[::-1], num_experts, cap)
    r["slot"] = r["slot"][::-1].copy()
    return r


def _mut_capacity_floor(num_tokens, num_experts, capacity_factor):
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.floor(capacity_factor * num_tokens / num_experts))


def _mut_capacity_other_order(num_tokens, num_experts, capacity_factor):
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.ceil(capacity_factor * (num_tokens / num_experts)))


def _mut_down_transposed(x_rows, w_gate_up, w_down):
    """Reshapes the [d, f] down weight to [f, d] instead of transposing it."""
    X = np.asarray(x_rows, dtype=np.float64)
    Wgu = np.asarray(w_gate_up, dtype=np.float64)
    Wd = np.asarray(w_down, dtype=np.float64)
    f = Wd.shape[1]
    h = M.silu(X @ Wgu[:f].T) * (X @ Wgu[f:].T)
    return h @ Wd.reshape(f, Wd.shape[0])


def _mut_combine_keeps_dropped(num_tokens, d_model, ids, gates, slot, expert_rows, shared=None, tokens=None):
    kept = np.zeros_like(slot)
    return M.__dict__["_orig_combine"](num_tokens, d_model, ids, gates, kept, _safe_rows(expert_rows, ids),
                                       shared=shared, tokens=tokens)


def _safe_rows(expert_rows, ids):
    def f(t, j):
        try:
            return expert_rows(t, j)
        except KeyError:
            return np.ones(1)
    return f


def _mut_offset_sign(x, w_router, logit_offset=None):
    x64 = np.asarray(x, dtype=np.float64)
    l = x64 @ np.asarray(w_router, dtype=np.float64).T
    if logit_offset is not None:
        l = l - np.asarray(logit_offset, dtype=np.float64)[None, :]
    return l


def _mut_router_transposed_weight(x, w_router, logit_offset=None):
    w = np.asarray(w_router, dtype=np.float64)
    x64 = np.asarray(x, dtype=np.float64)
    # a plausible indexing slip: uses the weight's columns in reversed order
    l = x64 @ w[:, ::-1].T
    if logit_offset is not None:
        l = l + np.asarray(logit_offset, dtype=np.float64)[None, :]
    return l


def _mut_aux_no_N(ids, probs, num_experts, alpha=1e-2):
    return M.__dict__["_orig_aux"](ids, probs, num_experts, alpha) / num_experts


MUTANTS = {
    "swap_gate_up": ("swiglu_ffn", _mut_swap_gate_up),
    "silu_sign": ("silu", _mut_silu_sign),
    "tie_high_index": ("topk_select", _mut_tie_high_index),
    "no_renormalisation": ("topk_gates", _mut_no_renorm),
    "fill_less_equal": ("capacity_fill", _mut_fill_le),
    "fill_reverse_order": ("capacity_fill", _mut_fill_reverse),
    "capacity_floor": ("capacity", _mut_capacity_floor),
    "capacity_other_order": ("capacity", _mut_capacity_other_order),
    "down_transposed": ("swiglu_ffn", _mut_down_transposed),
    "combine_keeps_dropped": ("combine", _mut_combine_keeps_dropped),
    "offset_sign": ("router_logits", _mut_offset_sign),
    "router_weight_reversed": ("router_logits", _mut_router_transposed_weight),
    "aux_without_N": ("aux_load_balancing_loss", _mut_aux_no_N),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(M.__dict__, "_orig_swiglu", M.swiglu_ffn)
    monkeypatch.setitem(M.__dict__, "_orig_fill", M.capacity_fill)
    monkeypatch.setitem(M.__dict__, "_orig_combine", M.combine)
    monkeypatch.setitem(M.__dict__, "_orig_aux", M.aux_load_balancing_loss)
    monkeypatch.setattr(M, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for t in PIN_TESTS:
        try:
            t()
        except pytest.skip.Exception:
            continue
        except Exception as exc:  # AssertionError or a shape error both count as caught
            failed.append((t.__name__, type(exc).__name__))
    assert failed, f"mutant {name} passed every pin"
