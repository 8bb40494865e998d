"""Helpers shared by the GPU parity tests: comparisons against the CPU oracle.

Tolerances (floating point):
  * layer outputs: row-normalised max relative error
        max_t ||got_t - ref_t||_inf / ||ref_t||_inf   over rows with ref_t != 0
    at most 2e-2 for bf16 layers and 1e-5 for float layers; rows whose reference is
    exactly zero (every assignment dropped, no shared expert) must be exactly zero;
  * gates: absolute 1e-6 (float exp on the GPU vs float64 in the oracle);
  * routing: ids may differ from the oracle's float64 choice only for tokens whose
    k-th and (k+1)-th oracle logits are closer than 1e-4; the oracle is then re-run
    with the GPU's ids, which absorbs the resulting capacity cascade.
Integer outputs (ids from identical logits, slots, counts, offsets, row order) are
compared exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BF16_TOL = 2e-2
F32_TOL = 1e-5
GATE_TOL = 1e-6
TIE_GAP = 1e-4


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


class HostExperts:
    """Lazily copies one expert's weights to the host (float64) when the oracle asks."""

    def __init__(self, w: torch.Tensor):
        self.w = w
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = to_np(self.w[e]).astype(np.float64)
        return self.cache[e]


def row_rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    ref_inf = np.abs(ref).max(axis=1) if ref.size else np.zeros(0)
    zero = ref_inf == 0
    if np.any(zero):
        assert np.all(got[zero] == 0.0), "rows whose reference is exactly zero must be exactly zero"
    if np.all(zero):
        return 0.0
    err = np.abs(got - ref).max(axis=1)
    return float((err[~zero] / ref_inf[~zero]).max())


def tol_for(dtype) -> float:
    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


def topk_gap(ref_logits: np.ndarray, k: int) -> np.ndarray:
    E = ref_logits.shape[1]
    if k >= E:
        return np.full(ref_logits.shape[0], np.inf)
    s = -np.sort(-ref_logits, axis=1)
    return s[:, k - 1] - s[:, k]


def check_ids_against_oracle(gpu_ids: np.ndarray, ref_logits: np.ndarray, k: int) -> np.ndarray:
    """Returns the tokens where the GPU's expert set differs from the oracle's; each must be a near tie."""
    ref_ids = oracle.topk_select(ref_logits, k)
    a = np.sort(gpu_ids, axis=1)
    b = np.sort(ref_ids, axis=1)
    differ = np.nonzero(np.any(a != b, axis=1))[0]
    if differ.size:
        gap = topk_gap(ref_logits, k)
        bad = differ[gap[differ] >= TIE_GAP]
        assert bad.size == 0, f"routing differs beyond near ties at tokens {bad[:10]} (gaps {gap[bad[:10]]})"
        # the GPU's choice must itself be a top-k within the tie gap
        for t in differ:
            kth = -np.sort(-ref_logits[t])[k - 1]
            assert np.all(ref_logits[t, gpu_ids[t]] >= kth - TIE_GAP)
    return differ


def check_dispatch_exact(ids: np.ndarray, E: int, cap, counts, offsets, slot, row_token, order="token",
                         logits=None, assigned=None) -> dict:
    """Bit-exact comparison with the oracle's fill; with `logits`, the two-pass fill that
    redirects overflow (and `assigned`, the serving experts, is compared too)."""
    if logits is None:
        ref = oracle.capacity_fill(ids, E, cap, order)
    else:
        ref = oracle.capacity_fill_reroute(ids, logits, E, cap, order)
        assert np.array_equal(np.asarray(assigned), ref["assigned"]), "assigned_ids"
    assert np.array_equal(np.asarray(counts), ref["counts"]), "expert_counts"
    assert np.array_equal(np.asarray(offsets), ref["offsets"]), "expert_offsets"
    assert np.array_equal(np.asarray(slot), ref["slot"]), "slot"
    R = int(ref["offsets"][-1])
    assert np.array_equal(np.asarray(row_token)[:R], ref["row_token"]), "row_token"
    return ref
