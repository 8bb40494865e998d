"""Router logits of the pages' worked example (the second demo of "Sparse Mixture-of-Experts",
section "Демо top-k router на PyTorch"), rebuilt from the seeded setup that
tests/golden/demo2_capacity_dropping.json states as data.

The draw depends on torch's CPU generator, which may change between torch versions; the
fixture applies only while the draw reproduces the page.  The guard is a direct count: for
top-1 routing each expert keeps min(n_e, C) tokens, so the balanced router's arg-max
histogram must give the printed drops sum_e max(0, n_e - C) at every printed capacity.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "demo2_capacity_dropping.json")


def demo2_fixture() -> dict:
    with open(GOLDEN) as fh:
        return json.load(fh)


def demo2_router_logits() -> dict:
    """{router name: float64 [T, E] logits} as the demo's seeded draw gives them (float32
    products, widened)."""
    torch = pytest.importorskip("torch")
    g = demo2_fixture()
    st = g["setup"]
    assert st["generator"] == "torch_cpu"
    torch.manual_seed(st["seed"])
    x = torch.randn(*st["hidden_shape"])
    logits = {}
    with torch.no_grad():
        for r in st["routers"]:
            out_f, in_f = r["shape"]
            lin = torch.nn.Linear(in_f, out_f, bias=False)  # draws its weight from the same generator
            if "boost_row" in r:
                lin.weight[r["boost_row"]] += r["boost"]
            logits[r["name"]] = lin(x).numpy().astype(np.float64)
    counts = np.bincount(logits["balanced"].argmax(axis=1), minlength=st["num_experts"])
    for cap, dropped in zip(g["balanced"]["capacity"], g["balanced"]["dropped"]):
        if int(np.maximum(counts - cap, 0).sum()) != dropped:
            pytest.skip("torch's seeded draw differs from the page's; the demo fixture does not apply")
    return logits
