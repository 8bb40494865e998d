"""Pins of the oracle's backward pass (``moe_backward``) against an independent
automatic differentiation (torch, float64, CPU) of a forward written here with
torch operations, against central finite differences of the oracle's own forward,
and against closed forms and special cases.  CPU only.
"""
import math

import numpy as np
import pytest

import oracle


def _case(rng, T, d, E, k, f, shared=0, offset=False):
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((E, d)) / math.sqrt(d)
    gu = rng.standard_normal((E, 2 * f, d)) / math.sqrt(d)
    dn = rng.standard_normal((E, d, f)) / math.sqrt(f)
    off = rng.standard_normal(E) if offset else None
    sgu = rng.standard_normal((2 * shared, d)) / math.sqrt(d) if shared else None
    sd = rng.standard_normal((d, shared)) / math.sqrt(shared) if shared else None
    dy = rng.standard_normal((T, d))
    return x, w_r, gu, dn, off, sgu, sd, dy


def _torch_grads(x, w_r, gu, dn, k, off, sgu, sd, dy, ids, slot, serving):
    """The layer's forward written with torch ops (routing tables given), differentiated
    by torch.autograd in float64."""
    torch = pytest.importorskip("torch")
    X = torch.tensor(x, requires_grad=True)
    Wr = torch.tensor(w_r, requires_grad=True)
    Wgu = torch.tensor(gu, requires_grad=True)
    Wd = torch.tensor(dn, requires_grad=True)
    logits = X @ Wr.T
    if off is not None:
        logits = logits + torch.tensor(off)
    sel = torch.gather(logits, 1, torch.tensor(ids, dtype=torch.int64))
    g = torch.softmax(sel, dim=1)
    f = dn.shape[2]
    rows = []
    for t in range(x.shape[0]):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(k):
            if slot[t, j] >= 0:
                e = int(serving[t, j])
                h = torch.nn.functional.silu(Wgu[e, :f] @ X[t]) * (Wgu[e, f:] @ X[t])
                acc = acc + g[t, j] * (Wd[e] @ h)
        rows.append(acc)
    out = torch.stack(rows)
    params = [X, Wr, Wgu, Wd]
    if sgu is not None:
        Sgu = torch.tensor(sgu, requires_grad=True)
        Sd = torch.tensor(sd, requires_grad=True)
        fs = sd.shape[1]
        hs = torch.nn.functional.silu(X @ Sgu[:fs].T) * (X @ Sgu[fs:].T)
        out = out + hs @ Sd.T
        params += [Sgu, Sd]
    (out * torch.tensor(dy)).sum().backward()
    return [p.grad.numpy() for p in params]


@pytest.mark.parametrize("T,d,E,k,f,cap,shared,offset,overflow", [
    (12, 8, 4, 2, 6, 4, 0, False, "drop"),
    (16, 6, 5, 3, 4, 5, 3, True, "drop"),
    (10, 5, 3, 1, 3, 3, 0, True, "drop"),
    (20, 7, 6, 2, 5, 4, 0, True, "reroute"),
    (9, 4, 4, 4, 2, None, 2, False, "drop"),
])
def test_backward_matches_torch_autograd(T, d, E, k, f, cap, shared, offset, overflow):
    rng = np.random.default_rng(T * 31 + E)
    x, w_r, gu, dn, off, sgu, sd, dy = _case(rng, T, d, E, k, f, shared, offset)
    b = oracle.moe_backward(x, w_r, gu, dn, k, cap, dy, off, w_shared_gate_up=sgu, w_shared_down=sd,
                            overflow=overflow)
    fwd = oracle.moe_forward(x, w_r, gu, dn, k, cap, off, overflow=overflow)
    serving = fwd["assigned"] if overflow == "reroute" else fwd["ids"]
    want = _torch_grads(x, w_r, gu, dn, k, off, sgu, sd, dy, fwd["ids"], fwd["slot"], serving)
    got = [b["dx"], b["dw_router"], b["dw_gate_up"], b["dw_down"]]
    if shared:
        got += [b["dw_shared_gate_up"], b["dw_shared_down"]]
    for name, g, w in zip(["dx", "dw_router", "dw_gate_up", "dw_down", "dw_sgu", "dw_sd"], got, want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_matches_finite_differences():
    """<grad, v> against (L(theta + eps v) - L(theta - eps v)) / (2 eps), L = sum(dy * out),
    for random directions v in x and in every weight; the routing must not change."""
    rng = np.random.default_rng(5)
    T, d, E, k, f = 6, 4, 3, 2, 3
    x, w_r, gu, dn, off, sgu, sd, dy = _case(rng, T, d, E, k, f, shared=2, offset=True)
    cap = 3
    b = oracle.moe_backward(x, w_r, gu, dn, k, cap, dy, off, w_shared_gate_up=sgu, w_shared_down=sd)
    base = oracle.moe_forward(x, w_r, gu, dn, k, cap, off, w_shared_gate_up=sgu, w_shared_down=sd)

    def loss(**kw):
        args = dict(x=x, w_router=w_r, w_gate_up=gu, w_down=dn, w_shared_gate_up=sgu, w_shared_down=sd)
        args.update(kw)
        r = oracle.moe_forward(args["x"], args["w_router"], args["w_gate_up"], args["w_down"], k, cap, off,
                               w_shared_gate_up=args["w_shared_gate_up"], w_shared_down=args["w_shared_down"])
        assert np.array_equal(r["ids"], base["ids"]) and np.array_equal(r["slot"], base["slot"])
        return float(np.sum(dy * r["out"]))

    eps = 1e-6
    for name, val, grad in [("x", x, b["dx"]), ("w_router", w_r, b["dw_router"]), ("w_gate_up", gu, b["dw_gate_up"]),
                            ("w_down", dn, b["dw_down"]), ("w_shared_gate_up", sgu, b["dw_shared_gate_up"]),
                            ("w_shared_down", sd, b["dw_shared_down"])]:
        for _ in range(3):
            v = rng.standard_normal(val.shape)
            fd = (loss(**{name: val + eps * v}) - loss(**{name: val - eps * v})) / (2 * eps)
            assert abs(fd - float(np.sum(grad * v))) <= 1e-6 * max(1.0, abs(fd)), name


def test_silu_grad_closed_forms():
    assert oracle.silu_grad(0.0) == 0.5
    s = 0.75  # sigmoid(ln 3)
    assert abs(oracle.silu_grad(math.log(3.0)) - s * (1 + math.log(3.0) * (1 - s))) < 1e-15
    z = np.linspace(-6, 6, 101)
    h = 1e-6
    fd = (oracle.silu(z + h) - oracle.silu(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.silu_grad(z), fd, atol=1e-8)


def test_top1_router_gets_no_gradient():
    """With k = 1 the renormalised gate is identically 1: the router weights and the
    logits receive exactly zero gradient."""
    rng = np.random.default_rng(8)
    x, w_r, gu, dn, off, _, _, dy = _case(rng, 20, 6, 4, 1, 5, offset=True)
    b = oracle.moe_backward(x, w_r, gu, dn, 1, 6, dy, off)
    assert np.all(b["dlogits"] == 0.0) and np.all(b["dw_router"] == 0.0)


def test_dropped_and_idle_experts_get_nothing():
    rng = np.random.default_rng(9)
    T, d, E, k, f = 14, 5, 4, 2, 3
    x, w_r, gu, dn, _, _, _, dy = _case(rng, T, d, E, k, f)
    off = np.array([9.0, 9.0, -50.0, -50.0])     # experts 2 and 3 never chosen
    b = oracle.moe_backward(x, w_r, gu, dn, k, 3, dy, off)
    assert np.all(b["dw_gate_up"][2:] == 0.0) and np.all(b["dw_down"][2:] == 0.0)
    z = oracle.moe_backward(x, w_r, gu, dn, k, 0, dy, off)       # capacity 0: everything dropped
    assert np.all(z["dx"] == 0.0) and np.all(z["dw_gate_up"] == 0.0) and np.all(z["dw_down"] == 0.0)
    assert np.all(z["dw_router"] == 0.0)


def test_gate_gradient_sums_to_zero_over_the_selected_logits():
    """Softmax over the selected logits is shift invariant: the logit gradient of each token
    sums to zero, and vanishes outside the selected experts."""
    rng = np.random.default_rng(10)
    x, w_r, gu, dn, off, _, _, dy = _case(rng, 25, 6, 6, 3, 4, offset=True)
    b = oracle.moe_backward(x, w_r, gu, dn, 3, None, dy, off)
    np.testing.assert_allclose(b["dlogits"].sum(axis=1), 0.0, atol=1e-12)
    mask = np.zeros_like(b["dlogits"], dtype=bool)
    np.put_along_axis(mask, b["ids"].astype(np.int64), True, axis=1)
    assert np.all(b["dlogits"][~mask] == 0.0)
