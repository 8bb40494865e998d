"""moe_forward_noalloc (workspace in the library's fixed per-GPU scratch array) against
moe_forward with a caller workspace, through the C ABI: bitwise equal outputs and routing on
two calls in a row, the second with a smaller layer (the array keeps the first call's
contents), and a clear MOE_ERR_WORKSPACE for a layer that needs more than the array holds."""
import ctypes

import pytest
import torch

from sparse_mixture_experts_level_amd import workloads as wl
from tests.moe_testlib import say

pytestmark = pytest.mark.gpu
ops = pytest.importorskip("sparse_mixture_experts_level_amd.ops")
DEV = "cuda"


def _both(w, seed):
    inp = wl.make_inputs(w, seed=seed, device=DEV)
    cap = ops.moe_capacity(w.num_tokens, w.num_experts, w.capacity_factor)
    layer = ops.MoELayer(inp, cap)
    assert ops.moe_workspace_size(layer.desc) <= ops.MOE_NOALLOC_WORKSPACE_BYTES
    want = layer.forward(with_routing=True).clone()
    want_r = {n: v.clone() for n, v in layer.routing.items()}
    out = torch.full_like(inp.x, 7.0)
    routing = {n: torch.full_like(v, -3) for n, v in layer.routing.items()}
    ops.moe_forward_noalloc(layer.desc, inp.w_router, inp.w_gate_up, inp.w_down, inp.x, inp.logit_offset, out,
                            routing=routing, w_shared_gate_up=inp.w_shared_gate_up,
                            w_shared_down=inp.w_shared_down)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), want.view(torch.uint8))  # bitwise
    R = int(want_r["expert_offsets"][-1])
    for n in want_r:
        if n == "row_token":  # written for the kept rows only
            assert torch.equal(routing[n][:R], want_r[n][:R]), n
        else:
            assert torch.equal(routing[n], want_r[n]), n


def test_noalloc_forward_equals_forward_on_two_calls():
    big = wl.get_workload("switch_bf16")  # 86 MiB of workspace: most of the array
    small = wl.Workload("small", 300, 256, 8, 2, 192, 1.25, "bf16", d_ff_shared=64, offset="boost4")
    say("noalloc forward: Switch-style layer, then a small layer with a shared expert")
    _both(big, 0)
    _both(small, 1)
    say("noalloc forward: the tiny float layer")
    _both(wl.get_workload("tiny_f32"), 2)


def test_noalloc_forward_rejects_a_layer_beyond_the_array():
    w = wl.get_workload("deepseek_v3_bf16")
    cap = ops.moe_capacity(w.num_tokens, w.num_experts, w.capacity_factor)
    desc = ops.make_desc(w.num_tokens, w.d_model, w.d_ff, w.num_experts, w.top_k, cap, w.d_ff_shared, w.torch_dtype)
    assert ops.moe_workspace_size(desc) > ops.MOE_NOALLOC_WORKSPACE_BYTES
    L = ops.lib()
    W = ops.MoeWeights()
    st = L.moe_forward_noalloc(ctypes.byref(desc), ctypes.byref(W), None, None, None, None, None)
    assert st == ops.MOE_ERR_WORKSPACE
    assert b"scratch array" in L.moe_last_error()
