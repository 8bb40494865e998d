"""Thin Python binding of libmoe.so (C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors living on the GPU (torch provides device
memory and the current HIP stream); their data pointers are handed to the C
entry points of the same names.  The library must be built
(``python -m sparse_mixture_experts_level_amd.build``); a missing library raises
instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "libmoe_debug.so")

MOE_NO_CAPACITY = -1
MOE_MAX_EXPERTS = 1024
MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_FILL_TOKEN_MAJOR, MOE_FILL_RANK_MAJOR = 0, 1
MOE_OVERFLOW_DROP, MOE_OVERFLOW_REROUTE = 0, 1

SYMBOLS = [
    "moe_capacity", "moe_capacity_topk", "moe_max_rows", "moe_workspace_size", "moe_grouped_gemm_workspace_size",
    "moe_status_string", "moe_last_error", "moe_router_logits", "moe_router_topk",
    "moe_dispatch_permute", "moe_dispatch_reroute", "moe_grouped_swiglu_gemm", "moe_grouped_gate_up_swiglu", "moe_grouped_down",
    "moe_combine_unpermute", "moe_router_aux_loss", "moe_forward", "moe_forward_expert_shard",
    "moe_backward_workspace_size", "moe_backward", "moe_tiled_weights_bytes", "moe_tile_expert_weights",
    "moe_check_topk_ids", "moe_debug_checks", "moe_forward_staged", "moe_forward_noalloc",
]
MOE_NOALLOC_WORKSPACE_BYTES = 128 << 20

# moe_stage: the stages moe_forward_staged marks, in launch order
STAGES = ["router", "dispatch", "pack_rows", "gate_up", "gate_up_tails", "down", "down_tails", "shared_pack_rows",
          "shared_gate_up", "shared_gate_up_tails", "shared_down", "shared_down_tails", "combine"]


class MoEError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} failed: {detail} (status {status})")
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("dtype", ctypes.c_int32), ("fill_order", ctypes.c_int32),
                ("overflow", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("w_shared_gate_up", ctypes.c_void_p), ("w_shared_down", ctypes.c_void_p),
                ("w_gate_up_tiled", ctypes.c_void_p), ("w_down_tiled", ctypes.c_void_p),
                ("w_shared_gate_up_tiled", ctypes.c_void_p), ("w_shared_down_tiled", ctypes.c_void_p)]


class MoeGrads(ctypes.Structure):
    _fields_ = [("dw_router", ctypes.c_void_p), ("dw_gate_up", ctypes.c_void_p), ("dw_down", ctypes.c_void_p),
                ("dw_shared_gate_up", ctypes.c_void_p), ("dw_shared_down", ctypes.c_void_p)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_gates", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("row_token", ctypes.c_void_p), ("assigned_ids", ctypes.c_void_p)]


_lib = None
_debug_lib = None


def lib() -> ctypes.CDLL:
    """Loads libmoe.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib() -> ctypes.CDLL:
    """Loads libmoe_debug.so (the same kernels; host checks of device-side preconditions)."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_mixture_experts_level_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(MoeDesc)
    L.moe_capacity.argtypes, L.moe_capacity.restype = [i32, i32, ctypes.c_double], i32
    L.moe_capacity_topk.argtypes, L.moe_capacity_topk.restype = [i32, i32, i32, ctypes.c_double], i32
    L.moe_max_rows.argtypes, L.moe_max_rows.restype = [dp], i64
    L.moe_workspace_size.argtypes, L.moe_workspace_size.restype = [dp], sz
    L.moe_grouped_gemm_workspace_size.argtypes, L.moe_grouped_gemm_workspace_size.restype = [i32, i64, i32, i32], sz
    L.moe_status_string.argtypes, L.moe_status_string.restype = [st], ctypes.c_char_p
    L.moe_last_error.argtypes, L.moe_last_error.restype = [], ctypes.c_char_p
    L.moe_router_logits.argtypes, L.moe_router_logits.restype = [dp, vp, vp, vp, vp, vp], st
    L.moe_router_topk.argtypes, L.moe_router_topk.restype = [dp, vp, vp, vp, vp], st
    L.moe_dispatch_permute.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch_permute.restype = st
    L.moe_dispatch_reroute.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch_reroute.restype = st
    L.moe_grouped_swiglu_gemm.argtypes = [i32, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_swiglu_gemm.restype = st
    L.moe_grouped_gate_up_swiglu.argtypes = [i32, i64, i32, i32, i32, i32, vp, vp, i64, vp, vp, vp, vp]
    L.moe_grouped_gate_up_swiglu.restype = st
    L.moe_grouped_down.argtypes = [i32, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.moe_grouped_down.restype = st
    L.moe_combine_unpermute.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_combine_unpermute.restype = st
    L.moe_router_aux_loss.argtypes = [dp, vp, vp, ctypes.c_float, vp, vp, sz, vp]
    L.moe_router_aux_loss.restype = st
    L.moe_forward.argtypes = [dp, ctypes.POINTER(MoeWeights), vp, vp, vp, ctypes.POINTER(MoeRouting), vp, sz, vp]
    L.moe_forward.restype = st
    L.moe_forward_staged.argtypes = [dp, ctypes.POINTER(MoeWeights), vp, vp, vp, ctypes.POINTER(MoeRouting), vp, sz,
                                     vp, ctypes.POINTER(vp)]
    L.moe_forward_staged.restype = st
    L.moe_forward_noalloc.argtypes = [dp, ctypes.POINTER(MoeWeights), vp, vp, vp, ctypes.POINTER(MoeRouting), vp]
    L.moe_forward_noalloc.restype = st
    L.moe_forward_expert_shard.argtypes = [dp, ctypes.POINTER(MoeWeights), i32, i32, i32, vp, vp, vp,
                                           ctypes.POINTER(MoeRouting), vp, sz, vp]
    L.moe_forward_expert_shard.restype = st
    L.moe_backward_workspace_size.argtypes, L.moe_backward_workspace_size.restype = [dp], sz
    L.moe_backward.argtypes = [dp, ctypes.POINTER(MoeWeights), vp, ctypes.POINTER(MoeRouting), vp, vp,
                               ctypes.POINTER(MoeGrads), vp, sz, vp]
    L.moe_backward.restype = st
    L.moe_tiled_weights_bytes.argtypes, L.moe_tiled_weights_bytes.restype = [dp, i32, i32], sz
    L.moe_tile_expert_weights.argtypes = [dp, i32, vp, vp, vp, vp, vp]
    L.moe_tile_expert_weights.restype = st
    L.moe_check_topk_ids.argtypes, L.moe_check_topk_ids.restype = [dp, vp], st
    L.moe_debug_checks.argtypes, L.moe_debug_checks.restype = [], i32
    return L


def _check(status: int, func: str, L=None) -> None:
    if status != MOE_OK:
        L = L or lib()
        raise MoEError(status, func, L.moe_last_error().decode() or L.moe_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_DTYPE_F32
    if dt == torch.bfloat16:
        return MOE_DTYPE_BF16
    raise ValueError(f"unsupported dtype {dt}")


_FILL = {"token": MOE_FILL_TOKEN_MAJOR, "rank": MOE_FILL_RANK_MAJOR, "slot": MOE_FILL_RANK_MAJOR}
_OVERFLOW = {"drop": MOE_OVERFLOW_DROP, "reroute": MOE_OVERFLOW_REROUTE}


def make_desc(num_tokens, d_model, d_ff, num_experts, top_k, capacity, d_ff_shared=0, dtype=torch.bfloat16,
              fill_order="token", overflow="drop") -> MoeDesc:
    fo = _FILL[fill_order] if isinstance(fill_order, str) else int(fill_order)
    ov = _OVERFLOW[overflow] if isinstance(overflow, str) else int(overflow)
    return MoeDesc(int(num_tokens), int(d_model), int(d_ff), int(num_experts), int(top_k),
                   MOE_NO_CAPACITY if capacity is None else int(capacity), int(d_ff_shared),
                   dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype), fo, ov)


# ------------------------------------------------------------------------ host helpers

def moe_capacity(num_tokens: int, num_experts: int, capacity_factor: Optional[float]) -> Optional[int]:
    c = lib().moe_capacity(int(num_tokens), int(num_experts), 0.0 if capacity_factor is None else float(capacity_factor))
    return None if c == MOE_NO_CAPACITY else int(c)


def moe_capacity_topk(num_tokens: int, num_experts: int, top_k: int,
                      capacity_factor: Optional[float]) -> Optional[int]:
    c = lib().moe_capacity_topk(int(num_tokens), int(num_experts), int(top_k),
                                0.0 if capacity_factor is None else float(capacity_factor))
    return None if c == MOE_NO_CAPACITY else int(c)


def moe_max_rows(desc: MoeDesc) -> int:
    return int(lib().moe_max_rows(ctypes.byref(desc)))


def moe_workspace_size(desc: MoeDesc) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(desc)))


def moe_grouped_gemm_workspace_size(num_groups: int, rows_max: int, d_ff: int, dtype) -> int:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().moe_grouped_gemm_workspace_size(int(num_groups), int(rows_max), int(d_ff), code))


def moe_check_topk_ids(desc: MoeDesc, topk_ids_host, L=None) -> None:
    """Host check of the ids precondition on a host int32 [T, k] array (numpy or CPU tensor)."""
    import numpy as np

    a = np.ascontiguousarray(topk_ids_host.numpy() if isinstance(topk_ids_host, torch.Tensor) else topk_ids_host,
                             dtype=np.int32)
    L = L or lib()
    _check(L.moe_check_topk_ids(ctypes.byref(desc), a.ctypes.data_as(ctypes.c_void_p)), "moe_check_topk_ids", L)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------ hot path

def moe_router_logits(desc, x, w_router, logit_offset, logits, stream=None) -> None:
    _check(lib().moe_router_logits(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(logit_offset), _ptr(logits),
                                   _stream(stream)), "moe_router_logits")


def moe_router_topk(desc, logits, topk_ids, topk_gates, stream=None) -> None:
    _check(lib().moe_router_topk(ctypes.byref(desc), _ptr(logits), _ptr(topk_ids), _ptr(topk_gates),
                                 _stream(stream)), "moe_router_topk")


def moe_dispatch_permute(desc, topk_ids, x, expert_counts, expert_offsets, slot, row_token, x_perm, ws,
                         stream=None, L=None) -> None:
    L = L or lib()
    _check(L.moe_dispatch_permute(ctypes.byref(desc), _ptr(topk_ids), _ptr(x), _ptr(expert_counts),
                                      _ptr(expert_offsets), _ptr(slot), _ptr(row_token), _ptr(x_perm), _ptr(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "moe_dispatch_permute", L)


def moe_dispatch_reroute(desc, logits, topk_ids, expert_counts, expert_offsets, slot, assigned_ids, row_token, ws,
                         stream=None) -> None:
    _check(lib().moe_dispatch_reroute(ctypes.byref(desc), _ptr(logits), _ptr(topk_ids), _ptr(expert_counts),
                                      _ptr(expert_offsets), _ptr(slot), _ptr(assigned_ids), _ptr(row_token),
                                      _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                      _stream(stream)),
           "moe_dispatch_reroute")


def moe_grouped_swiglu_gemm(num_groups, rows_max, group_rows_max, d_model, d_ff, dtype, x_rows, group_offsets,
                            w_gate_up, w_down, y_rows, ws, stream=None) -> None:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    _check(lib().moe_grouped_swiglu_gemm(int(num_groups), int(rows_max), int(group_rows_max), int(d_model), int(d_ff),
                                         code, _ptr(x_rows), _ptr(group_offsets), _ptr(w_gate_up), _ptr(w_down),
                                         _ptr(y_rows), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                         _stream(stream)), "moe_grouped_swiglu_gemm")


def moe_grouped_gate_up_swiglu(num_groups, rows_max, group_rows_max, d_model, d_ff, dtype, x_rows, group_offsets,
                               w_gate_up, h_rows, row_index=None, stream=None) -> None:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    n_x = 0 if row_index is None else x_rows.shape[0]
    _check(lib().moe_grouped_gate_up_swiglu(int(num_groups), int(rows_max), int(group_rows_max), int(d_model),
                                            int(d_ff), code, _ptr(x_rows), _ptr(row_index), int(n_x),
                                            _ptr(group_offsets), _ptr(w_gate_up), _ptr(h_rows), _stream(stream)),
           "moe_grouped_gate_up_swiglu")


def moe_grouped_down(num_groups, rows_max, group_rows_max, d_model, d_ff, dtype, h_rows, group_offsets, w_down,
                     y_rows, stream=None) -> None:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    _check(lib().moe_grouped_down(int(num_groups), int(rows_max), int(group_rows_max), int(d_model), int(d_ff), code,
                                  _ptr(h_rows), _ptr(group_offsets), _ptr(w_down), _ptr(y_rows), _stream(stream)),
           "moe_grouped_down")


def moe_combine_unpermute(desc, y_perm, topk_ids, topk_gates, slot, expert_offsets, shared_out, out,
                          stream=None, L=None) -> None:
    L = L or lib()
    _check(L.moe_combine_unpermute(ctypes.byref(desc), _ptr(y_perm), _ptr(topk_ids), _ptr(topk_gates), _ptr(slot),
                                   _ptr(expert_offsets), _ptr(shared_out), _ptr(out), _stream(stream)),
           "moe_combine_unpermute", L)


def moe_router_aux_loss(desc, logits, expert_counts, alpha, loss, ws, stream=None) -> None:
    _check(lib().moe_router_aux_loss(ctypes.byref(desc), _ptr(logits), _ptr(expert_counts), float(alpha), _ptr(loss),
                                     _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "moe_router_aux_loss")


def moe_tiled_weights_bytes(desc, num_experts: int, which: int) -> int:
    return int(lib().moe_tiled_weights_bytes(ctypes.byref(desc), int(num_experts), int(which)))


def moe_tile_expert_weights(desc, num_experts, w_gate_up, w_down, w_gate_up_tiled, w_down_tiled,
                            stream=None) -> None:
    _check(lib().moe_tile_expert_weights(ctypes.byref(desc), int(num_experts), _ptr(w_gate_up), _ptr(w_down),
                                         _ptr(w_gate_up_tiled), _ptr(w_down_tiled), _stream(stream)),
           "moe_tile_expert_weights")


def tiled_weights(desc, w_gate_up, w_down, stream=None):
    """The tile-major copies of w_gate_up [n, 2f, d] and w_down [n, d, f] (bf16, n experts),
    allocated here as uint8 tensors and written by moe_tile_expert_weights."""
    n = w_gate_up.shape[0]
    gu = torch.empty(moe_tiled_weights_bytes(desc, n, 0), dtype=torch.uint8, device=w_gate_up.device)
    dn = torch.empty(moe_tiled_weights_bytes(desc, n, 1), dtype=torch.uint8, device=w_down.device)
    moe_tile_expert_weights(desc, n, w_gate_up, w_down, gu, dn, stream=stream)
    return gu, dn


def tiled_shared_weights(desc, w_shared_gate_up, w_shared_down, stream=None):
    """The tile-major copies of the shared expert's [2 f_s, d] and [d, f_s] weights: one expert
    of width d_ff_shared."""
    one = MoeDesc(**{n: getattr(desc, n) for n, _ in MoeDesc._fields_})
    one.num_experts, one.top_k, one.d_ff, one.d_ff_shared, one.capacity = 1, 1, desc.d_ff_shared, 0, MOE_NO_CAPACITY
    return tiled_weights(one, w_shared_gate_up.unsqueeze(0), w_shared_down.unsqueeze(0), stream=stream)


def _weights(w_router, w_gate_up, w_down, w_shared_gate_up, w_shared_down, tiled, shared_tiled=None):
    gu_t, dn_t = tiled if tiled is not None else (None, None)
    sgu_t, sdn_t = shared_tiled if shared_tiled is not None else (None, None)
    return MoeWeights(_ptr(w_router), _ptr(w_gate_up), _ptr(w_down), _ptr(w_shared_gate_up), _ptr(w_shared_down),
                      _ptr(gu_t), _ptr(dn_t), _ptr(sgu_t), _ptr(sdn_t))


def moe_forward(desc, w_router, w_gate_up, w_down, x, logit_offset, out, ws, routing: Optional[dict] = None,
                w_shared_gate_up=None, w_shared_down=None, stream=None, tiled=None, shared_tiled=None) -> None:
    """tiled / shared_tiled: optional tile-major copies from tiled_weights() / tiled_shared_weights()."""
    W = _weights(w_router, w_gate_up, w_down, w_shared_gate_up, w_shared_down, tiled, shared_tiled)
    R = None
    if routing is not None:
        R = MoeRouting(*(_ptr(routing.get(n)) for n, _ in MoeRouting._fields_))
    _check(lib().moe_forward(ctypes.byref(desc), ctypes.byref(W), _ptr(x), _ptr(logit_offset), _ptr(out),
                             ctypes.byref(R) if R is not None else None, _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


def moe_forward_noalloc(desc, w_router, w_gate_up, w_down, x, logit_offset, out, routing: Optional[dict] = None,
                        w_shared_gate_up=None, w_shared_down=None, stream=None, tiled=None,
                        shared_tiled=None) -> None:
    """moe_forward with the library's fixed per-GPU scratch array as its workspace."""
    W = _weights(w_router, w_gate_up, w_down, w_shared_gate_up, w_shared_down, tiled, shared_tiled)
    R = None
    if routing is not None:
        R = MoeRouting(*(_ptr(routing.get(n)) for n, _ in MoeRouting._fields_))
    _check(lib().moe_forward_noalloc(ctypes.byref(desc), ctypes.byref(W), _ptr(x), _ptr(logit_offset), _ptr(out),
                                     ctypes.byref(R) if R is not None else None, _stream(stream)),
           "moe_forward_noalloc")


def stage_events():
    """MOE_NUM_STAGES + 1 timing events for moe_forward_staged (torch events, created by
    recording them once on the current stream)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
    for e in evs:
        e.record()
    return evs


def moe_forward_staged(desc, w_router, w_gate_up, w_down, x, logit_offset, out, ws, events,
                       routing: Optional[dict] = None, w_shared_gate_up=None, w_shared_down=None, stream=None,
                       tiled=None, shared_tiled=None) -> None:
    """moe_forward with events[s + 1] recorded after stage s (events from stage_events())."""
    W = _weights(w_router, w_gate_up, w_down, w_shared_gate_up, w_shared_down, tiled, shared_tiled)
    R = None
    if routing is not None:
        R = MoeRouting(*(_ptr(routing.get(n)) for n, _ in MoeRouting._fields_))
    if len(events) != len(STAGES) + 1:
        raise ValueError(f"moe_forward_staged needs {len(STAGES) + 1} events")
    evs = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(lib().moe_forward_staged(ctypes.byref(desc), ctypes.byref(W), _ptr(x), _ptr(logit_offset), _ptr(out),
                                    ctypes.byref(R) if R is not None else None, _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(), _stream(stream), evs),
           "moe_forward_staged")


def moe_forward_expert_shard(desc, w_router, w_gate_up_local, w_down_local, expert_begin, expert_end, add_shared, x,
                             logit_offset, out_partial, ws, routing: Optional[dict] = None, w_shared_gate_up=None,
                             w_shared_down=None, stream=None, tiled=None, shared_tiled=None) -> None:
    W = _weights(w_router, w_gate_up_local, w_down_local, w_shared_gate_up, w_shared_down, tiled, shared_tiled)
    R = None
    if routing is not None:
        R = MoeRouting(*(_ptr(routing.get(n)) for n, _ in MoeRouting._fields_))
    _check(lib().moe_forward_expert_shard(ctypes.byref(desc), ctypes.byref(W), int(expert_begin), int(expert_end),
                                          int(bool(add_shared)), _ptr(x), _ptr(logit_offset), _ptr(out_partial),
                                          ctypes.byref(R) if R is not None else None, _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward_expert_shard")


def moe_backward_workspace_size(desc: MoeDesc) -> int:
    return int(lib().moe_backward_workspace_size(ctypes.byref(desc)))


def moe_backward(desc, w_router, w_gate_up, w_down, x, routing: dict, dy, dx, grads: dict, ws,
                 w_shared_gate_up=None, w_shared_down=None, stream=None, tiled=None, shared_tiled=None) -> None:
    W = _weights(w_router, w_gate_up, w_down, w_shared_gate_up, w_shared_down, tiled, shared_tiled)
    R = MoeRouting(*(_ptr(routing.get(n)) for n, _ in MoeRouting._fields_))
    G = MoeGrads(*(_ptr(grads.get(n)) for n, _ in MoeGrads._fields_))
    _check(lib().moe_backward(ctypes.byref(desc), ctypes.byref(W), _ptr(x), ctypes.byref(R), _ptr(dy), _ptr(dx),
                              ctypes.byref(G), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)),
           "moe_backward")


class MoELayer:
    """Holds one layer's device tensors and a workspace, and runs moe_forward.

    Convenience only: allocation happens here, once, never inside a forward call."""

    def __init__(self, inputs, capacity, device="cuda", fill_order="token", overflow="drop", tiled=False,
                 shared_tiled=False):
        w = inputs.workload
        self.inputs = inputs
        self.desc = make_desc(w.num_tokens, w.d_model, w.d_ff, w.num_experts, w.top_k, capacity,
                              w.d_ff_shared, w.torch_dtype, fill_order=fill_order, overflow=overflow)
        self.ws = workspace(moe_workspace_size(self.desc), device)
        self.out = torch.empty_like(inputs.x)
        T, E, k = w.num_tokens, w.num_experts, w.top_k
        R = moe_max_rows(self.desc)
        i32 = dict(dtype=torch.int32, device=device)
        self.routing = {
            "logits": torch.empty((T, E), dtype=torch.float32, device=device),
            "topk_ids": torch.empty((T, k), **i32),
            "topk_gates": torch.empty((T, k), dtype=torch.float32, device=device),
            "expert_counts": torch.empty((E,), **i32),
            "expert_offsets": torch.empty((E + 1,), **i32),
            "slot": torch.empty((T, k), **i32),
            "row_token": torch.empty((max(R, 1),), **i32),
            "assigned_ids": torch.empty((T, k), **i32),
        }
        # the routed weights' tile-major copies, prepared once (bf16)
        self.tiled = tiled_weights(self.desc, inputs.w_gate_up, inputs.w_down) if tiled else None
        self.shared_tiled = (tiled_shared_weights(self.desc, inputs.w_shared_gate_up, inputs.w_shared_down)
                             if shared_tiled and w.d_ff_shared else None)

    def forward_staged(self, events, with_routing=False, stream=None):
        i = self.inputs
        moe_forward_staged(self.desc, i.w_router, i.w_gate_up, i.w_down, i.x, i.logit_offset, self.out, self.ws,
                           events, routing=self.routing if with_routing else None,
                           w_shared_gate_up=i.w_shared_gate_up, w_shared_down=i.w_shared_down, stream=stream,
                           tiled=self.tiled, shared_tiled=self.shared_tiled)
        return self.out

    def forward(self, with_routing=True, stream=None):
        i = self.inputs
        moe_forward(self.desc, i.w_router, i.w_gate_up, i.w_down, i.x, i.logit_offset, self.out, self.ws,
                    routing=self.routing if with_routing else None, w_shared_gate_up=i.w_shared_gate_up,
                    w_shared_down=i.w_shared_down, stream=stream, tiled=self.tiled, shared_tiled=self.shared_tiled)
        return self.out
