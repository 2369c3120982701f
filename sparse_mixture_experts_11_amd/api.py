"""Python binding of the MoE C ABI: argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors (device memory on the caller's stream) and raises MoeError on a
status other than MOE_OK.  No step of the layer runs in Python: each call
forwards pointers and sizes to libmoe.so and returns.
"""
from __future__ import annotations

import ctypes
from typing import Mapping, Optional

import torch

from . import _lib as L
from ._lib import MoeDesc, MoeOutputs, MoeWeights  # noqa: F401

_DT = {"f32": L.MOE_F32, "bf16": L.MOE_BF16, "fp8": L.MOE_FP8_E4M3, "mxfp4": L.MOE_MXFP4}
_GATE = {"renorm": L.MOE_GATE_RENORM, "prob": L.MOE_GATE_PROB}
_ACT = {"swiglu": L.MOE_ACT_SWIGLU, "situ": L.MOE_ACT_SITU_GLU}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = L.load().moe_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str) -> None:
    if status != L.MOE_OK:
        raise MoeError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def moe_desc_init() -> MoeDesc:
    d = MoeDesc()
    L.load().moe_desc_init(ctypes.byref(d))
    return d


def make_desc(*, T, d, h, N, k, capacity, act_dtype, w_dtype, router_dtype, gate, act, beta_g,
              beta_u, l, n_shared, h_shared, rms_eps, aux_alpha) -> MoeDesc:
    """Descriptor with every field given explicitly (no defaults on purpose)."""
    x = moe_desc_init()
    x.T, x.d, x.h, x.N, x.k = int(T), int(d), int(h), int(N), int(k)
    x.capacity = int(capacity)
    x.act_dtype = _DT.get(act_dtype, act_dtype)
    x.w_dtype = _DT.get(w_dtype, w_dtype)
    x.router_dtype = _DT.get(router_dtype, router_dtype)
    x.gate = _GATE.get(gate, gate)
    x.act = _ACT.get(act, act)
    x.beta_g, x.beta_u = float(beta_g), float(beta_u)
    x.l, x.n_shared, x.h_shared = int(l), int(n_shared), int(h_shared)
    x.rms_eps, x.aux_alpha = float(rms_eps), float(aux_alpha)
    return x


def moe_status_string(status: int) -> str:
    return L.load().moe_status_string(status).decode()


def moe_workspace_bytes(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(L.load().moe_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "moe_workspace_bytes")
    return int(n.value)


def moe_capacity_from_factor(T: int, N: int, k: int, c: float) -> int:
    return int(L.load().moe_capacity_from_factor(T, N, k, c))


def workspace(desc: MoeDesc, device="cuda") -> torch.Tensor:
    return torch.empty(moe_workspace_bytes(desc), dtype=torch.uint8, device=device)


def moe_route(desc, u, W_route, topk_idx, topk_w, stats, ws, stream=None) -> None:
    _check(L.load().moe_route(ctypes.byref(desc), _ptr(u), _ptr(W_route), _ptr(topk_idx),
                              _ptr(topk_w), _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_route")


def moe_route_biased(desc, u, W_route, bias, topk_idx, topk_w, stats, ws, stream=None) -> None:
    """moe_route picking the top-k of z + bias (bias: [N] fp32 device tensor or None)."""
    _check(L.load().moe_route_biased(ctypes.byref(desc), _ptr(u), _ptr(W_route), _ptr(bias),
                                     _ptr(topk_idx), _ptr(topk_w), _ptr(stats), _ptr(ws),
                                     ws.numel(), _stream(stream)), "moe_route_biased")


QB_EXACT, QB_HISTOGRAM = 0, 1


def moe_qb_update(desc, u, W_route, bias, new_bias, ws, q=0, method=QB_EXACT,
                  stream=None) -> None:
    """One Quantile Balancing step: new_bias[j] = q-th smallest (or its
    histogram estimate) of cutoff_t - z_tj; q = 0 selects round(kT/N)."""
    _check(L.load().moe_qb_update(ctypes.byref(desc), _ptr(u), _ptr(W_route), _ptr(bias),
                                  int(q), int(method), _ptr(new_bias), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_qb_update")


def moe_route_backward(desc, u, W_route, topk_idx, row_of, stats, y_perm, dy, dz, dW_route, du,
                       ws, aux_scale=1.0, stream=None) -> None:
    _check(L.load().moe_route_backward(ctypes.byref(desc), _ptr(u), _ptr(W_route),
                                       _ptr(topk_idx), _ptr(row_of), _ptr(stats), _ptr(y_perm),
                                       _ptr(dy), float(aux_scale), _ptr(dz), _ptr(dW_route),
                                       _ptr(du), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_route_backward")


def moe_backward_workspace_bytes(desc) -> int:
    n = ctypes.c_size_t(0)
    _check(L.load().moe_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "moe_backward_workspace_bytes")
    return n.value


def backward_workspace(desc, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_backward_workspace_bytes(desc), 1), dtype=torch.uint8,
                       device=device)


def moe_experts_backward(desc, weights: Mapping[str, torch.Tensor], u, topk_w, offsets,
                         kept_offsets, perm, row_of, dy, dx, ws, dW_gate=None, dW_up=None,
                         dW_down=None, gate_up=None, stream=None) -> None:
    """gate_up: the forward's saved G | U rows (outputs "gate_up"), or None
    to recompute them."""
    w = _weights(weights)
    _check(L.load().moe_experts_backward(ctypes.byref(desc), ctypes.byref(w), _ptr(u),
                                         _ptr(topk_w), _ptr(offsets), _ptr(kept_offsets),
                                         _ptr(perm), _ptr(row_of), _ptr(gate_up), _ptr(dy),
                                         _ptr(dx), _ptr(dW_gate), _ptr(dW_up), _ptr(dW_down),
                                         _ptr(ws), ws.numel(), _stream(stream)),
           "moe_experts_backward")


def moe_latent_backward(desc, weights: Mapping[str, torch.Tensor], u,
                        fwd: Mapping[str, torch.Tensor], dy, grads: Mapping[str, torch.Tensor],
                        ws, aux_scale: float = 0.0, stream=None) -> None:
    """grads: du, dz, dW_route, dW_ldown, dW_lup, dW_gate, dW_up, dW_down and,
    with shared experts, dWs_gate, dWs_up, dWs_down (fp32 tensors)."""
    w = _weights(weights)
    g = L.MoeLatentGrads()
    for name, _ in L.MoeLatentGrads._fields_:
        t = grads.get(name)
        setattr(g, name, None if t is None else _ptr(t).value)
    _check(L.load().moe_latent_backward(ctypes.byref(desc), ctypes.byref(w), _ptr(u),
                                        _outputs(fwd), _ptr(dy), float(aux_scale),
                                        ctypes.byref(g), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_latent_backward")


def moe_dispatch(desc, topk_idx, counts, offsets, kept_offsets, perm, row_of, drop, ws,
                 stream=None) -> None:
    _check(L.load().moe_dispatch(ctypes.byref(desc), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                                 _ptr(kept_offsets), _ptr(perm), _ptr(row_of), _ptr(drop),
                                 _ptr(ws), ws.numel(), _stream(stream)), "moe_dispatch")


def moe_expert_ffn(desc, x, perm, offsets, kept_offsets, W_gate, W_up, W_down, y_perm, ws,
                   stream=None) -> None:
    _check(L.load().moe_expert_ffn(ctypes.byref(desc), _ptr(x), _ptr(perm), _ptr(offsets),
                                   _ptr(kept_offsets), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
                                   _ptr(y_perm), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_ffn")


def moe_expert_ffn_scaled(desc, x, perm, offsets, kept_offsets, W_gate, W_up, W_down,
                          gate_scale, up_scale, down_scale, y_perm, ws, stream=None) -> None:
    _check(L.load().moe_expert_ffn_scaled(ctypes.byref(desc), _ptr(x), _ptr(perm), _ptr(offsets),
                                          _ptr(kept_offsets), _ptr(W_gate), _ptr(W_up),
                                          _ptr(W_down), _ptr(gate_scale), _ptr(up_scale),
                                          _ptr(down_scale), _ptr(y_perm), _ptr(ws), ws.numel(),
                                          _stream(stream)), "moe_expert_ffn_scaled")


def moe_combine(desc, y_perm, row_of, topk_w, y, stream=None) -> None:
    _check(L.load().moe_combine(ctypes.byref(desc), _ptr(y_perm), _ptr(row_of), _ptr(topk_w),
                                _ptr(y), _stream(stream)), "moe_combine")


def _weights(w: Mapping[str, torch.Tensor]) -> MoeWeights:
    s = MoeWeights()
    for name, _ in MoeWeights._fields_:
        t = w.get(name)
        setattr(s, name, None if t is None else _ptr(t).value)
    return s


def _outputs(out: Optional[Mapping[str, torch.Tensor]]):
    if out is None:
        return None
    s = MoeOutputs()
    for name, _ in MoeOutputs._fields_:
        t = out.get(name)
        setattr(s, name, None if t is None else _ptr(t).value)
    return ctypes.byref(s)


def moe_forward(desc, weights: Mapping[str, torch.Tensor], u, y, out=None, ws=None,
                stream=None) -> None:
    w = _weights(weights)
    _check(L.load().moe_forward(ctypes.byref(desc), ctypes.byref(w), _ptr(u), _ptr(y),
                                _outputs(out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_forward")


def moe_forward_noalloc(desc, weights: Mapping[str, torch.Tensor], u, y, out=None,
                        stream=None) -> None:
    w = _weights(weights)
    _check(L.load().moe_forward_noalloc(ctypes.byref(desc), ctypes.byref(w), _ptr(u), _ptr(y),
                                        _outputs(out), _stream(stream)), "moe_forward_noalloc")


def moe_forward_traced(desc, weights, u, y, out, ws, events, stream=None) -> None:
    """events: list of torch.cuda.Event(enable_timing=True); recorded between stages."""
    w = _weights(weights)
    for e in events:
        if not e.cuda_event:   # torch creates its event handle on first record
            e.record()
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(L.load().moe_forward_traced(ctypes.byref(desc), ctypes.byref(w), _ptr(u), _ptr(y),
                                       _outputs(out), _ptr(ws), ws.numel(), _stream(stream),
                                       handles, len(events)), "moe_forward_traced")


def moe_stage_names(desc) -> list:
    n = ctypes.c_int32(0)
    lib = L.load()
    lib.moe_stage_name(ctypes.byref(desc), 1, ctypes.byref(n))
    return [lib.moe_stage_name(ctypes.byref(desc), i, None).decode() for i in range(1, n.value + 1)]
