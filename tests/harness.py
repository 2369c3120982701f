"""Device-side helpers shared by the GPU tests, the smoke check and the
benchmark: descriptor from a workload recipe, upload of the seeded stored
inputs, and output buffers.  No part of the layer is computed here."""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

import sparse_mixture_experts_11_amd as moe
from synth import configs as C


def capacity_of(cfg: C.Layer) -> int:
    """Integer capacity for the library: converted by the library's own helper."""
    if cfg.capacity_factor is None:
        return -1
    return moe.moe_capacity_from_factor(cfg.T, cfg.N, cfg.k, cfg.capacity_factor)


def desc_for(cfg: C.Layer, capacity: Optional[int] = None):
    return moe.make_desc(
        T=cfg.T, d=cfg.d, h=cfg.h, N=cfg.N, k=cfg.k,
        capacity=capacity_of(cfg) if capacity is None else capacity,
        act_dtype=cfg.act_dtype, w_dtype=cfg.w_dtype, router_dtype=cfg.router_dtype,
        gate=cfg.gate, act=cfg.act, beta_g=cfg.beta_g, beta_u=cfg.beta_u,
        l=cfg.l, n_shared=cfg.n_shared, h_shared=cfg.h_shared, rms_eps=cfg.rms_eps,
        aux_alpha=cfg.aux_alpha)


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Stored numpy array -> device tensor of the same bits (bf16 stays bf16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype in (np.int32, np.int64):
        return torch.from_numpy(a.astype(np.int32)).to(device)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    raise TypeError(a.dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy stored array (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _torch_dtype(stored: str):
    return torch.bfloat16 if stored == "bf16" else torch.float32


def upload_stacked(cfg: C.Layer, which: str, device="cuda", chunk_experts: int = 0) -> torch.Tensor:
    """Stacked routed-expert tensor on the device, generated expert by expert
    through a pinned staging buffer (never the whole tensor on the host)."""
    xw, h, N = cfg.x_width, cfg.h, cfg.N
    shape = (N, h, xw) if which in ("gate", "up") else (N, xw, h)
    per = h * xw
    dev = torch.empty(shape, dtype=_torch_dtype(cfg.w_dtype), device=device)
    npdt = np.uint16 if cfg.w_dtype == "bf16" else np.float32
    step = chunk_experts or max(1, min(N, (256 << 20) // (per * npdt().itemsize)))
    stage = torch.empty(step * per, dtype=torch.int16 if cfg.w_dtype == "bf16" else torch.float32,
                        pin_memory=True)
    stage_np = stage.numpy().view(npdt)
    import synth as S
    tid, std = {"gate": (S.TID_W_GATE, 1 / math.sqrt(xw)), "up": (S.TID_W_UP, 1 / math.sqrt(xw)),
                "down": (S.TID_W_DOWN, 1 / math.sqrt(h))}[which]
    flat = dev.view(-1) if cfg.w_dtype == "f32" else dev.view(torch.int16).view(-1)
    for e0 in range(0, N, step):
        n = min(step, N - e0)
        S.normal_stored(cfg.seed, tid, n * per, std, cfg.w_dtype, start=e0 * per,
                        out=stage_np[:n * per])
        flat[e0 * per:(e0 + n) * per].copy_(stage[:n * per], non_blocking=False)
    return dev


def upload_stacked_fp8(cfg: C.Layer, which: str, device="cuda"):
    """FP8 routed-expert tensor on the device: (E4M3 codes uint8 [N, rows,
    cols], fp32 row scales [N, rows]), generated a few experts at a time."""
    xw, h, N = cfg.x_width, cfg.h, cfg.N
    rows, cols = (h, xw) if which in ("gate", "up") else (xw, h)
    per = rows * cols
    import synth as S
    tid, std = {"gate": (S.TID_W_GATE, 1 / math.sqrt(xw)), "up": (S.TID_W_UP, 1 / math.sqrt(xw)),
                "down": (S.TID_W_DOWN, 1 / math.sqrt(h))}[which]
    codes = torch.empty((N, rows, cols), dtype=torch.uint8, device=device)
    scale = torch.empty((N, rows), dtype=torch.float32, device=device)
    step = max(1, min(N, (256 << 20) // per))
    stage = torch.empty(step * per, dtype=torch.uint8, pin_memory=True)
    for e0 in range(0, N, step):
        n = min(step, N - e0)
        m = S.normal_fp8_rows(cfg.seed, tid, n * rows, cols, std, start=e0 * per,
                              codes=stage.numpy()[:n * per])
        codes.view(-1)[e0 * per:(e0 + n) * per].copy_(stage[:n * per], non_blocking=False)
        scale[e0:e0 + n].copy_(torch.from_numpy(m.scale.reshape(n, rows)))
    return codes, scale


def upload_stacked_mxfp4(cfg: C.Layer, which: str, device="cuda"):
    """MXFP4 routed-expert tensor on the device: (packed E2M1 codes uint8
    [N, rows, cols/2], E8M0 scale bytes [N, rows, cols/32])."""
    xw, h, N = cfg.x_width, cfg.h, cfg.N
    rows, cols = (h, xw) if which in ("gate", "up") else (xw, h)
    import synth as S
    tid, std = {"gate": (S.TID_W_GATE, 1 / math.sqrt(xw)), "up": (S.TID_W_UP, 1 / math.sqrt(xw)),
                "down": (S.TID_W_DOWN, 1 / math.sqrt(h))}[which]
    packed = torch.empty((N, rows, cols // 2), dtype=torch.uint8, device=device)
    scale = torch.empty((N, rows, cols // 32), dtype=torch.uint8, device=device)
    step = max(1, min(N, (256 << 20) // (rows * cols // 2)))
    for e0 in range(0, N, step):
        n = min(step, N - e0)
        m = S.normal_mxfp4_rows(cfg.seed, tid, n * rows, cols, std, start=e0 * rows * cols)
        packed[e0:e0 + n].copy_(torch.from_numpy(m.packed.reshape(n, rows, cols // 2)))
        scale[e0:e0 + n].copy_(torch.from_numpy(m.block_scale.reshape(n, rows, cols // 32)))
    return packed, scale


def upload_layer(cfg: C.Layer, device="cuda") -> Dict[str, torch.Tensor]:
    w = {"W_route": to_device(cfg.w_route(), device)}
    if cfg.w_dtype == "fp8":
        for name in ("gate", "up", "down"):
            w["W_" + name], w[name + "_scale"] = upload_stacked_fp8(cfg, name, device)
    elif cfg.w_dtype == "mxfp4":
        for name in ("gate", "up", "down"):
            w["W_" + name], w[name + "_scale"] = upload_stacked_mxfp4(cfg, name, device)
    else:
        for name in ("gate", "up", "down"):
            w["W_" + name] = upload_stacked(cfg, name, device)
    if cfg.latent:
        w["W_ldown"] = to_device(cfg.w_ldown(), device)
        w["W_lup"] = to_device(cfg.w_lup(), device)
        if cfg.n_shared:
            for name in ("gate", "up", "down"):
                w["Ws_" + name] = to_device(cfg.shared_tensor(name), device)
    return w


def out_buffers(cfg: C.Layer, device="cuda") -> Dict[str, torch.Tensor]:
    E = cfg.T * cfg.k
    i32 = dict(dtype=torch.int32, device=device)
    return {"topk_idx": torch.empty(E, **i32), "topk_w": torch.empty(E, dtype=torch.float32,
                                                                     device=device),
            "stats": torch.empty(2 * cfg.N + 2, dtype=torch.float32, device=device),
            "counts": torch.empty(cfg.N, **i32), "offsets": torch.empty(cfg.N + 1, **i32),
            "kept_offsets": torch.empty(cfg.N + 1, **i32), "perm": torch.empty(E, **i32),
            "row_of": torch.empty(E, **i32), "drop": torch.empty(E, dtype=torch.uint8,
                                                                 device=device)}


def y_buffer(cfg: C.Layer, device="cuda") -> torch.Tensor:
    return torch.empty((cfg.T, cfg.d), dtype=_torch_dtype(cfg.act_dtype), device=device)


def expand_device_output(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a device output (bf16 or fp32)."""
    return t.detach().double().cpu().numpy()
