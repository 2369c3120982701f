"""moe_forward_noalloc (the forward on the library's static per-GPU scratch,
for callers that cannot allocate) against moe_forward with a caller
workspace: bitwise-equal outputs on consecutive calls, each later call
smaller than the one before it (the scratch keeps the earlier call's bytes),
across the decode, tiled and latent paths; layers beyond the scratch size
are refused before any launch."""
from __future__ import annotations

import sys

import pytest
import torch

import sparse_mixture_experts_11_amd as moe
from sparse_mixture_experts_11_amd import _lib as L
from synth import configs as C
from tests import harness as H

pytestmark = pytest.mark.gpu

MIX_S = C.MIXTRAL_PREFILL.with_(name="mixtral_small", d=1024, h=2048)
LAT_S = C.LATENT.with_(name="latent_small", d=512, l=384, h=256, N=96, k=6, h_shared=256)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _run_pair(cfg):
    """The same inputs through moe_forward (fresh workspace) and
    moe_forward_noalloc; every output compared bit for bit."""
    desc = H.desc_for(cfg)
    assert moe.moe_workspace_bytes(desc) <= L.MOE_STATIC_SCRATCH_BYTES
    w = H.upload_layer(cfg)
    u = H.to_device(cfg.u())
    y_ref, out_ref = H.y_buffer(cfg), H.out_buffers(cfg)
    moe.moe_forward(desc, w, u, y_ref, out_ref, moe.workspace(desc))
    y, out = H.y_buffer(cfg), H.out_buffers(cfg)
    y.fill_(float("nan"))
    moe.moe_forward_noalloc(desc, w, u, y, out)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    for key in out:
        assert torch.equal(out[key], out_ref[key]), key


@pytest.mark.parametrize("seq", [
    # decode kernels: T = 64 then T = 20 (and a fresh-process first call)
    (MIX_S.with_(T=64), MIX_S.with_(T=20)),
    # tiled grouped GEMM at 4096 tokens (19 MiB of scratch), then one token
    (C.MCU_BATCH, C.MCU_DECODE),
    # latent layer: router GEMM, projections, shared experts; then smaller
    (LAT_S.with_(T=64), LAT_S.with_(T=7)),
], ids=["decode", "tiled_then_t1", "latent"])
def test_noalloc_matches_forward_twice(seq):
    for cfg in seq:
        log(f"[noalloc] {cfg.name} T={cfg.T} d={cfg.d} N={cfg.N} k={cfg.k} "
            f"scratch {moe.moe_workspace_bytes(H.desc_for(cfg))} B")
        _run_pair(cfg)


def test_noalloc_refuses_layers_beyond_scratch():
    cfg = C.MIXTRAL_PREFILL
    desc = H.desc_for(cfg)
    log(f"[noalloc] refuses {cfg.name}: needs {moe.moe_workspace_bytes(desc)} B")
    assert moe.moe_workspace_bytes(desc) > L.MOE_STATIC_SCRATCH_BYTES
    u = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    y = torch.full((cfg.T, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    w = {name: dummy for name in ("W_route", "W_gate", "W_up", "W_down")}
    with pytest.raises(moe.MoeError) as exc:
        moe.moe_forward_noalloc(desc, w, u, y)
    assert exc.value.status == L.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
