"""moe_forward captured in a HIP graph (the library allocates nothing,
writes no memset nodes and never synchronises the host, so one forward is
capturable as a whole) and replayed: every replay, with eager work and
host synchronisations between replays, must give exactly the eager
forward's outputs.  Decode-sized layers (launch-bound) and a tiled one."""
from __future__ import annotations

import pytest
import torch

import sparse_mixture_experts_11_amd as moe
from tests import harness as H
from tests.test_gpu_parity import CASES, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["mcu_t1", "mixtral_small_t37_decode", "mixtral_small_t1000",
                                  "latent_small_t700"])
def test_forward_graph_replay_matches_eager(name):
    cfg = CASES[name]
    log(f"[graph] {name}")
    desc = H.desc_for(cfg)
    w = H.upload_layer(cfg)
    u = H.to_device(cfg.u())
    ws = moe.workspace(desc)
    y_eager = H.y_buffer(cfg)
    out_eager = H.out_buffers(cfg)
    moe.moe_forward(desc, w, u, y_eager, out_eager, ws)
    torch.cuda.synchronize()
    y = H.y_buffer(cfg)
    out = H.out_buffers(cfg)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        moe.moe_forward(desc, w, u, y, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(desc, w, u, y, out, ws)
    for rep in range(4):
        y.fill_(0)
        for t in out.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), rep
        for key in out:
            assert torch.equal(out[key], out_eager[key]), (rep, key)
        # eager work between replays
        moe.moe_forward(desc, w, u, y_eager, out_eager, ws)
        torch.cuda.synchronize()
