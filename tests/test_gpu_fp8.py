"""FP8 E4M3 routed-expert weights (one fp32 scale per weight row) on the GPU
against the fp64 oracle, which expands each row as scale times the codes'
exact values.  Covers the decode kernels (few rows per expert), the grouped
GEMM at both m-tile heights, capacity drops, the latent layer, and the
full-size Mixtral decode and prefill workloads."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_11_amd as moe
from synth import configs as C
from tests import harness as H
from tests import parity as PR
from tests.test_gpu_parity import (CASES, check_forward, log, oracle_capacity, oracle_forward,
                                   run_forward, sample_tokens)
import synth as S

pytestmark = pytest.mark.gpu

FP8_CASES = {name: CASES[name].with_(name=name + "_fp8", w_dtype="fp8") for name in (
    "mcu_t1",                       # decode kernels, K below one window (tail loop only)
    "mcu_t4096",                    # GEMM with K = 128 in the down projection
    "mixtral_small_t37_decode",     # decode kernels
    "mixtral_small_t64_decode",     # decode kernels, four token groups
    "mixtral_k2176_t30_decode",     # decode: pipelined windows and a remainder
    "mixtral_k2176_t60_decode",
    "mixtral_small_t1000",          # GEMM, 256-row m-tiles
    "mixtral_small_t1200_bm192",    # GEMM, 192-row m-tiles
    "switch_small_t2000",           # top-1 with capacity drops
    "latent_small_t700",            # latent layer: experts at width l, bf16 projections
    "latent_small_decode_t20",      # latent layer through the decode kernels
)}


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_forward_parity(name):
    cfg = FP8_CASES[name]
    log(f"[fp8 forward] {cfg.name} T={cfg.T} d={cfg.d} h={cfg.h} N={cfg.N} k={cfg.k}")
    ref = oracle_forward(cfg)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out)


@pytest.mark.parametrize("name", ["mcu_t1", "mixtral_small_t37_decode", "mixtral_small_t1000",
                                  "switch_small_t2000", "latent_small_t700"])
def test_fp8_stage_expert_ffn(name):
    cfg = FP8_CASES[name]
    log(f"[fp8 expert_ffn] {cfg.name}")
    desc = H.desc_for(cfg)
    ref = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    rd = O.dispatch(ref["idx"], cfg.N, oracle_capacity(cfg))
    if cfg.latent:
        x_st = S.normal_stored(cfg.seed + 100, 99, cfg.T * cfg.l, 1.0, cfg.act_dtype).reshape(
            cfg.T, cfg.l)
    else:
        x_st = cfg.u()
    act = O.make_act(cfg.act, cfg.beta_g, cfg.beta_u)
    rows = O.expert_rows(O.expand(x_st), rd, lambda e: cfg.expert(e), act, cfg.k)
    R = int(rd["kept_offsets"][-1])
    w = H.upload_layer(cfg)
    y_perm = torch.full((max(R, 1), cfg.x_width), float("nan"), device="cuda")
    moe.moe_expert_ffn_scaled(desc, H.to_device(x_st), H.to_device(rd["perm"]),
                              H.to_device(rd["offsets"]), H.to_device(rd["kept_offsets"]),
                              w["W_gate"], w["W_up"], w["W_down"], w["gate_scale"],
                              w["up_scale"], w["down_scale"], y_perm, moe.workspace(desc))
    torch.cuda.synchronize()
    yr = np.stack([rows[r] for r in range(R)])
    err = PR.rel_err(H.to_host(y_perm)[:R].astype(np.float64), yr)
    log(f"  rel err {err:.3e}")
    assert err <= PR.TOL[cfg.act_dtype]


def test_fp8_scales_are_per_row():
    # Every row scale of every matrix times its own random factor in [0.5, 2]:
    # the output must follow the oracle with the same edited scales (a scale
    # applied along the wrong axis or to the wrong matrix fails this).
    cfg = FP8_CASES["mixtral_small_t37_decode"]
    log(f"[fp8 scale edit] {cfg.name}")
    w = H.upload_layer(cfg)
    rng = np.random.default_rng(11)
    f = {m: rng.uniform(0.5, 2.0, size=w[m + "_scale"].shape).astype(np.float32)
         for m in ("gate", "up", "down")}
    for m in f:
        w[m + "_scale"] *= torch.from_numpy(f[m]).cuda()

    def experts(e):
        g, u, dn = cfg.expert(e)
        return tuple(S.Fp8Rows(x.codes, (x.scale * f[m][e]).astype(np.float32))
                     for x, m in ((g, "gate"), (u, "up"), (dn, "down")))
    ref = O.forward(cfg.u(), cfg.w_route(), experts, k=cfg.k, gate=cfg.gate, act=cfg.act,
                    capacity=oracle_capacity(cfg), beta_g=cfg.beta_g, beta_u=cfg.beta_u,
                    alpha=cfg.aux_alpha)
    y, out = run_forward(cfg, weights=w)
    check_forward(cfg, ref, y, out)


@pytest.mark.timeout(600)
def test_fp8_full_size_mixtral_decode():
    cfg = C.MIXTRAL_DECODE_FP8
    log(f"[fp8 full] {cfg.name}")
    ref = oracle_forward(cfg)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out)


@pytest.mark.timeout(600)
def test_fp8_full_size_mixtral_prefill():
    cfg = C.MIXTRAL_PREFILL_FP8
    log(f"[fp8 full] {cfg.name}")
    tokens = sample_tokens(cfg.T, 24, cfg.seed)
    ref = oracle_forward(cfg, tokens=tokens)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out, tokens=tokens)
