"""MXFP4 routed-expert weights (OCP MX FP4: E2M1 codes two a byte, one E8M0
scale per 32 elements of a row) on the GPU against the fp64 oracle, which
expands every block as its scale times the codes' exact values.  Decode
kernels (up to 64 tokens): windows that fall in the tail loop only, the main
loop on both projections, four token groups, the latent layer.  Tiled GEMM
(more tokens): both m-tile heights, capacity drops, contraction widths that
are not a multiple of 256, wider than one 4096-k scale chunk (a full and a
short second chunk; a second chunk of two k-steps), the latent layer.
Edited block scales on both paths, and the full-size Mixtral decode and
prefill and LatentMoE workloads."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_11_amd as moe
from synth import configs as C
from tests import harness as H
from tests import parity as PR
from tests.test_gpu_parity import CASES, MIX_S, check_forward, log, oracle_capacity, oracle_forward, run_forward
import synth as S

pytestmark = pytest.mark.gpu

MX_CASES = {name: cfg.with_(name=name + "_mxfp4", w_dtype="mxfp4") for name, cfg in (
    ("mcu_t1", CASES["mcu_t1"]),                                    # K = 512 / 128: tail loop only
    ("mixtral_small_t37_decode", CASES["mixtral_small_t37_decode"]),  # down K = 2048: one window
    ("mixtral_small_t64_decode", CASES["mixtral_small_t64_decode"]),  # four token groups
    ("mix_d2048_t40", MIX_S.with_(T=40, d=2048, h=2048)),           # main loop on both
    # gate/up K = 1152 (not a multiple of 512): the per-k-step loop for all
    # of K; down K = 2560: one 512-k window a wave and a 128-k remainder
    ("mix_d1152_t24_decode", MIX_S.with_(T=24, d=1152, h=2560)),
    ("switch_small_t48_decode", CASES["switch_small_t48_decode"]),  # top-1 with capacity
    ("latent_small_decode_t20", CASES["latent_small_decode_t20"]),  # latent layer
    # tiled GEMM
    ("mixtral_small_t1000", CASES["mixtral_small_t1000"]),          # 256-row m-tiles
    ("mixtral_small_t1200_bm192", CASES["mixtral_small_t1200_bm192"]),  # 192-row m-tiles
    ("switch_small_t2000", CASES["switch_small_t2000"]),            # capacity drops
    ("mix_d1152_t300", MIX_S.with_(T=300, d=1152, h=1920)),         # K/128 odd, h % 256 != 0
    ("mix_h5120_t600", MIX_S.with_(T=600, d=1024, h=5120)),         # down K = 5120: 2 chunks
    ("mix_d4224_t400", MIX_S.with_(T=400, d=4224, h=1024)),         # gate/up K: 64 + 2 k-steps
    ("latent_small_t700", CASES["latent_small_t700"]),              # latent layer
)}


@pytest.mark.parametrize("name", list(MX_CASES))
def test_mxfp4_forward_parity(name):
    cfg = MX_CASES[name]
    log(f"[mxfp4 forward] {cfg.name} T={cfg.T} d={cfg.d} h={cfg.h} N={cfg.N} k={cfg.k}")
    ref = oracle_forward(cfg)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out)


@pytest.mark.parametrize("name", ["mcu_t1", "mix_d2048_t40", "latent_small_decode_t20",
                                  "mix_d1152_t300", "mix_h5120_t600", "latent_small_t700"])
def test_mxfp4_stage_expert_ffn(name):
    cfg = MX_CASES[name]
    log(f"[mxfp4 expert_ffn] {cfg.name}")
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


@pytest.mark.parametrize("name", ["mix_d2048_t40", "mix_d1152_t300", "mix_h5120_t600"])
def test_mxfp4_block_scales_are_per_block(name):
    # Every E8M0 scale byte moved by a random -2..+2: the output must follow
    # the oracle with the same edited bytes (a scale applied to the wrong run
    # of 32, the wrong row or the wrong matrix fails this).
    cfg = MX_CASES[name]
    log(f"[mxfp4 scale edit] {cfg.name}")
    w = H.upload_layer(cfg)
    rng = np.random.default_rng(12)
    delta = {m: rng.integers(-2, 3, size=tuple(w[m + "_scale"].shape)).astype(np.int64)
             for m in ("gate", "up", "down")}
    for m in delta:
        edited = H.to_host(w[m + "_scale"]).astype(np.int64) + delta[m]
        w[m + "_scale"] = torch.from_numpy(edited.astype(np.uint8)).cuda()

    def experts(e):
        g, u, dn = cfg.expert(e)
        return tuple(S.MxFp4Rows(x.packed, (x.block_scale.astype(np.int64) + delta[m][e])
                                 .astype(np.uint8))
                     for x, m in ((g, "gate"), (u, "up"), (dn, "down")))
    ref = O.forward(cfg.u(), cfg.w_route(), experts, k=cfg.k, gate=cfg.gate, act=cfg.act,
                    capacity=oracle_capacity(cfg), beta_g=cfg.beta_g, beta_u=cfg.beta_u,
                    alpha=cfg.aux_alpha)
    y, out = run_forward(cfg, weights=w)
    check_forward(cfg, ref, y, out)


@pytest.mark.timeout(600)
def test_mxfp4_full_size_mixtral_decode():
    cfg = C.MIXTRAL_DECODE_MXFP4
    log(f"[mxfp4 full] {cfg.name}")
    ref = oracle_forward(cfg)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out)


@pytest.mark.timeout(1200)
def test_mxfp4_full_size_latent():
    from tests.test_gpu_parity import sample_tokens
    cfg = C.LATENT_MXFP4
    log(f"[mxfp4 full] {cfg.name}: uploading {cfg.N} experts")
    tokens = sample_tokens(cfg.T, 6, cfg.seed)
    ref = oracle_forward(cfg, tokens=tokens)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out, tokens=tokens)


@pytest.mark.timeout(900)
def test_mxfp4_full_size_mixtral_prefill():
    from tests.test_gpu_parity import sample_tokens
    cfg = C.MIXTRAL_PREFILL_MXFP4
    log(f"[mxfp4 full] {cfg.name}")
    tokens = sample_tokens(cfg.T, 24, cfg.seed)
    ref = oracle_forward(cfg, tokens=tokens)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out, tokens=tokens)
