"""The LatentMoE backward on the GPU (moe_latent_backward) against the fp64
oracle's latent_backward.  The library is fed the oracle's routing, dispatch
and expert outputs (rounded to fp32, as the forward hands them over), and a
seeded upstream gradient dy; every gradient is compared: du, dz, dW_route,
dW_ldown, dW_lup, the routed experts' and the shared experts' weights.
Cases: two and one shared experts, none, a capacity limit with the aux term,
a router column count that is not a multiple of 4, few tokens (T padded in
the token-long contractions, most experts unselected: their gradients must
be exact zeros), and one case fed by the GPU's own forward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_11_amd as moe
import synth as S
from tests import harness as H
from tests import parity as PR
from tests.test_gpu_parity import CASES, log, oracle_capacity

pytestmark = pytest.mark.gpu

LAT = CASES["latent_small_t700"]
LB_CASES = {
    "latent_small_t700": LAT,                                          # 2 shared experts
    "latent_small_n97": CASES["latent_small_n97"],                     # N % 4 != 0, 1 shared
    "latent_small_noshared": LAT.with_(name="latent_small_noshared", T=500, n_shared=0,
                                      h_shared=0),
    "latent_small_cap_aux": LAT.with_(name="latent_small_cap_aux", T=640, capacity_factor=1.0),
    "latent_small_t20": CASES["latent_small_decode_t20"],              # T < 64, empty experts
}
AUX = {"latent_small_cap_aux": 0.8}


def oracle_backward(cfg, dy64, aux):
    return O.latent_backward(cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), cfg.w_ldown(),
                             cfg.w_lup(), lambda j: cfg.shared(j), cfg.n_shared, dy64, k=cfg.k,
                             gate=cfg.gate, act=cfg.act, capacity=oracle_capacity(cfg),
                             beta_g=cfg.beta_g, beta_u=cfg.beta_u, rms_eps=cfg.rms_eps,
                             alpha=cfg.aux_alpha, aux_scale=aux)


def grad_buffers(cfg):
    f = lambda *s: torch.full(s, float("nan"), device="cuda")  # noqa: E731
    g = {"du": f(cfg.T, cfg.d), "dz": f(cfg.T, cfg.N), "dW_route": f(cfg.N, cfg.d),
         "dW_ldown": f(cfg.l, cfg.d), "dW_lup": f(cfg.d, cfg.l),
         "dW_gate": f(cfg.N, cfg.h, cfg.l), "dW_up": f(cfg.N, cfg.h, cfg.l),
         "dW_down": f(cfg.N, cfg.l, cfg.h)}
    if cfg.n_shared:
        g.update(dWs_gate=f(cfg.n_shared, cfg.h_shared, cfg.d),
                 dWs_up=f(cfg.n_shared, cfg.h_shared, cfg.d),
                 dWs_down=f(cfg.n_shared, cfg.d, cfg.h_shared))
    return g


def fwd_from_oracle(ref):
    """The forward's outputs as the library would hold them, from the oracle."""
    rt, disp = ref["route"], ref["disp"]
    st = O.balance_stats(rt["p"], 0.01)  # only f enters the backward
    stats = np.concatenate([st["f"], st["P"], [st["n_sum_fP"], st["aux"]]])
    i32 = lambda x: H.to_device(np.asarray(x).astype(np.int32))  # noqa: E731
    f32 = lambda x: H.to_device(S.round_to(np.asarray(x, dtype=np.float64), "f32"))  # noqa: E731
    return {"topk_idx": i32(rt["idx"].reshape(-1)), "topk_w": f32(rt["a"].reshape(-1)),
            "stats": f32(stats), "offsets": i32(disp["offsets"]),
            "kept_offsets": i32(disp["kept_offsets"]), "perm": i32(disp["perm"]),
            "row_of": i32(disp["row_of"]), "y_perm": f32(ref["y_rows"])}


def compare(cfg, g, ref):
    errs = {}
    for key in g:
        errs[key] = PR.rel_err(H.to_host(g[key]).astype(np.float64), ref[key])
    log("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= PR.TOL["bf16"], errs
    # Only the selected experts receive gradient: exact zeros elsewhere.
    empty = np.flatnonzero(np.diff(ref["disp"]["kept_offsets"]) == 0)
    for e in empty:
        for key in ("dW_gate", "dW_up", "dW_down"):
            assert not torch.any(g[key][e] != 0), (key, e)
    return errs


@pytest.mark.parametrize("name", list(LB_CASES))
def test_latent_backward_parity(name):
    cfg = LB_CASES[name]
    aux = AUX.get(name, 0.0)
    log(f"[latent backward] {name} T={cfg.T} d={cfg.d} l={cfg.l} h={cfg.h} N={cfg.N} "
        f"k={cfg.k} S={cfg.n_shared} aux={aux}")
    dy_st = S.normal_stored(43, 96, cfg.T * cfg.d, 0.5, "bf16").reshape(cfg.T, cfg.d)
    ref = oracle_backward(cfg, O.expand(dy_st), aux)
    if cfg.capacity_factor is not None:
        assert int(ref["disp"]["drop"].sum()) > 0
    if name == "latent_small_t20":
        assert np.any(np.diff(ref["disp"]["kept_offsets"]) == 0)
    desc = H.desc_for(cfg)
    w = H.upload_layer(cfg)
    g = grad_buffers(cfg)
    moe.moe_latent_backward(desc, w, H.to_device(cfg.u()), fwd_from_oracle(ref),
                            H.to_device(dy_st), g, moe.backward_workspace(desc), aux_scale=aux)
    torch.cuda.synchronize()
    compare(cfg, g, ref)


@pytest.mark.parametrize("save_gate_up", [False, True])
def test_latent_backward_after_gpu_forward(save_gate_up):
    """The GPU forward's own outputs feed the backward (same selection as the
    oracle's on this seed: every token's margin is far from a tie), with the
    routed experts' G | U recomputed or kept by the forward."""
    cfg = LAT
    log(f"[latent backward] chained forward -> backward latent_small_t700, saved G|U "
        f"{save_gate_up}")
    dy_st = S.normal_stored(44, 96, cfg.T * cfg.d, 0.5, "bf16").reshape(cfg.T, cfg.d)
    ref = oracle_backward(cfg, O.expand(dy_st), 0.3)
    desc = H.desc_for(cfg)
    w = H.upload_layer(cfg)
    out = H.out_buffers(cfg)
    R = int(ref["disp"]["kept_offsets"][-1])
    out["y_perm"] = torch.empty((R, cfg.l), dtype=torch.float32, device="cuda")
    if save_gate_up:
        out["gate_up"] = torch.empty((R, 2 * cfg.h), dtype=torch.bfloat16, device="cuda")
    u = H.to_device(cfg.u())
    moe.moe_forward(desc, w, u, H.y_buffer(cfg), out, moe.workspace(desc))
    torch.cuda.synchronize()
    assert np.array_equal(H.to_host(out["topk_idx"]).reshape(cfg.T, cfg.k), ref["route"]["idx"])
    g = grad_buffers(cfg)
    moe.moe_latent_backward(desc, w, u, out, H.to_device(dy_st), g, moe.backward_workspace(desc),
                            aux_scale=0.3)
    torch.cuda.synchronize()
    compare(cfg, g, ref)


@pytest.mark.timeout(1500)
def test_latent_backward_full_size_sampled():
    """The full LatentMoE workload (T=8192, 896 experts, top-16, 2 shared):
    GPU forward, then every gradient on the GPU; du and dz compared on
    sampled tokens against the oracle's per-token form (their 16 experts
    each), with the aux term on."""
    from synth import configs as C
    from tests.test_gpu_parity import sample_tokens
    cfg = C.LATENT
    aux = 0.5
    log(f"[latent backward full] {cfg.name}: uploading {cfg.N} experts")
    desc = H.desc_for(cfg)
    w = H.upload_layer(cfg)
    u = H.to_device(cfg.u())
    out = H.out_buffers(cfg)
    out["y_perm"] = torch.empty((cfg.T * cfg.k, cfg.l), dtype=torch.float32, device="cuda")
    ws = moe.workspace(desc)
    moe.moe_forward(desc, w, u, H.y_buffer(cfg), out, ws)
    torch.cuda.synchronize()
    del ws
    dy_st = S.normal_stored(45, 96, cfg.T * cfg.d, 0.5, "bf16").reshape(cfg.T, cfg.d)
    g = grad_buffers(cfg)
    log("  backward")
    moe.moe_latent_backward(desc, w, u, out, H.to_device(dy_st), g, moe.backward_workspace(desc),
                            aux_scale=aux)
    torch.cuda.synchronize()
    tokens = sample_tokens(cfg.T, 4, cfg.seed)
    log(f"  oracle on tokens {tokens.tolist()}")
    ref = O.latent_backward_tokens(cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), cfg.w_ldown(),
                                   cfg.w_lup(), lambda j: cfg.shared(j), cfg.n_shared,
                                   O.expand(dy_st[tokens]), tokens, k=cfg.k, gate=cfg.gate,
                                   act=cfg.act, beta_g=cfg.beta_g, beta_u=cfg.beta_u,
                                   rms_eps=cfg.rms_eps, alpha=cfg.aux_alpha, aux_scale=aux)
    gidx = H.to_host(out["topk_idx"]).reshape(cfg.T, cfg.k)[tokens]
    same = np.array([set(a.tolist()) == set(b.tolist()) for a, b in zip(gidx, ref["idx"])])
    assert same.all() or np.all(ref["margin"][~same] < PR.NEAR_TIE)
    du = H.to_host(g["du"][torch.as_tensor(tokens, device="cuda")]).astype(np.float64)
    dz = H.to_host(g["dz"][torch.as_tensor(tokens, device="cuda")]).astype(np.float64)
    e_du = PR.rel_err(du[same], ref["du"][same])
    e_dz = PR.rel_err(dz[same], ref["dz"][same])
    log(f"  du rel err {e_du:.2e}, dz rel err {e_dz:.2e} on {int(same.sum())} tokens")
    assert max(e_du, e_dz) <= PR.TOL["bf16"]
