"""GPU parity: the HIP library, called through its C ABI, against the fp64 oracle
on the same seeded inputs.  Stage tests feed each entry point oracle-made
inputs; end-to-end tests run moe_forward and compare every output."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_11_amd as moe
from synth import configs as C
from tests import harness as H
from tests import parity as PR
import synth as S

pytestmark = pytest.mark.gpu

# Parity cases the oracle finishes in seconds: several tiles and ragged tails.
MIX_S = C.MIXTRAL_PREFILL.with_(name="mixtral_small_t1000", T=1000, d=1024, h=2048)
CASES = {
    "tiny": C.TINY,
    "tiny_k4": C.TINY.with_(name="tiny_k4", k=4),
    "tiny_planted_c4": C.TINY_PLANTED,
    "tiny_planted_c6": C.TINY_PLANTED.with_(capacity_factor=1.5),
    "tiny_planted_c10": C.TINY_PLANTED.with_(capacity_factor=2.5),
    "tiny_planted_empty_expert": C.TINY_PLANTED.with_(planted=tuple([0] * 10 + [1] * 5 + [3]),
                                                      capacity_factor=1.5),
    "mcu_t1": C.MCU_DECODE,
    "mcu_t4096": C.MCU_BATCH,
    "mixtral_small_t1000": MIX_S,
    "mixtral_small_t37_decode": MIX_S.with_(T=37),
    "mixtral_small_t64_decode": MIX_S.with_(T=64),
    # decode with K = 2176: each wave's 544-wide k range holds several
    # pipelined weight windows and a 32-wide remainder (two and four token groups)
    "mixtral_k2176_t30_decode": MIX_S.with_(T=30, d=2176, h=2176),
    "mixtral_k2176_t60_decode": MIX_S.with_(T=60, d=2176, h=2176),
    "mixtral_small_t65": MIX_S.with_(T=65),
    "mixtral_small_t3000_tiled": MIX_S.with_(T=3000),
    # about 300 rows per expert: 192-row m-tiles, two or three per expert
    "mixtral_small_t1200_bm192": MIX_S.with_(T=1200),
    "switch_small_t2000": C.SWITCH_SKEWED.with_(T=2000, d=1024, h=1024),
    "switch_small_t48_decode": C.SWITCH_SKEWED.with_(T=48, d=1024, h=1024),
    "switch_small_t6000_tiled": C.SWITCH_SKEWED.with_(T=6000, d=1024, h=1024),
    "latent_small_t700": C.LATENT.with_(T=700, d=512, l=384, h=256, N=96, k=6, h_shared=256),
    "latent_small_stream_t900": C.LATENT.with_(T=900, d=512, l=512, h=256, N=96, k=6,
                                               h_shared=256),
    "latent_small_wave_router": C.LATENT.with_(T=300, d=512, l=256, h=256, N=40, k=4,
                                               h_shared=128, n_shared=1),
    "latent_small_decode_t20": C.LATENT.with_(T=20, d=512, l=384, h=256, N=96, k=6, h_shared=256),
    # router logits through the GEMM with a column count that is not a
    # multiple of 4
    "latent_small_n97": C.LATENT.with_(T=300, d=512, l=256, h=256, N=97, k=5, h_shared=128,
                                       n_shared=1),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_capacity(cfg):
    if cfg.capacity_factor is None:
        return None
    return O.capacity_from_factor(cfg.T, cfg.N, cfg.k, cfg.capacity_factor)


def oracle_forward(cfg, tokens=None):
    experts = lambda e: cfg.expert(e)  # noqa: E731
    cap = oracle_capacity(cfg)
    u = cfg.u()
    if cfg.latent:
        return O.latent_forward(u, cfg.w_route(), experts, cfg.w_ldown(), cfg.w_lup(),
                                lambda j: cfg.shared(j), cfg.n_shared, k=cfg.k, gate=cfg.gate,
                                act=cfg.act, capacity=cap, beta_g=cfg.beta_g, beta_u=cfg.beta_u,
                                rms_eps=cfg.rms_eps, alpha=cfg.aux_alpha, tokens=tokens)
    return O.forward(u, cfg.w_route(), experts, k=cfg.k, gate=cfg.gate, act=cfg.act,
                     capacity=cap, beta_g=cfg.beta_g, beta_u=cfg.beta_u, alpha=cfg.aux_alpha,
                     tokens=tokens)


def run_forward(cfg, weights=None, u=None):
    desc = H.desc_for(cfg)
    w = weights if weights is not None else H.upload_layer(cfg)
    u = u if u is not None else H.to_device(cfg.u())
    y = H.y_buffer(cfg)
    out = H.out_buffers(cfg)
    ws = moe.workspace(desc)
    moe.moe_forward(desc, w, u, y, out, ws)
    torch.cuda.synchronize()
    return y, out


def check_forward(cfg, ref, y, out, tokens=None):
    """Compare a moe_forward result against the oracle (all tokens or a sample)."""
    T, k = cfg.T, cfg.k
    gidx = H.to_host(out["topk_idx"])
    routing = PR.compare_routing(cfg, gidx, ref)
    ok = PR.usable_tokens(cfg, ref, routing)
    # Combine weights.
    gw = H.to_host(out["topk_w"]).reshape(T, k)
    werr = np.abs(gw[routing["same"]] - ref["a"][routing["same"]]).max()
    assert werr <= PR.W_TOL[cfg.act_dtype], werr
    # Dispatch: bit-exact when no near tie flipped.
    if routing["flipped"] == 0:
        PR.compare_dispatch({key: H.to_host(out[key]) for key in
                             ("counts", "offsets", "kept_offsets", "perm", "row_of", "drop")},
                            ref["disp"])
    # Balance statistics (argmax shares exact, means to fp32 accuracy).
    st = H.to_host(out["stats"])
    N = cfg.N
    if routing["flipped"] == 0:
        assert np.array_equal(np.rint(st[:N] * T).astype(np.int64),
                              np.rint(ref["stats"]["f"] * T).astype(np.int64))
    assert np.allclose(st[N:2 * N], ref["stats"]["P"], rtol=1e-4, atol=1e-6)
    assert abs(st[2 * N] - ref["stats"]["n_sum_fP"]) <= 1e-4 * max(1.0, ref["stats"]["n_sum_fP"])
    # Outputs.
    yg = H.expand_device_output(y)
    if tokens is not None:
        yg = yg[tokens]
        ok = ok[tokens]
    err = PR.rel_err(yg[ok], ref["y"][ok])
    log(f"  {cfg.name}: rel err {err:.3e}, near ties {routing['near']}, flipped "
        f"{routing['flipped']}, compared {int(ok.sum())} tokens")
    assert err <= PR.TOL[cfg.act_dtype], err
    return routing


# ---------------------------------------------------------------------------
# End-to-end on parity-size cases
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", list(CASES))
def test_forward_parity(name):
    cfg = CASES[name]
    log(f"[forward] {name} T={cfg.T} d={cfg.d} h={cfg.h} N={cfg.N} k={cfg.k}")
    ref = oracle_forward(cfg)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out)
    if cfg.planted is not None:
        # The worked example: loads [10,3,2,1]; C = 4/6/10 drop 6/4/0.
        drops = int(H.to_host(out["drop"]).sum())
        assert drops == int(ref["disp"]["drop"].sum())


def test_planted_drops_match_page_example():
    for c, drops in ((1.0, 6), (1.5, 4), (2.5, 0)):
        cfg = C.TINY_PLANTED.with_(capacity_factor=c)
        log(f"[planted] capacity factor {c}")
        y, out = run_forward(cfg)
        assert H.to_host(out["counts"]).tolist() == [10, 3, 2, 1]
        dr = H.to_host(out["drop"])
        assert int(dr.sum()) == drops
        yd = H.expand_device_output(y)[dr.astype(bool)]
        assert np.all(yd == 0.0)


def test_zero_capacity_gives_zero_output():
    cfg = MIX_S.with_(T=300)
    log("[capacity 0]")
    desc = H.desc_for(cfg, capacity=0)
    w = H.upload_layer(cfg)
    u = H.to_device(cfg.u())
    y = H.y_buffer(cfg)
    y.fill_(1.0)
    out = H.out_buffers(cfg)
    moe.moe_forward(desc, w, u, y, out, moe.workspace(desc))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    assert int(H.to_host(out["drop"]).sum()) == cfg.T * cfg.k


def test_deterministic_bitwise():
    for cfg in (MIX_S, CASES["latent_small_t700"], C.MCU_DECODE):
        log(f"[determinism] {cfg.name}")
        w = H.upload_layer(cfg)
        u = H.to_device(cfg.u())
        y1, o1 = run_forward(cfg, w, u)
        y2, o2 = run_forward(cfg, w, u)
        assert torch.equal(y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1,
                           y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2)
        for key in o1:
            assert torch.equal(o1[key], o2[key]), key


# One case per expert-kernel family: fp32 SIMT (tiny), decode-sized T (mcu_t1,
# T = 37), the tiled grouped GEMM with 256- and 192-row m-tiles, and the
# latent layer (router GEMM, routed experts at width l).
PERTURB_CASES = ["tiny", "mcu_t1", "mixtral_small_t37_decode", "mixtral_small_t1000",
                 "mixtral_small_t1200_bm192", "latent_small_t700"]


@pytest.mark.parametrize("name", PERTURB_CASES)
def test_unselected_expert_perturbation(name):
    """Only selected experts take part ([LAT]'s check that only selected
    experts receive gradient, in its forward form): an expert kept out of
    every token's selection by a very negative selection bias can have its
    weights scaled by 1000 without changing a single output bit.  The biased
    forward itself is compared with the oracle's."""
    cfg = CASES[name]
    banned = [cfg.N - 1, 0] if cfg.N > 4 else [cfg.N - 1]
    bias = np.zeros(cfg.N, dtype=np.float32)
    bias[banned] = -1e9
    log(f"[perturb] {name}: experts {banned} kept out by the selection bias")
    w = H.upload_layer(cfg)
    w["selection_bias"] = H.to_device(bias)
    u = H.to_device(cfg.u())
    y0, o0 = run_forward(cfg, w, u)
    gidx = H.to_host(o0["topk_idx"])
    assert not np.isin(gidx, banned).any()
    ref = O.forward(cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), k=cfg.k, gate=cfg.gate,
                    act=cfg.act, capacity=oracle_capacity(cfg), beta_g=cfg.beta_g,
                    beta_u=cfg.beta_u, alpha=cfg.aux_alpha, bias=bias.astype(np.float64)) \
        if not cfg.latent else O.latent_forward(
            cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), cfg.w_ldown(), cfg.w_lup(),
            lambda j: cfg.shared(j), cfg.n_shared, k=cfg.k, gate=cfg.gate, act=cfg.act,
            capacity=oracle_capacity(cfg), beta_g=cfg.beta_g, beta_u=cfg.beta_u,
            rms_eps=cfg.rms_eps, alpha=cfg.aux_alpha, bias=bias.astype(np.float64))
    gi = gidx.reshape(cfg.T, cfg.k)
    same = np.all(gi == ref["idx"], axis=1)
    assert same.sum() >= cfg.T - max(1, cfg.T // 100)
    err = PR.rel_err(H.expand_device_output(y0)[same], ref["y"][same])
    log(f"  biased forward vs oracle: rel err {err:.3e} on {int(same.sum())} tokens")
    assert err <= PR.TOL[cfg.act_dtype]
    for e in banned:
        for key in ("W_gate", "W_up", "W_down"):
            w[key][e] *= 1000.0
    y1, _ = run_forward(cfg, w, u)
    a = y0.view(torch.int16) if y0.dtype == torch.bfloat16 else y0
    b = y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1
    assert torch.equal(a, b)


HOT_DECODE_CASES = [
    # (case, expert weights): at decode sizes a workgroup holds one 16-token
    # group of an expert up to T = 32 and two beyond, and the grid's z takes
    # the rest; here every token goes to one or two experts, so those extra
    # workgroups do the work.
    ("mixtral_small_t32_decode", "bf16"),
    ("mixtral_small_t32_decode", "mxfp4"),
    ("mixtral_small_t64_decode", "bf16"),
    ("mixtral_small_t64_decode", "fp8"),
    ("mixtral_small_t64_decode", "mxfp4"),
    ("mixtral_small_t37_decode", "mxfp4"),
    ("mixtral_k2176_t30_decode", "fp8"),
    ("mixtral_k2176_t60_decode", "bf16"),
]


# Hot-expert cases beyond CASES: T = 32, two workgroups of one group each
# on the hot experts (the MXFP4 down on 512-k windows).
HOT_ONLY = {"mixtral_small_t32_decode": MIX_S.with_(T=32)}


@pytest.mark.parametrize("name,wfmt", HOT_DECODE_CASES, ids=lambda v: str(v))
def test_decode_hot_experts(name, wfmt):
    cfg = CASES[name] if name in CASES else HOT_ONLY[name]
    if wfmt != "bf16":
        cfg = cfg.with_(name=f"{cfg.name}_{wfmt}", w_dtype=wfmt)
    hot = [2, 5]
    bias = np.zeros(cfg.N, dtype=np.float32)
    bias[hot[0]] = 1e4
    if cfg.k > 1:
        bias[hot[1]] = 5e3
    log(f"[hot decode] {cfg.name} T={cfg.T}: every token to experts {hot[:cfg.k]}")
    w = H.upload_layer(cfg)
    w["selection_bias"] = H.to_device(bias)
    y, out = run_forward(cfg, w)
    counts = H.to_host(out["counts"])
    assert counts[hot[0]] == cfg.T
    ref = O.forward(cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), k=cfg.k, gate=cfg.gate,
                    act=cfg.act, capacity=oracle_capacity(cfg), beta_g=cfg.beta_g,
                    beta_u=cfg.beta_u, alpha=cfg.aux_alpha, bias=bias.astype(np.float64))
    gi = H.to_host(out["topk_idx"]).reshape(cfg.T, cfg.k)
    assert np.array_equal(gi, ref["idx"])
    err = PR.rel_err(H.expand_device_output(y), ref["y"])
    log(f"  rel err {err:.3e}")
    assert err <= PR.TOL[cfg.act_dtype]


# ---------------------------------------------------------------------------
# Stage tests: each entry point fed oracle-made inputs
# ---------------------------------------------------------------------------

# Expert-kernel families: SIMT (fp32), decode (T <= 64), tiled grouped GEMM
# (otherwise; one and several m-tiles per expert, 256- and 192-row tiles).
STAGE_CASES = ["tiny", "tiny_planted_c4", "mcu_t4096", "mixtral_small_t1000",
               "mixtral_small_t3000_tiled", "mixtral_small_t1200_bm192",
               "mixtral_small_t37_decode", "switch_small_t2000",
               "switch_small_t6000_tiled", "latent_small_t700", "latent_small_stream_t900"]


@pytest.mark.parametrize("name", STAGE_CASES)
def test_stage_route(name):
    cfg = CASES[name]
    log(f"[route] {name}")
    desc = H.desc_for(cfg)
    ref = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    E = cfg.T * cfg.k
    idx = torch.empty(E, dtype=torch.int32, device="cuda")
    w = torch.empty(E, dtype=torch.float32, device="cuda")
    st = torch.empty(2 * cfg.N + 2, dtype=torch.float32, device="cuda")
    moe.moe_route(desc, H.to_device(cfg.u()), H.to_device(cfg.w_route()), idx, w, st,
                  moe.workspace(desc))
    torch.cuda.synchronize()
    routing = PR.compare_routing(cfg, H.to_host(idx), ref)
    same = routing["same"]
    gw = H.to_host(w).reshape(cfg.T, cfg.k)
    assert np.abs(gw[same] - ref["a"][same]).max() <= PR.W_TOL[cfg.act_dtype]
    stats = O.balance_stats(ref["p"], cfg.aux_alpha)
    s = H.to_host(st)
    assert np.allclose(s[cfg.N:2 * cfg.N], stats["P"], rtol=1e-4, atol=1e-6)
    assert abs(s[2 * cfg.N + 1] - stats["aux"]) <= 1e-4 * max(stats["aux"], 1e-3)


# Router shapes beyond the workloads: fewer than 8 experts, every d = 512 CH
# of the LDS-resident router (CH = 1, 2, 4, 8), fp32 router weights, a
# selection bias, a token count that is not a multiple of the 4-token groups.
ROUTE_SHAPES = [
    dict(T=1001, d=2048, N=6, k=3, router_dtype="bf16", bias=False),
    dict(T=1001, d=2048, N=6, k=3, router_dtype="bf16", bias=True),
    dict(T=523, d=512, N=5, k=1, router_dtype="f32", bias=True),
    dict(T=2050, d=1024, N=8, k=2, router_dtype="f32", bias=False),
    dict(T=4099, d=4096, N=7, k=2, router_dtype="bf16", bias=True),
    # d = 4096 (the tile router's CH = 8): a token count just past the
    # one-block-per-token router, a partial last 4-token group with every
    # expert selected, three experts with top-1 and a selection bias
    dict(T=300, d=4096, N=8, k=2, router_dtype="bf16", bias=False),
    dict(T=2061, d=4096, N=8, k=8, router_dtype="bf16", bias=False),
    dict(T=2500, d=4096, N=3, k=1, router_dtype="bf16", bias=True),
    dict(T=300, d=1536, N=8, k=2, router_dtype="bf16", bias=False),  # older wave router
    # N > 64: router GEMM, then the top-k over its logits (in two K-halves
    # while the GEMM's tiles would fill under three quarters of the CUs)
    dict(T=700, d=1024, N=97, k=4, router_dtype="bf16", bias=False, h=128),
    dict(T=1500, d=512, N=300, k=8, router_dtype="bf16", bias=True, h=128),
    dict(T=513, d=512, N=1024, k=16, router_dtype="bf16", bias=False, h=128),
    dict(T=2000, d=256, N=896, k=16, router_dtype="bf16", bias=True, h=128),  # one K pass
    dict(T=300, d=768, N=65, k=2, router_dtype="bf16", bias=False, h=128),
]


@pytest.mark.parametrize("shape", ROUTE_SHAPES, ids=lambda s: "T{T}_d{d}_N{N}_k{k}_{router_dtype}"
                         "{b}".format(b="_bias" if s["bias"] else "", **s))
def test_stage_route_shapes(shape):
    sh = dict(shape)
    with_bias = sh.pop("bias")
    sh.setdefault("h", 256)
    cfg = C.MIXTRAL_PREFILL.with_(name="route_shape", seed=11, **sh)
    log(f"[route shape] {sh} bias={with_bias}")
    desc = H.desc_for(cfg)
    bias = None
    if with_bias:
        bias = np.linspace(-0.3, 0.3, cfg.N).astype(np.float32)
    ref = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate,
                  None if bias is None else bias.astype(np.float64))
    E = cfg.T * cfg.k
    idx = torch.empty(E, dtype=torch.int32, device="cuda")
    w = torch.empty(E, dtype=torch.float32, device="cuda")
    st = torch.empty(2 * cfg.N + 2, dtype=torch.float32, device="cuda")
    ws = moe.workspace(desc)
    if bias is None:
        moe.moe_route(desc, H.to_device(cfg.u()), H.to_device(cfg.w_route()), idx, w, st, ws)
    else:
        moe.moe_route_biased(desc, H.to_device(cfg.u()), H.to_device(cfg.w_route()),
                             H.to_device(bias), idx, w, st, ws)
    torch.cuda.synchronize()
    routing = PR.compare_routing(cfg, H.to_host(idx), ref)
    same = routing["same"]
    gw = H.to_host(w).reshape(cfg.T, cfg.k)
    assert np.abs(gw[same] - ref["a"][same]).max() <= PR.W_TOL[cfg.act_dtype]
    stats = O.balance_stats(ref["p"], cfg.aux_alpha)
    s = H.to_host(st)
    if routing["flipped"] == 0:
        assert np.array_equal(np.rint(s[:cfg.N] * cfg.T).astype(np.int64),
                              np.rint(stats["f"] * cfg.T).astype(np.int64))
    assert np.allclose(s[cfg.N:2 * cfg.N], stats["P"], rtol=1e-4, atol=1e-6)
    assert abs(s[2 * cfg.N + 1] - stats["aux"]) <= 1e-4 * max(stats["aux"], 1e-3)
    # The forward (statistics finished by the dispatch launches) agrees with
    # the router's own statistics.
    w_all = H.upload_layer(cfg)
    if bias is not None:
        w_all["selection_bias"] = H.to_device(bias)
    y, out = run_forward(cfg, w_all)
    assert torch.equal(out["topk_idx"], idx)
    assert np.allclose(H.to_host(out["stats"]), s, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("d", [512, 256], ids=["two_k_halves", "one_k_pass"])
def test_stage_route_logits_exact_ties(d):
    """Duplicated router rows give bit-identical logits (every output column
    sums the same products in the same order), so the top-k over logits must
    break those ties by index: of a duplicated pair (a < b), b is chosen only
    after a, in a later slot."""
    cfg = C.MIXTRAL_PREFILL.with_(name="route_ties", T=600, d=d, h=128, N=130, k=8, seed=12,
                                  router_dtype="bf16")
    log(f"[route ties] d={d}")
    desc = H.desc_for(cfg)
    wr = np.array(cfg.w_route())
    pairs = [(5, 70), (6, 7), (64, 128), (0, 129)]
    for a, b in pairs:
        wr[b] = wr[a]
    E = cfg.T * cfg.k
    idx = torch.empty(E, dtype=torch.int32, device="cuda")
    w = torch.empty(E, dtype=torch.float32, device="cuda")
    st = torch.empty(2 * cfg.N + 2, dtype=torch.float32, device="cuda")
    ws = moe.workspace(desc)
    moe.moe_route(desc, H.to_device(cfg.u()), H.to_device(wr), idx, w, st, ws)
    torch.cuda.synchronize()
    gi = H.to_host(idx).reshape(cfg.T, cfg.k)
    ref = O.route(O.expand(cfg.u()), O.expand(wr), cfg.k, cfg.gate)
    routing = PR.compare_routing(cfg, gi.reshape(-1), ref)
    both = 0
    for t in range(cfg.T):
        row = list(gi[t])
        assert len(set(row)) == cfg.k
        for a, b in pairs:
            if b in row:
                assert a in row and row.index(a) < row.index(b), (t, row, a, b)
                both += 1
    assert both > 0, "no token selected a duplicated pair"
    assert routing["flipped"] <= routing["near"]


@pytest.mark.parametrize("shape", [
    dict(T=4099, d=4096, N=7, k=2),     # tile router (N <= 8, large T)
    dict(T=100, d=1024, N=8, k=2),      # small-T router
    dict(T=700, d=1024, N=97, k=4),     # logit GEMM + top-k
], ids=lambda s: "T{T}_N{N}".format(**s))
def test_stage_route_nan_scores(shape):
    """A router row of NaNs makes that expert's scores NaN for every token:
    the selection must still give k distinct experts below N per token (the
    NaN expert ranks last), so that nothing downstream indexes out of range."""
    cfg = C.MIXTRAL_PREFILL.with_(name="route_nan", h=128, seed=13, router_dtype="bf16", **shape)
    log(f"[route nan] {shape}")
    desc = H.desc_for(cfg)
    wr = np.array(cfg.w_route())
    wr[3] = 0x7FC0  # bf16 quiet NaN
    E = cfg.T * cfg.k
    idx = torch.empty(E, dtype=torch.int32, device="cuda")
    w = torch.empty(E, dtype=torch.float32, device="cuda")
    st = torch.empty(2 * cfg.N + 2, dtype=torch.float32, device="cuda")
    ws = moe.workspace(desc)
    moe.moe_route(desc, H.to_device(cfg.u()), H.to_device(wr), idx, w, st, ws)
    torch.cuda.synchronize()
    gi = H.to_host(idx).reshape(cfg.T, cfg.k)
    assert gi.min() >= 0 and gi.max() < cfg.N
    assert all(len(set(r)) == cfg.k for r in gi)
    assert not (gi == 3).any()


@pytest.mark.parametrize("name", STAGE_CASES + ["switch_small_t48_decode"])
def test_stage_dispatch(name):
    cfg = CASES[name]
    log(f"[dispatch] {name}")
    desc = H.desc_for(cfg)
    ref = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    rd = O.dispatch(ref["idx"], cfg.N, oracle_capacity(cfg))
    out = H.out_buffers(cfg)
    moe.moe_dispatch(desc, H.to_device(ref["idx"].reshape(-1)), out["counts"], out["offsets"],
                     out["kept_offsets"], out["perm"], out["row_of"], out["drop"],
                     moe.workspace(desc))
    torch.cuda.synchronize()
    PR.compare_dispatch({k: H.to_host(out[k]) for k in
                         ("counts", "offsets", "kept_offsets", "perm", "row_of", "drop")}, rd)


def test_stage_dispatch_random_assignments():
    # Many experts, many chunks, capacity: random distinct top-k rows; the
    # last five take the single-block path (at most 1024 entries), up to its
    # limits of 1024 entries and 1024 experts.
    rng = np.random.default_rng(0)
    for T, N, k, cap in ((5000, 896, 16, 70), (3000, 8, 2, 700), (100, 1024, 32, 2),
                         (2049, 64, 3, -1), (32, 1024, 32, 1), (512, 8, 2, 100), (1, 8, 2, -1),
                         (33, 96, 6, 3), (200, 5, 5, 150)):
        log(f"[dispatch random] T={T} N={N} k={k} cap={cap}")
        cfg = C.LATENT.with_(T=T, N=N, k=k)
        idx = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
        desc = H.desc_for(cfg, capacity=cap)
        out = H.out_buffers(cfg)
        moe.moe_dispatch(desc, H.to_device(idx.reshape(-1)), out["counts"], out["offsets"],
                         out["kept_offsets"], out["perm"], out["row_of"], out["drop"],
                         moe.workspace(desc))
        torch.cuda.synchronize()
        rd = O.dispatch(idx, N, None if cap < 0 else cap)
        PR.compare_dispatch({key: H.to_host(out[key]) for key in
                             ("counts", "offsets", "kept_offsets", "perm", "row_of", "drop")}, rd)


@pytest.mark.parametrize("name", STAGE_CASES + ["mcu_t1", "latent_small_decode_t20"])
def test_stage_expert_ffn(name):
    cfg = CASES[name]
    log(f"[expert_ffn] {name}")
    desc = H.desc_for(cfg)
    u64 = O.expand(cfg.u())
    ref = O.route(u64, O.expand(cfg.w_route()), cfg.k, cfg.gate)
    rd = O.dispatch(ref["idx"], cfg.N, oracle_capacity(cfg))
    # Expert input: u, or for the latent layer a seeded stand-in for x_l.
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
    moe.moe_expert_ffn(desc, H.to_device(x_st), H.to_device(rd["perm"]),
                       H.to_device(rd["offsets"]), H.to_device(rd["kept_offsets"]), w["W_gate"],
                       w["W_up"], w["W_down"], y_perm, moe.workspace(desc))
    torch.cuda.synchronize()
    if R == 0:
        return
    yr = np.stack([rows[r] for r in range(R)])
    err = PR.rel_err(H.to_host(y_perm)[:R].astype(np.float64), yr)
    log(f"  rel err {err:.3e}")
    assert err <= PR.TOL[cfg.act_dtype]


@pytest.mark.parametrize("name", STAGE_CASES)
def test_stage_combine(name):
    cfg = CASES[name]
    log(f"[combine] {name}")
    desc = H.desc_for(cfg)
    ref = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    rd = O.dispatch(ref["idx"], cfg.N, oracle_capacity(cfg))
    R = max(int(rd["kept_offsets"][-1]), 1)
    width = cfg.x_width
    y_rows = S.normal_stored(cfg.seed + 7, 98, R * width, 1.0, "f32").reshape(R, width)
    a32 = S.round_to(ref["a"], "f32")
    want = O.combine_rows(O.expand(y_rows), rd["row_of"], O.expand(a32),
                          rms_eps=cfg.rms_eps if cfg.latent else None)
    out_dtype = torch.bfloat16 if (cfg.latent or cfg.act_dtype == "bf16") else torch.float32
    y = torch.empty((cfg.T, width), dtype=out_dtype, device="cuda")
    moe.moe_combine(desc, H.to_device(y_rows), H.to_device(rd["row_of"]),
                    H.to_device(a32.reshape(-1)), y)
    torch.cuda.synchronize()
    err = PR.rel_err(H.expand_device_output(y), want)
    # fp32 sums then one rounding to the output dtype.
    tol = 2 ** -8 if out_dtype == torch.bfloat16 else 1e-6
    assert err <= tol, err


# ---------------------------------------------------------------------------
# Full-size workloads: every routing/dispatch output, sampled y rows
# ---------------------------------------------------------------------------


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


def tile_edge_tokens(cfg, experts=None, tiles=(256, 192)):
    """Tokens whose rows sit at the edges of the expert GEMMs' m-tiles: in
    each expert's kept range, its first two and last two rows (the last one
    in the ragged final tile) and the rows either side of every multiple of
    the m-tile height (both heights the library chooses between).  The
    dispatch is the oracle's, over every token."""
    r = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    disp = O.dispatch(r["idx"], cfg.N, oracle_capacity(cfg))
    toks = set()
    for e in (range(cfg.N) if experts is None else experts):
        lo, L = int(disp["offsets"][e]), int(disp["kept_counts"][e])
        if L == 0:
            continue
        js = {0, min(1, L - 1), L - 1, max(L - 2, 0)}
        for bm in tiles:
            for m in range(bm, L, bm):
                js |= {m - 1, m}
        toks |= {int(disp["perm"][lo + j]) // cfg.k for j in js}
    return toks, disp


@pytest.mark.parametrize("cfg", [C.MIXTRAL_PREFILL, C.MIXTRAL_DECODE, C.SWITCH_SKEWED,
                                 C.MCU_BATCH, C.MCU_DECODE, C.TINY],
                         ids=lambda c: c.name)
@pytest.mark.timeout(600)
def test_full_size_forward(cfg):
    log(f"[full] {cfg.name}")
    tokens = None
    if cfg.T > 64:
        edges = tile_edge_tokens(cfg)[0]
        tokens = np.array(sorted(set(sample_tokens(cfg.T, 24, cfg.seed).tolist()) | edges))
        log(f"  {len(tokens)} sampled tokens, {len(edges)} of them at m-tile edges")
    ref = oracle_forward(cfg, tokens=tokens)
    y, out = run_forward(cfg)
    routing = check_forward(cfg, ref, y, out, tokens=tokens)
    if cfg is C.SWITCH_SKEWED:
        counts = H.to_host(out["counts"])
        log(f"  loads {counts.tolist()} capacity {H.capacity_of(cfg)} "
            f"dropped {int(H.to_host(out['drop']).sum())}")
    assert routing["near"] <= cfg.T // 100


@pytest.mark.timeout(1200)
def test_full_size_latent():
    cfg = C.LATENT
    log(f"[full] {cfg.name}: uploading {cfg.N} experts")
    # Six random tokens, plus the m-tile edges of the expert holding the most
    # rows (two 192-row tiles, the second ragged) and of the one holding the
    # fewest (a single ragged tile).
    r = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    L = np.bincount(r["idx"].reshape(-1), minlength=cfg.N)
    edges, _ = tile_edge_tokens(cfg, experts=[int(L.argmax()), int(L.argmin())], tiles=(192,))
    tokens = np.array(sorted(set(sample_tokens(cfg.T, 6, cfg.seed).tolist()) | edges))
    log(f"  {len(tokens)} sampled tokens, {len(edges)} at m-tile edges (loads {L.max()}, {L.min()})")
    ref = oracle_forward(cfg, tokens=tokens)
    y, out = run_forward(cfg)
    check_forward(cfg, ref, y, out, tokens=tokens)
