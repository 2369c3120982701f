"""Pins of the fp64 oracle against facts fixed outside the oracle itself:
values the pages print for worked examples, closed forms, library routines
for special cases, invariants, and brute force on tiny inputs.

Each test names the passage it follows.  Page 3 is "MoE: how sparse
activation saves compute"; page 5 is "Stable LatentMoE interactive demo".
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth
from synth import configs as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def tiny_experts(cfg):
    return lambda e: cfg.expert(e)


# ---------------------------------------------------------------------------
# Capacity and drops (page 3, §01, §3.5 eq. C, §3.8, §09 ex. 2-3, appendix)
# ---------------------------------------------------------------------------


def test_capacity_example_uneven_and_even():
    g = gold("capacity_example.json")
    T, N = g["T"], g["N"]
    uneven = np.array(g["uneven_assignment"])[:, None]
    even = (np.arange(T) % N)[:, None]
    for i, c in enumerate(g["factors"]):
        cap = O.capacity_from_factor(T, N, 1, c)
        assert cap == g["capacity"][i]
        d = O.dispatch(uneven, N, cap)
        assert d["counts"].tolist() == g["uneven_loads"]
        assert d["overflow"] == g["uneven_dropped"][i]
        assert int(d["drop"].sum()) == g["uneven_dropped"][i]
        assert d["empty_slots"] == g["uneven_empty_slots"][i]
        assert d["static_slots"] == g["static_slots"][i]
        de = O.dispatch(even, N, cap)
        assert de["overflow"] == g["even_dropped"][i] == int(de["drop"].sum())


def test_capacity_counts_dispatches_for_topk():
    # §3.5 second paragraph: with k slots per token, capacity is sized on k*T.
    assert O.capacity_from_factor(16, 4, 2, 1.0) == 8
    assert O.capacity_from_factor(16384, 8, 1, 1.25) == 2560


def test_token_order_drops_first_c_kept():
    # Reading: the first C tokens reaching an expert are kept.
    idx = np.array(C.PLANTED_ASSIGNMENT)[:, None]
    d = O.dispatch(idx, 4, 4)
    dropped_tokens = np.nonzero(d["drop"])[0].tolist()
    assert dropped_tokens == [4, 5, 6, 7, 8, 9]
    d6 = O.dispatch(idx, 4, 6)
    assert np.nonzero(d6["drop"])[0].tolist() == [6, 7, 8, 9]


# ---------------------------------------------------------------------------
# Balance statistics (page 3, §3.4 eqs. f, P, L_aux; §04 printed values)
# ---------------------------------------------------------------------------


def test_aux_balanced_and_collapsed():
    g = gold("aux_example.json")
    T, N, v = g["T"], g["N"], g["logit_value"]
    bal = np.zeros((T, N))
    bal[np.arange(T), np.arange(T) % N] = v
    col = np.zeros((T, N))
    col[:, 0] = v
    sb = O.balance_stats(O.softmax(bal), alpha=0.01)
    assert np.allclose(sb["f"], g["balanced"]["f"], atol=0)
    assert np.allclose(sb["P"], g["balanced"]["P"], atol=1e-15)
    assert round(sb["n_sum_fP"], 4) == g["balanced"]["n_sum_fP"]
    sc = O.balance_stats(O.softmax(col), alpha=0.01)
    assert sc["f"].tolist() == g["collapsed"]["f"]
    assert [round(x, 4) for x in sc["P"]] == g["collapsed"]["P_4dp"]
    assert round(sc["n_sum_fP"], 4) == g["collapsed"]["n_sum_fP_4dp"]
    # Closed forms: P_0 = e^2/(e^2+3), the others 1/(e^2+3); N sum f P = 4 P_0.
    e2 = math.exp(2.0)
    assert abs(sc["P"][0] - e2 / (e2 + 3)) < 1e-15
    assert abs(sc["P"][1] - 1 / (e2 + 3)) < 1e-15
    assert abs(sc["n_sum_fP"] - 4 * e2 / (e2 + 3)) < 1e-14
    assert abs(sc["aux"] - 0.01 * sc["n_sum_fP"]) < 1e-16


def test_f_is_argmax_before_capacity():
    # f counts argmax choices, independent of how many were dropped.
    idx = np.array(C.PLANTED_ASSIGNMENT)
    p = np.full((16, 4), 0.1)
    p[np.arange(16), idx] = 0.7
    s = O.balance_stats(p, 0.01)
    assert (s["f"] * 16).tolist() == [10, 3, 2, 1]


# ---------------------------------------------------------------------------
# Parameter ledger (page 3, §01 and §3.3)
# ---------------------------------------------------------------------------


def test_param_ledger_matches_page():
    g = gold("ledger_example.json")
    L = O.param_ledger(g["N"], g["k"], g["d"], g["h"])
    assert L["one"] == g["one"] and L["all"] == g["all"] and L["active"] == g["active"]
    assert L["all"] / L["active"] == g["ratio"] == g["N"] / g["k"]
    assert round(L["all"] * 2 / 2**30, 3) == g["bf16_gib_3dp"]


def test_forward_touches_only_k_experts_per_token():
    # The forward evaluates exactly the k selected experts of a token, i.e.
    # k*3dh expert parameters out of N*3dh (active/total = k/N).
    cfg = C.TINY
    seen = []

    def experts(e):
        seen.append(e)
        return cfg.expert(e)

    u = cfg.u()[:1]
    out = O.forward(u, cfg.w_route(), experts, k=cfg.k)
    assert sorted(seen) == sorted(out["idx"][0].tolist())
    L = O.param_ledger(cfg.N, cfg.k, cfg.d, cfg.h)
    touched = sum(sum(w.size for w in cfg.expert(e)) for e in seen)
    assert touched == L["active"] and L["all"] // L["active"] == cfg.N // cfg.k


# ---------------------------------------------------------------------------
# Routing worked example (page 3, §3.6 and §04: seed 7 -> loads [8,7,8,9])
# ---------------------------------------------------------------------------


def test_seed7_routing_loads():
    g = gold("routing_seed7.json")
    torch.manual_seed(g["seed"])
    x = torch.randn(g["T"], g["d"])
    gate = torch.nn.Linear(g["d"], g["N"], bias=False)
    r = O.route(x.double().numpy(), gate.weight.detach().double().numpy(), g["k"], "renorm")
    assert list(r["idx"].shape) == g["idx_shape"]
    loads = np.bincount(r["idx"].reshape(-1), minlength=g["N"]).tolist()
    assert loads == g["loads"] and sum(loads) == g["T"] * g["k"]
    # The fp32 selection of the page's code agrees (margins are large).
    probs = F.softmax(gate(x).float(), dim=-1)
    _, ti = probs.topk(g["k"], dim=-1)
    assert np.array_equal(ti.numpy(), r["idx"])


# ---------------------------------------------------------------------------
# Softmax, top-k and gate weights against torch (page 3, §3.2)
# ---------------------------------------------------------------------------


def test_softmax_topk_against_torch():
    rng = np.random.default_rng(0)
    z = rng.normal(size=(200, 8)) * 3
    p = O.softmax(z)
    assert np.allclose(p, torch.softmax(torch.from_numpy(z), dim=1).numpy(), atol=1e-15, rtol=0)
    for k in (1, 2, 3, 8):
        idx = O.select_topk(p, k)
        tv, ti = torch.topk(torch.from_numpy(p), k, dim=1)
        assert np.array_equal(idx, ti.numpy())
        a = O.gate_weights(p, idx, "renorm")
        assert np.allclose(a.sum(1), 1.0, atol=1e-15)
        assert np.allclose(a, (tv / tv.sum(1, keepdim=True)).numpy(), atol=1e-15)
        assert np.allclose(O.gate_weights(p, idx, "prob"), tv.numpy(), atol=0)
    # k = 1 renormalised weight is exactly 1; the Switch weight is max p.
    idx1 = O.select_topk(p, 1)
    assert np.all(O.gate_weights(p, idx1, "renorm") == 1.0)
    assert np.allclose(O.gate_weights(p, idx1, "prob")[:, 0], p.max(1), atol=0)


def test_topk_ties_go_to_lower_index_and_margin():
    z = np.array([[1.0, 2.0, 2.0, 0.5], [3.0, 3.0, 3.0, 3.0]])
    p = O.softmax(z)
    assert O.select_topk(p, 2).tolist() == [[1, 2], [0, 1]]
    m = O.topk_margin(z, 2)
    assert m[0] == 1.0 and m[1] == 0.0
    assert np.isinf(O.topk_margin(z, 4)).all()


def test_router_logits_orientation():
    # z = W_route u with W_route [N, d]: the same as torch's F.linear.
    rng = np.random.default_rng(1)
    u = rng.normal(size=(5, 7))
    w = rng.normal(size=(3, 7))
    ref = F.linear(torch.from_numpy(u), torch.from_numpy(w)).numpy()
    assert np.allclose(O.router_logits(u, w), ref, atol=1e-14)


# ---------------------------------------------------------------------------
# Dispatch (page 3, §3.6 and the appendix's torch.where grouping)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("T,N,k,cap", [(64, 4, 2, None), (300, 8, 2, 40), (100, 16, 4, 20),
                                       (50, 8, 1, 3)])
def test_dispatch_matches_torch_where_order(T, N, k, cap):
    rng = np.random.default_rng(T + N)
    idx = np.stack([rng.permutation(N)[:k] for _ in range(T)])
    d = O.dispatch(idx, N, cap)
    assert int(d["counts"].sum()) == k * T            # sum_i L_i = kT (§3.6)
    ti = torch.from_numpy(idx)
    for e in range(N):
        tok, slot = torch.where(ti == e)
        seg = d["perm"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.array_equal(seg // k, tok.numpy())
        assert np.array_equal(seg % k, slot.numpy())
        kept = min(len(seg), cap) if cap is not None else len(seg)
        assert np.array_equal(d["row_of"][seg[:kept]],
                              d["kept_offsets"][e] + np.arange(kept))
        assert np.all(d["row_of"][seg[kept:]] == -1)
        assert np.all(d["drop"][seg[kept:]] == 1) and np.all(d["drop"][seg[:kept]] == 0)
    if cap is not None:
        assert d["overflow"] == int(np.maximum(d["counts"] - cap, 0).sum()) == int(d["drop"].sum())


# ---------------------------------------------------------------------------
# Expert and full layer (page 3, §3.1, §3.2; appendix dense reference)
# ---------------------------------------------------------------------------


def test_single_expert_is_torch_swiglu():
    # N = 1, k = 1, renorm: the layer is one SwiGLU FFN.  Non-square shapes so
    # a transposed operand cannot pass.
    rng = np.random.default_rng(2)
    T, d, h = 9, 12, 20
    u = rng.normal(size=(T, d))
    wg, wu = rng.normal(size=(h, d)) / 3, rng.normal(size=(h, d)) / 3
    wd = rng.normal(size=(d, h)) / 4
    out = O.forward(u, np.ones((1, d)), lambda e: (wg, wu, wd), k=1)
    tu = torch.from_numpy(u)
    ref = F.linear(F.silu(F.linear(tu, torch.from_numpy(wg))) * F.linear(tu, torch.from_numpy(wu)),
                   torch.from_numpy(wd)).numpy()
    assert np.allclose(out["y"], ref, atol=1e-13, rtol=0)
    assert out["y"].shape == (T, d)                   # output width d (§3.6)


def test_silu_against_torch():
    x = np.linspace(-50, 50, 1001)
    assert np.allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), atol=1e-15, rtol=1e-15)


@pytest.mark.parametrize("cfg", [C.TINY, C.TINY.with_(k=1, gate="prob"),
                                 C.TINY.with_(capacity_factor=0.6),
                                 C.TINY_PLANTED, C.TINY_PLANTED.with_(capacity_factor=1.5)])
def test_sparse_equals_dense_brute_force(cfg):
    cap = (None if cfg.capacity_factor is None
           else O.capacity_from_factor(cfg.T, cfg.N, cfg.k, cfg.capacity_factor))
    u, wr = cfg.u(), cfg.w_route()
    sp = O.forward(u, wr, tiny_experts(cfg), k=cfg.k, gate=cfg.gate, capacity=cap)
    de = O.forward_dense(u, wr, tiny_experts(cfg), k=cfg.k, gate=cfg.gate, capacity=cap)
    assert O.relative_error(sp["y"], de) <= 1e-13


def test_k_equals_n_is_probability_weighted_dense_sum():
    cfg = C.TINY.with_(k=4)
    u, wr = cfg.u(), cfg.w_route()
    out = O.forward(u, wr, tiny_experts(cfg), k=4)
    p = O.softmax(O.expand(u) @ O.expand(wr).T)
    ref = sum(p[:, [e]] * O.expert_forward(O.expand(u), *(O.expand(w) for w in cfg.expert(e)),
                                           O.swiglu) for e in range(4))
    assert O.relative_error(out["y"], ref) < 1e-13


def test_planted_variant_end_to_end():
    cfg = C.TINY_PLANTED
    u, wr = cfg.u(), cfg.w_route()
    for c, drops in ((1.0, 6), (1.5, 4), (2.5, 0)):
        cap = O.capacity_from_factor(cfg.T, cfg.N, 1, c)
        out = O.forward(u, wr, tiny_experts(cfg), k=1, gate="prob", capacity=cap)
        assert out["idx"][:, 0].tolist() == C.PLANTED_ASSIGNMENT
        assert out["disp"]["counts"].tolist() == [10, 3, 2, 1]
        assert int(out["disp"]["drop"].sum()) == drops
        dropped = np.nonzero(out["disp"]["drop"])[0]
        assert np.all(out["y"][dropped] == 0.0)          # overflow skips the layer
        assert out["margin"].min() > 7.0


def test_unselected_expert_perturbation_leaves_y_identical():
    cfg = C.TINY
    u, wr = cfg.u(), cfg.w_route()
    base = O.forward(u, wr, tiny_experts(cfg), k=2)
    used = set(base["idx"].reshape(-1).tolist())
    unused = [e for e in range(cfg.N) if e not in used]
    # Route a single token so that some expert is certainly unselected.
    u1 = u[:1]
    b1 = O.forward(u1, wr, tiny_experts(cfg), k=2)
    off = [e for e in range(cfg.N) if e not in b1["idx"][0]]
    assert off

    def big(e):
        g, up, dn = cfg.expert(e)
        if e in off:
            return g * 1e3, up * 1e3, dn * 1e3
        return g, up, dn

    p1 = O.forward(u1, wr, big, k=2)
    assert np.array_equal(p1["y"], b1["y"])
    del unused


# ---------------------------------------------------------------------------
# LatentMoE pieces (page 5: width separation, RMSNorm, SiTU-GLU)
# ---------------------------------------------------------------------------


def test_rmsnorm_against_torch():
    rng = np.random.default_rng(3)
    r = rng.normal(size=(6, 33)) * 5
    ref = F.rms_norm(torch.from_numpy(r), (33,), eps=1e-6).numpy()
    assert np.allclose(O.rmsnorm(r, 1e-6), ref, atol=1e-14, rtol=0)


def test_situ_glu_limits_and_bound():
    rng = np.random.default_rng(4)
    g, v = rng.normal(size=1000) * 3, rng.normal(size=1000) * 3
    assert np.allclose(O.situ_glu(g, v, 1e9, 1e9), O.swiglu(g, v), rtol=1e-12, atol=1e-15)
    big = np.concatenate([np.linspace(-1e6, 1e6, 2001), [np.inf, -np.inf]])
    G, V = np.meshgrid(big, big)
    a = O.situ_glu(G, V, 4.0, 25.0)
    assert np.all(np.abs(a) <= 100.0)                 # beta_g * beta_u bound
    assert np.abs(a).max() <= O.silu(np.array(4.0)) * 25.0 + 1e-12
    # Small arguments: the caps are near-identity (tanh(x/b)*b ~ x).
    s = np.array([1e-3, -2e-3])
    assert np.allclose(O.situ_glu(s, s, 4.0, 25.0), O.swiglu(s, s), rtol=1e-6)


SMALL_LATENT = C.LATENT.with_(name="latent_small", T=40, d=32, l=16, h=24, N=8, k=2,
                              n_shared=2, h_shared=24, w_dtype="f32", act_dtype="f32",
                              router_dtype="f32")


def _latent(cfg, **kw):
    return O.latent_forward(cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), cfg.w_ldown(),
                            cfg.w_lup(), lambda j: cfg.shared(j), cfg.n_shared, k=cfg.k,
                            act=cfg.act, rms_eps=cfg.rms_eps, **kw)


def test_latent_identity_projections_reduce_to_rmsnorm_of_plain():
    cfg = C.TINY.with_(act="swiglu")
    u, wr = cfg.u(), cfg.w_route()
    plain = O.forward(u, wr, tiny_experts(cfg), k=cfg.k)["y"]
    eye = np.eye(cfg.d)
    lat = O.latent_forward(u, wr, tiny_experts(cfg), eye, eye, None, 0, k=cfg.k,
                           act="swiglu", rms_eps=1e-6)["y"]
    ref = F.rms_norm(torch.from_numpy(plain), (cfg.d,), eps=1e-6).numpy()
    assert np.allclose(lat, ref, atol=1e-13)


def test_latent_sparse_equals_dense_and_scale_invariance():
    cfg = SMALL_LATENT
    out = _latent(cfg)
    # Dense brute force of the routed branch at width l.
    u = O.expand(cfg.u())
    xl = u @ O.expand(cfg.w_ldown()).T
    r = out
    rsum = np.zeros((cfg.T, cfg.l))
    act = O.make_act("situ")
    for e in range(cfg.N):
        w = np.zeros(cfg.T)
        for s in range(cfg.k):
            w += (r["idx"][:, s] == e) * r["a"][:, s]
        rsum += w[:, None] * O.expert_forward(xl, *(O.expand(x) for x in cfg.expert(e)), act)
    assert O.relative_error(out["r"], rsum) < 1e-13
    # Scaling every routed expert's down matrix leaves y unchanged (RMSNorm);
    # the scale is taken in fp64 after expansion so the stored values stay exact.
    def scaled_expert(e):
        g, up, dn = cfg.expert(e)
        return g, up, O.expand(dn) * 7.0

    kw = dict(k=cfg.k, act="situ", rms_eps=0.0)
    scaled = O.latent_forward(cfg.u(), cfg.w_route(), scaled_expert, cfg.w_ldown(), cfg.w_lup(),
                              lambda j: cfg.shared(j), cfg.n_shared, **kw)
    base0 = O.latent_forward(cfg.u(), cfg.w_route(), lambda e: cfg.expert(e), cfg.w_ldown(),
                             cfg.w_lup(), lambda j: cfg.shared(j), cfg.n_shared, **kw)
    assert O.relative_error(scaled["y"], base0["y"]) < 1e-13


def test_latent_shared_experts_are_torch_swiglu():
    # Zero routed down matrices: the routed branch is RMSNorm(0) = 0 and y is
    # the sum of the shared SwiGLU experts.
    cfg = SMALL_LATENT
    out = O.latent_forward(cfg.u(), cfg.w_route(),
                           lambda e: (cfg.expert(e)[0], cfg.expert(e)[1], 0 * cfg.expert(e)[2]),
                           cfg.w_ldown(), cfg.w_lup(), lambda j: cfg.shared(j), cfg.n_shared,
                           k=cfg.k, act="situ", rms_eps=1e-6)
    tu = torch.from_numpy(O.expand(cfg.u()))
    ref = 0
    for j in range(cfg.n_shared):
        g, up, dn = (torch.from_numpy(O.expand(w)) for w in cfg.shared(j))
        ref = ref + F.linear(F.silu(F.linear(tu, g)) * F.linear(tu, up), dn)
    assert np.allclose(out["y"], ref.numpy(), atol=1e-13)


def test_latent_parameter_saving_closed_form():
    g = gold("latent_saving.json")
    s = O.latent_param_saving(g["d"], g["l"], g["H"], g["E"])
    assert abs(s - g["saving_approx"]) < g["tolerance"]


# ---------------------------------------------------------------------------
# Stored-value expansion and bf16 rounding (page 2, §六: the fp16 subnormal
# lesson -- every hand-written conversion is tested on its special cases)
# ---------------------------------------------------------------------------


def test_expand_bf16_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.expand(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _bf16_value(b):
    return float(O.expand(np.array([b], dtype=np.uint16))[0])


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.normal(size=3000) * 10.0 ** rng.integers(-45, 39, 3000),
                         [0.0, -0.0, 1e-45, 9.2e-41, 1.1754942e-38, 1.1754944e-38,
                          3.3895e38, 3.3896e38, 3.4e38, 1e300, -1e-300]])
    grid = O.expand(np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16))  # +0 .. +Inf
    grid[0x7F80] = 2.0 ** 128   # IEEE: overflow is decided as if the exponent were unbounded
    for x in xs:
        b = synth.f64_to_bf16_bits(x)
        ax = abs(x)
        j = np.searchsorted(grid, ax)
        cands = [c for c in (j - 1, j) if 0 <= c < grid.size]
        best = min(cands, key=lambda c: (abs(grid[c] - ax), c & 1))
        expect = best | (0x8000 if math.copysign(1.0, x) < 0 else 0)
        assert b == expect, (x, hex(b), hex(expect))
    assert synth.f64_to_bf16_bits(float("inf")) == 0x7F80
    assert synth.f64_to_bf16_bits(float("-inf")) == 0xFF80
    assert math.isnan(_bf16_value(synth.f64_to_bf16_bits(float("nan"))))
    # Exact ties: 1 + 2^-8 lies between 1 and 1 + 2^-7, goes to even (1.0).
    assert synth.f64_to_bf16_bits(1.0 + 2 ** -8) == 0x3F80
    assert synth.f64_to_bf16_bits(1.0 + 3 * 2 ** -8) == 0x3F82
    # Smallest subnormal and its half (tie to even -> 0).
    assert synth.f64_to_bf16_bits(2.0 ** -133) == 0x0001
    assert synth.f64_to_bf16_bits(2.0 ** -134) == 0x0000
    assert synth.f64_to_bf16_bits(3 * 2.0 ** -134) == 0x0002


def test_round_matches_torch_on_fp32_exact_values():
    # For values that are exact fp32 numbers torch's fp32->bf16 conversion is a
    # single rounding, so it must agree with the direct rounding.
    rng = np.random.default_rng(6)
    x = rng.normal(size=100000).astype(np.float32).astype(np.float64)
    ours = synth.round_to(x, "bf16")
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours.view(np.int16), ref)


def test_combine_rows_and_expert_rows_rebuild_forward():
    # The staged oracle (expert rows, then combine) equals the one-pass forward,
    # with and without capacity.
    for cfg in (C.TINY, C.TINY_PLANTED):
        cap = (None if cfg.capacity_factor is None
               else O.capacity_from_factor(cfg.T, cfg.N, cfg.k, cfg.capacity_factor))
        u, wr = cfg.u(), cfg.w_route()
        out = O.forward(u, wr, tiny_experts(cfg), k=cfg.k, gate=cfg.gate, capacity=cap)
        d = out["disp"]
        rows = O.expert_rows(O.expand(u), d, tiny_experts(cfg), O.swiglu, cfg.k)
        R = int(d["kept_offsets"][-1])
        assert sorted(rows) == list(range(R))
        y_rows = np.stack([rows[r] for r in range(R)])
        y = O.combine_rows(y_rows, d["row_of"], out["a"])
        assert O.relative_error(y, out["y"]) < 1e-14


# ---------------------------------------------------------------------------
# Quantile Balancing (page "Stable LatentMoE interactive demo", QB passage):
# with the cutoffs a_t fixed, b'_j is the q-th smallest required_tj.
# ---------------------------------------------------------------------------


def _qb_logits(seed, T, N, hot=()):
    rng = np.random.default_rng(seed)
    u = rng.normal(size=(T, 64))
    w = rng.normal(size=(N, 64)) / 8.0
    for j in hot:
        w[j] *= 6.0
    return u @ w.T


def test_qb_hand_example():
    # k = 1, T = 4, N = 2, b = 0: a_t = max_j z_tj = [2, 1, 1, 3];
    # required columns: expert 0 [0, 0, 1, 0], expert 1 [2, 0.6, 0, 4];
    # q = round(1 * 4 / 2) = 2, so b' = [0, 0.6] (second smallest of each).
    z = np.array([[2.0, 0.0], [1.0, 0.4], [0.0, 1.0], [3.0, -1.0]])
    b0 = np.zeros(2)
    assert O.qb_target(4, 2, 1) == 2
    assert np.allclose(O.qb_cutoff(z, b0, 1), [2.0, 1.0, 1.0, 3.0])
    assert np.allclose(O.qb_required(z, b0, 1), [[0, 2], [0, 0.6], [1, 0], [0, 4]])
    assert np.allclose(O.qb_bias_exact(z, b0, 1, 2), [0.0, 0.6])


def test_qb_exact_is_the_q_th_order_statistic():
    # Fewer than q tokens need strictly less bias than b'_j, at least q need at
    # most b'_j: the defining property of the q-th smallest required value.
    for seed, (T, N, k) in enumerate(((200, 8, 2), (333, 24, 3), (64, 5, 1))):
        z = _qb_logits(seed, T, N)
        b = np.random.default_rng(seed + 50).normal(size=N) * 0.3
        q = O.qb_target(T, N, k)
        bx = O.qb_bias_exact(z, b, k, q)
        req = O.qb_required(z, b, k)
        assert np.all((req < bx[None, :]).sum(axis=0) < q)
        assert np.all((req <= bx[None, :]).sum(axis=0) >= q)


def test_qb_shift_of_the_bias_shifts_the_update():
    # Adding c to every b_j leaves the selection alone and raises every cutoff
    # by c, so every required value and the update shift by c.
    z = _qb_logits(3, 300, 12)
    b = np.random.default_rng(4).normal(size=12) * 0.2
    q = O.qb_target(300, 12, 2)
    for c in (0.75, -3.0):
        assert np.allclose(O.qb_bias_exact(z, b + c, 2, q), O.qb_bias_exact(z, b, 2, q) + c,
                           atol=1e-12)
        assert np.allclose(O.qb_bias_histogram(z, b + c, 2, q),
                           O.qb_bias_histogram(z, b, 2, q) + c, atol=1e-9)


def test_qb_histogram_within_one_bin_of_exact():
    for seed, (T, N, k) in enumerate(((500, 16, 2), (2000, 8, 1), (100, 40, 4))):
        z = _qb_logits(seed + 10, T, N)
        b = np.zeros(N)
        q = O.qb_target(T, N, k)
        req = O.qb_required(z, b, k)
        width = (req.max(axis=0) - req.min(axis=0)) / 256
        err = np.abs(O.qb_bias_histogram(z, b, k, q) - O.qb_bias_exact(z, b, k, q))
        assert np.all(err <= width * (1 + 1e-9))


def test_qb_zero_bias_is_plain_routing():
    rng = np.random.default_rng(8)
    u = rng.normal(size=(50, 32))
    w = rng.normal(size=(10, 32))
    r0 = O.route(u, w, 3, "renorm")
    rb = O.route(u, w, 3, "renorm", bias=np.zeros(10))
    assert np.array_equal(r0["idx"], rb["idx"])
    assert np.allclose(r0["a"], rb["a"], atol=0)


def test_qb_bias_moves_selection_but_not_weights_source():
    # A large bias on one expert makes every token select it, and its weight is
    # still the renormalised unbiased probability.
    rng = np.random.default_rng(9)
    u = rng.normal(size=(30, 16))
    w = rng.normal(size=(6, 16))
    b = np.zeros(6)
    b[4] = 1e3
    r = O.route(u, w, 2, "renorm", bias=b)
    assert np.all(r["idx"][:, 0] == 4)
    p = O.softmax(O.router_logits(u, w))
    ps = np.take_along_axis(p, r["idx"], axis=1)
    assert np.allclose(r["a"], ps / ps.sum(axis=1, keepdims=True), rtol=1e-14)


def test_qb_update_cools_hot_experts():
    # Two experts with 6x router rows take far more than their share; a few
    # Quantile Balancing steps (each recomputing the cutoffs) bring the
    # busiest expert much closer to the target load.
    T, N, k = 4000, 16, 2
    z = _qb_logits(12, T, N, hot=(0, 1))
    q = O.qb_target(T, N, k)
    b = np.zeros(N)
    before = O.qb_loads(z, b, k).max()
    for _ in range(3):
        b = O.qb_bias_exact(z, b, k, q)
    after = O.qb_loads(z, b, k).max()
    assert before > 3 * q
    assert after < 1.5 * q


# ---------------------------------------------------------------------------
# FP8 E4M3 expert weights (page 5, SiTU-GLU passage: E4M3's largest value is
# 448).  The format itself is OCP FP8 E4M3.
# ---------------------------------------------------------------------------


def test_e4m3_decode_matches_torch():
    # torch's float8_e4m3fn is an independent implementation of the format.
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    ref = ref.numpy()
    mine = O.E4M3_TABLE
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_landmarks():
    v = O.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0       # largest finite (page 5)
    assert v(0x38) == 1.0 and v(0xB8) == -1.0
    assert v(0x01) == 2.0 ** -9                          # smallest subnormal
    assert v(0x08) == 2.0 ** -6                          # smallest normal
    assert v(0x07) == 7 * 2.0 ** -9                      # largest subnormal
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert np.isfinite(O.E4M3_TABLE).sum() == 254
    pos = O.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..0x7E increase


def test_fp8_rows_expand_by_hand():
    m = synth.Fp8Rows(np.array([[0x38, 0x40, 0x3C], [0xB8, 0x00, 0x01]], dtype=np.uint8),
                      np.array([2.0, 0.5], dtype=np.float32))
    # 0x40 = 2^(8-7) = 2, 0x3C = 1.5, 0x01 = 2^-9; each row times its own scale
    want = np.array([[2.0, 4.0, 3.0], [-0.5, 0.0, 2.0 ** -10]])
    assert np.array_equal(O.expand(m), want)


def test_synth_e4m3_encoder_matches_torch():
    # The generator's nearest-even rounding against torch's cast, on values
    # exact in fp32 (so torch's float -> fp8 path rounds them once): random
    # magnitudes over the whole range, subnormals, exact ties and saturation.
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(4000) * 40.0,
        rng.uniform(-2 ** -6, 2 ** -6, 1000),
        (O.E4M3_TABLE[1:0x7E] + O.E4M3_TABLE[2:0x7F]) / 2,   # midpoints
        -(O.E4M3_TABLE[1:0x7E] + O.E4M3_TABLE[2:0x7F]) / 2,
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11],
    ]).astype(np.float32).astype(np.float64)
    mine = np.array([synth.f64_to_e4m3(v) for v in x], dtype=np.uint8)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(mine, ref.numpy())
    assert synth.f64_to_e4m3(1000.0) == 0x7E and synth.f64_to_e4m3(-500.0) == 0xFE


def test_synth_fp8_rows_follow_the_bf16_draws():
    rows, cols, std = 6, 256, 0.05
    q = synth.normal_fp8_rows(3, synth.TID_W_GATE, rows, cols, std, start=512)
    v = synth.normal_f64(3, synth.TID_W_GATE, rows * cols, std, start=512).reshape(rows, cols)
    assert np.allclose(q.scale, np.abs(v).max(axis=1) / 448.0, rtol=1e-7, atol=0)
    w = O.expand(q)
    # E4M3 keeps 3 mantissa bits: relative rounding error <= 2^-4 above the
    # subnormal range, absolute <= 2^-10 * scale below it.
    err = np.abs(w - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, q.scale[:, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.array_equal(np.abs(w).max(axis=1), q.scale.astype(np.float64) * 448.0)


# ---------------------------------------------------------------------------
# MXFP4 expert weights (page "Kestrel-MCU notes #13", section 二: 4-bit
# experts).  The format is OCP MX FP4: E2M1 elements, one E8M0 scale per 32.
# ---------------------------------------------------------------------------


def test_e8m0_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    ref = ref.numpy()
    assert np.array_equal(np.isnan(O.E8M0_TABLE), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(O.E8M0_TABLE[ok], ref[ok])
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(0) == 2.0 ** -127


def test_e2m1_is_the_e4m3_subset():
    # An E2M1 value with exponent field e > 0 and mantissa bit m is the E4M3
    # value with exponent field e + 6 (bias 1 -> 7) and mantissa bits m << 2;
    # the subnormal 0.5 is E4M3 0x30.  torch decodes the E4M3 side.
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(16):
        sign, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        if e == 0:
            code8 = (sign << 7) | (0x30 if m else 0x00)
        else:
            code8 = (sign << 7) | ((e + 6) << 3) | (m << 2)
        assert O.e2m1_value(c) == e4[code8], c
    assert sorted(set(abs(v) for v in O.E2M1_TABLE)) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_mxfp4_expand_by_hand():
    # One row of 64: block 0 scale 2^0, block 1 scale 2^-3.  Byte 0 = 0x72:
    # element 0 = code 2 (1.0), element 1 = code 7 (6.0).
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x72
    packed[0, 16] = 0x9B      # elements 32, 33: code 0xB (-1.5), code 0x9 (-0.5)
    m = synth.MxFp4Rows(packed, np.array([[127, 124]], dtype=np.uint8))
    w = O.expand(m)
    want = np.zeros((1, 64))
    want[0, 0], want[0, 1] = 1.0, 6.0
    want[0, 32], want[0, 33] = -1.5 / 8, -0.5 / 8
    assert np.array_equal(w, want)


def test_synth_e2m1_encoder_brute_force():
    # Nearest E2M1 value by exhaustive search, ties to the even code.
    vals = [O.e2m1_value(c) for c in range(8)]
    rng = np.random.default_rng(9)
    xs = list(rng.uniform(-7, 7, 3000)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 6.0, 9.0]
    for x in xs:
        a = min(abs(x), 6.0)
        best = min(range(8), key=lambda c: (abs(a - vals[c]), c & 1))
        want = best | (8 if x < 0 else 0)
        assert synth.f64_to_e2m1(x) == want, x


def test_synth_mxfp4_rows_follow_the_bf16_draws():
    rows, cols, std = 5, 128, 0.05
    q = synth.normal_mxfp4_rows(3, synth.TID_W_UP, rows, cols, std, start=256)
    v = synth.normal_f64(3, synth.TID_W_UP, rows * cols, std, start=256).reshape(rows, cols)
    blk = v.reshape(rows, cols // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    assert np.array_equal(q.block_scale.astype(int) - 127, np.floor(np.log2(amax)).astype(int) - 2)
    w = O.expand(q).reshape(rows, cols // 32, 32)
    # Elements of [0.5, 4) times the block scale keep 1 mantissa bit: error
    # <= a quarter of the value's binade step; the top binade saturates at 6.
    sc = 2.0 ** (q.block_scale.astype(int) - 127)
    assert np.all(np.abs(w - blk) <= np.maximum(np.abs(blk) / 4, 0.25 * sc[..., None]) + 1e-15)


# ---------------------------------------------------------------------------
# Router backward (page 3, §3.2 eqs. z, p, a, y and §3.4 eq. L_aux,
# differentiated with the selection, the expert outputs and f held fixed)
# ---------------------------------------------------------------------------


def _rb_case(seed, T=24, d=16, N=6, k=2, gate="renorm", cap=None):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    w = rng.standard_normal((N, d)) / math.sqrt(d)
    r = O.route(u, w, k, gate)
    disp = O.dispatch(r["idx"], N, cap)
    R = int(disp["kept_offsets"][-1])
    y_rows = rng.standard_normal((max(R, 1), d))
    dy = rng.standard_normal((T, d))
    f = O.balance_stats(r["p"], 0.01)["f"]
    return u, w, r, disp, y_rows, dy, f


def _rb_loss(u, w, idx, row_of, y_rows, dy, gate, f, alpha, aux_scale):
    # The forward loss with the selection held at idx: <dy, y> + aux_scale L_aux.
    p = O.softmax(O.router_logits(u, w))
    a = O.gate_weights(p, idx, gate)
    y = O.combine_rows(y_rows, row_of, a)
    N = w.shape[0]
    return float(np.sum(dy * y)) + aux_scale * alpha * N * float(np.sum(f * p.mean(axis=0)))


@pytest.mark.parametrize("gate,cap", [("renorm", None), ("prob", None), ("renorm", 6)])
def test_route_backward_matches_torch_autograd(gate, cap):
    u, w, r, disp, y_rows, dy, f = _rb_case(3, gate=gate, cap=cap)
    k = r["idx"].shape[1]
    alpha, lam = 0.01, 3.0
    g = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, dy, gate=gate, f=f,
                         alpha=alpha, aux_scale=lam)
    # An independent torch forward; autograd differentiates it.
    ut = torch.tensor(u, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    pt = torch.softmax(ut @ wt.T, dim=1)
    it = torch.tensor(r["idx"])
    ps = torch.gather(pt, 1, it)
    at = ps / ps.sum(dim=1, keepdim=True) if gate == "renorm" else ps
    rows = torch.tensor(disp["row_of"].reshape(-1, k))
    F = torch.tensor(y_rows)[rows.clamp(min=0)] * (rows >= 0).unsqueeze(-1)
    y = (at.unsqueeze(-1) * F).sum(dim=1)
    N = w.shape[0]
    loss = (torch.tensor(dy) * y).sum() + lam * alpha * N * (torch.tensor(f) * pt.mean(0)).sum()
    loss.backward()
    assert np.allclose(g["dW_route"], wt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["du"], ut.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_route_backward_central_differences():
    u, w, r, disp, y_rows, dy, f = _rb_case(4)
    alpha, lam = 0.01, 2.0
    g = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, dy, gate="renorm", f=f,
                         alpha=alpha, aux_scale=lam)
    assert np.all(r["margin"] > 1e-3)   # steps below cannot change the selection
    eps = 1e-6
    for (n, c) in [(0, 0), (2, 5), (5, 15), (3, 7)]:
        wp, wm = w.copy(), w.copy()
        wp[n, c] += eps
        wm[n, c] -= eps
        num = (_rb_loss(u, wp, r["idx"], disp["row_of"], y_rows, dy, "renorm", f, alpha, lam) -
               _rb_loss(u, wm, r["idx"], disp["row_of"], y_rows, dy, "renorm", f, alpha, lam)) / (2 * eps)
        assert abs(num - g["dW_route"][n, c]) <= 1e-6 * max(1.0, abs(num))


def test_route_backward_invariants():
    u, w, r, disp, y_rows, dy, f = _rb_case(5)
    g = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, dy, gate="renorm", f=f,
                         alpha=0.01, aux_scale=1.0)
    # The softmax gradient sums to zero over the experts of each token.
    assert np.allclose(g["dz"].sum(axis=1), 0.0, atol=1e-12)
    # With f perfectly balanced, L_aux = alpha N sum_i P_i / N = alpha is
    # constant, so the aux term contributes no gradient.
    N = w.shape[0]
    zero_dy = np.zeros_like(dy)
    flat = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, zero_dy, gate="renorm",
                            f=np.full(N, 1.0 / N), alpha=0.01, aux_scale=5.0)
    assert np.abs(flat["dz"]).max() < 1e-15
    # ... while an unbalanced f pushes the hot expert's logits down.
    hot = np.zeros(N)
    hot[0] = 1.0
    push = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, zero_dy, gate="renorm",
                            f=hot, alpha=0.01, aux_scale=5.0)
    assert np.all(push["dz"][:, 0] > 0)   # gradient ascent direction: descent lowers z_0


def test_route_backward_renorm_over_all_experts_is_the_prob_gate():
    # With k = N, sum_S p = 1, so renorm and prob weights coincide; their
    # gate gradients differ by a per-token constant that the softmax removes.
    u, w, r, disp, y_rows, dy, f = _rb_case(6, N=4, k=4)
    a = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, dy, gate="renorm", f=f,
                         alpha=0.01, aux_scale=1.0)
    b = O.route_backward(u, w, r["idx"], disp["row_of"], y_rows, dy, gate="prob", f=f,
                         alpha=0.01, aux_scale=1.0)
    assert np.allclose(a["dz"], b["dz"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("act,cap", [("swiglu", None), ("situ", None), ("swiglu", 5)])
def test_experts_backward_matches_torch_autograd(act, cap):
    rng = np.random.default_rng(8)
    T, d, h, N, k = 20, 12, 10, 4, 2
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d)) / math.sqrt(d)
    W = [(rng.standard_normal((h, d)) / math.sqrt(d), rng.standard_normal((h, d)) / math.sqrt(d),
          rng.standard_normal((d, h)) / math.sqrt(h)) for _ in range(N)]
    r = O.route(x, wr, k, "renorm")
    disp = O.dispatch(r["idx"], N, cap)
    dy = rng.standard_normal((T, d))
    bg, bu = 1.5, 2.0   # small caps so the tanh factors matter
    g = O.experts_backward(x, disp, r["a"], lambda e: W[e], dy, act=act, k=k, beta_g=bg, beta_u=bu)
    # Independent torch forward of the expert part (weights a held fixed).
    xt = torch.tensor(x, requires_grad=True)
    Wt = [tuple(torch.tensor(m, requires_grad=True) for m in ws) for ws in W]
    y = torch.zeros((T, d), dtype=torch.float64)
    for t in range(T):
        for s in range(k):
            if disp["row_of"][t * k + s] < 0:
                continue
            wg, wu, wd = Wt[int(r["idx"][t, s])]
            gg, vv = wg @ xt[t], wu @ xt[t]
            if act == "situ":
                gg, vv = bg * torch.tanh(gg / bg), bu * torch.tanh(vv / bu)
            y[t] = y[t] + float(r["a"][t, s]) * (wd @ (torch.nn.functional.silu(gg) * vv))
    (torch.tensor(dy) * y).sum().backward()
    assert np.allclose(g["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for e in range(N):
        assert np.allclose(g["dW_gate"][e], Wt[e][0].grad.numpy() if Wt[e][0].grad is not None
                           else 0.0, rtol=1e-10, atol=1e-12)
        assert np.allclose(g["dW_up"][e], Wt[e][1].grad.numpy() if Wt[e][1].grad is not None
                           else 0.0, rtol=1e-10, atol=1e-12)
        assert np.allclose(g["dW_down"][e], Wt[e][2].grad.numpy() if Wt[e][2].grad is not None
                           else 0.0, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# LatentMoE backward (page 5: the width-separation, RMSNorm and SiTU-GLU
# passages, differentiated; the demo checks that only selected experts
# receive gradient)
# ---------------------------------------------------------------------------


def _latent_case(seed, T=24, d=16, l=12, H=10, N=6, S=2, hs=9):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d)) / math.sqrt(d)
    wld = rng.standard_normal((l, d)) / math.sqrt(d)
    wlu = rng.standard_normal((d, l)) / math.sqrt(l)
    W = [(rng.standard_normal((H, l)) / math.sqrt(l), rng.standard_normal((H, l)) / math.sqrt(l),
          rng.standard_normal((l, H)) / math.sqrt(H)) for _ in range(N)]
    Sw = [(rng.standard_normal((hs, d)) / math.sqrt(d), rng.standard_normal((hs, d)) / math.sqrt(d),
           rng.standard_normal((d, hs)) / math.sqrt(hs)) for _ in range(S)]
    dy = rng.standard_normal((T, d))
    return u, wr, wld, wlu, W, Sw, dy


@pytest.mark.parametrize("cap,aux", [(None, 0.0), (7, 0.7)])
def test_latent_backward_matches_torch_autograd(cap, aux):
    T, d, l, N, k, S = 24, 16, 12, 6, 2, 2
    u, wr, wld, wlu, W, Sw, dy = _latent_case(12)
    bg, bu, eps, alpha = 1.5, 2.0, 1e-3, 0.01
    g = O.latent_backward(u, wr, lambda e: W[e], wld, wlu, lambda j: Sw[j], S, dy, k=k,
                          act="situ", capacity=cap, beta_g=bg, beta_u=bu, rms_eps=eps,
                          alpha=alpha, aux_scale=aux)
    if cap is not None:
        assert int(g["disp"]["drop"].sum()) > 0
    # Independent torch forward: route on u, renormalised top-k, token-order
    # capacity, experts at width l with SiTU-GLU, RMSNorm, W_lup, shared
    # SwiGLU experts at width d, and the aux term with f held fixed.
    leaf = lambda m: torch.tensor(m, requires_grad=True)  # noqa: E731
    ut, wrt, wldt, wlut = leaf(u), leaf(wr), leaf(wld), leaf(wlu)
    Wt = [tuple(leaf(m) for m in ws) for ws in W]
    St = [tuple(leaf(m) for m in ws) for ws in Sw]
    z = ut @ wrt.T
    z.retain_grad()
    p = torch.softmax(z, dim=1)
    top = torch.topk(p, k, dim=1).indices
    psel = torch.gather(p, 1, top)
    a = psel / psel.sum(dim=1, keepdim=True)
    kept = np.ones((T, k), dtype=bool)
    if cap is not None:
        seen = np.zeros(N, dtype=int)
        for t in range(T):
            for s in range(k):
                e = int(top[t, s])
                kept[t, s] = seen[e] < cap
                seen[e] += 1
    xl = ut @ wldt.T
    rows = []
    for t in range(T):
        acc = torch.zeros(l, dtype=torch.float64)
        for s in range(k):
            if kept[t, s]:
                wg, wu, wd = Wt[int(top[t, s])]
                gg, vv = wg @ xl[t], wu @ xl[t]
                gg, vv = bg * torch.tanh(gg / bg), bu * torch.tanh(vv / bu)
                acc = acc + a[t, s] * (wd @ (F.silu(gg) * vv))
        rows.append(acc)
    r = torch.stack(rows)
    y = F.rms_norm(r, (l,), eps=eps) @ wlut.T
    for sg, su, sd in St:
        y = y + (F.silu(ut @ sg.T) * (ut @ su.T)) @ sd.T
    f = torch.tensor(np.bincount(np.argmax(p.detach().numpy(), axis=1), minlength=N) / T)
    loss = (torch.tensor(dy) * y).sum() + aux * alpha * N * (f * p.mean(dim=0)).sum()
    loss.backward()
    close = lambda x, ref: np.allclose(x, 0.0 if ref is None else ref.numpy(),  # noqa: E731
                                       rtol=1e-9, atol=1e-11)
    assert close(g["du"], ut.grad)
    assert close(g["dz"], z.grad)
    assert close(g["dW_route"], wrt.grad)
    assert close(g["dW_ldown"], wldt.grad)
    assert close(g["dW_lup"], wlut.grad)
    for e in range(N):
        assert close(g["dW_gate"][e], Wt[e][0].grad)
        assert close(g["dW_up"][e], Wt[e][1].grad)
        assert close(g["dW_down"][e], Wt[e][2].grad)
    for j in range(S):
        assert close(g["dWs_gate"][j], St[j][0].grad)
        assert close(g["dWs_up"][j], St[j][1].grad)
        assert close(g["dWs_down"][j], St[j][2].grad)


def test_latent_backward_only_selected_experts_receive_gradient():
    # 6 tokens, top-1 over 12 experts: at least 6 experts are never selected.
    u, wr, wld, wlu, W, Sw, dy = _latent_case(13, T=6, N=12)
    g = O.latent_backward(u, wr, lambda e: W[e], wld, wlu, lambda j: Sw[j], 2, dy, k=1,
                          act="situ", rms_eps=1e-6)
    used = set(int(e) for e in g["route"]["idx"].ravel())
    assert len(used) <= 6
    for e in range(12):
        total = sum(float(np.abs(g[n][e]).sum()) for n in ("dW_gate", "dW_up", "dW_down"))
        assert (total > 0) == (e in used)


def test_rmsnorm_backward_against_torch_and_scale_free():
    rng = np.random.default_rng(14)
    r = rng.standard_normal((5, 7)) * 3.0
    dn = rng.standard_normal((5, 7))
    for eps in (1e-6, 0.3):
        rt = torch.tensor(r, requires_grad=True)
        (torch.tensor(dn) * F.rms_norm(rt, (7,), eps=eps)).sum().backward()
        assert np.allclose(O.rmsnorm_backward(r, dn, eps), rt.grad.numpy(), rtol=1e-12,
                           atol=1e-14)
    # eps = 0: RMSNorm(c r) = RMSNorm(r), so the gradient has no component along r.
    dr = O.rmsnorm_backward(r, dn, 0.0)
    assert np.max(np.abs((dr * r).sum(axis=1))) < 1e-12


@pytest.mark.parametrize("cap,aux", [(None, 0.0), (7, 0.6)])
def test_latent_backward_tokens_matches_whole_layer(cap, aux):
    # The sampled-token form (used at full size) gives the whole-layer
    # backward's du and dz rows for those tokens, capacity drops included.
    u, wr, wld, wlu, W, Sw, dy = _latent_case(15)
    kw = dict(k=2, act="situ", capacity=cap, beta_g=1.5, beta_u=2.0, rms_eps=1e-3, aux_scale=aux)
    g = O.latent_backward(u, wr, lambda e: W[e], wld, wlu, lambda j: Sw[j], 2, dy, **kw)
    if cap is not None:
        assert int(g["disp"]["drop"].sum()) > 0
    tokens = np.array([0, 3, 11, 17, 23])
    t = O.latent_backward_tokens(u, wr, lambda e: W[e], wld, wlu, lambda j: Sw[j], 2, dy[tokens],
                                 tokens, **kw)
    assert np.allclose(t["du"], g["du"][tokens], rtol=1e-12, atol=1e-13)
    assert np.allclose(t["dz"], g["dz"][tokens], rtol=1e-12, atol=1e-13)
    assert np.allclose(t["dr"], g["dr"][tokens], rtol=1e-12, atol=1e-13)


def test_relative_error_hand_worked():
    """The parity checker max|y - y_ref| / max|y_ref|, worked by hand:
    y_ref = [[1.5, -2], [2, 0]] has max |.| = 2; y = [[1, -2], [3, 0.5]]
    differs by [[-0.5, 0], [1, 0.5]], largest 1, so the error is 1 / 2.  The
    denominator is the reference's (swapping the arguments gives 1 / 3), the
    largest element, not an average or a norm (a mean-based form gives 0.5 /
    1.375), and a transposed operand is caught: y^T - y_ref =
    [[-0.5, 5], [-4, 0.5]], error 5 / 2."""
    y_ref = np.array([[1.5, -2.0], [2.0, 0.0]])
    y = np.array([[1.0, -2.0], [3.0, 0.5]])
    assert O.relative_error(y, y_ref) == 0.5
    assert O.relative_error(y_ref, y) == 1.0 / 3.0
    assert O.relative_error(y.T, y_ref) == 2.5
    assert O.relative_error(y_ref, y_ref) == 0.0
    # bf16 outputs compared as fp32 values: the error is taken in fp64.
    assert O.relative_error(y.astype(np.float32), y_ref) == 0.5
    # An all-zero reference (a token whose every slot was dropped) reports
    # the absolute difference.
    assert O.relative_error(np.array([0.0, 0.25]), np.zeros(2)) == 0.25
