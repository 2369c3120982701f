"""Host-side logic of bench.py that needs no GPU: the CPU-baseline leg (the
oracle timed on pre-generated weights) on small plain, capacity-limited and
latent layers, and the report sections built from a run's outputs."""
from __future__ import annotations

import numpy as np

import bench
from synth import configs as C


def _check(r, n_max):
    assert r["value"] > 0 and r["unit"] == "tokens/s" and r["kind"] == "oracle"
    assert r["cores"] >= 1
    assert "before timing" in r["sample"]
    st = r["single_thread_extrapolated"]
    assert st["cores"] == 1 and st["value"] > 0 and "extrapolation" in st["sample"]
    n = int(r["sample"].split("first ")[1].split(" ")[0])
    assert 1 <= n <= n_max


def test_cpu_baseline_plain():
    cfg = C.MIXTRAL_PREFILL.with_(T=200, d=64, h=96)
    _check(bench.cpu_baseline(cfg, 130, target_s=0.05), cfg.T)


def test_cpu_baseline_capacity_limited():
    cfg = C.SWITCH_SKEWED.with_(T=300, d=64, h=64)
    _check(bench.cpu_baseline(cfg, 100, target_s=0.05), cfg.T)


def test_cpu_baseline_latent():
    cfg = C.LATENT.with_(T=100, d=64, l=32, h=48, N=24, k=4, h_shared=32)
    _check(bench.cpu_baseline(cfg, 100, target_s=0.05), cfg.T)
    # A budget that holds only a few experts shrinks the sample.
    r = bench.cpu_baseline(cfg, 100, target_s=0.05, expert_budget_bytes=6 * 3 * 48 * 32 * 8)
    _check(r, 2)


def test_balance_stats_leg_matches_definition():
    cfg = C.SWITCH_SKEWED.with_(T=500, d=64, h=64)
    s = bench.cpu_baseline_balance_stats(cfg)
    assert abs(sum(s["f"]) - 1.0) < 1e-12 and abs(sum(s["P"]) - 1.0) < 1e-12
    assert abs(s["n_sum_fP"] - cfg.N * float(np.dot(s["f"], s["P"]))) < 1e-12
    assert abs(s["aux"] - cfg.aux_alpha * s["n_sum_fP"]) < 1e-15


def test_switch_section_ledger():
    cfg = C.SWITCH_SKEWED.with_(T=80, d=64, h=64, N=4)
    counts = np.array([50, 20, 10, 0])
    cap = 25   # ceil(1.25 * 80 / 4)
    N = cfg.N
    stats = np.concatenate([counts / 80.0, np.full(N, 0.25), [1.0, 0.01]]).astype(np.float32)
    r = {"alg": bench.algorithmic(cfg, np.minimum(counts, cap)), "counts": counts,
         "kept": np.minimum(counts, cap), "stats": stats, "ms_per_step": 1.0,
         "stages_ms": {"expert_gate_up": 0.5}, "sclk_mhz": None}
    sec = bench.switch_section(cfg, r)
    assert sec["capacity"] == cap
    assert sec["dropped"] == 25 and sec["empty_slots"] == 0 + 5 + 15 + 25
    assert sec["kept"] == [25, 20, 10, 0]
    assert sec["expert_gate_up_kept_rows"]["rows"] == 55
    assert abs(sec["aux"] - 0.01) < 1e-9


def test_sclk_sampler_without_sysfs():
    s = bench.SclkSampler()
    s.path = None
    with s:
        pass
    assert s.summary() is None
