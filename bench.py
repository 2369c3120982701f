"""MoE-layer forward benchmark on one MI355X.

Default workload: the Mixtral-shape layer (d=4096, h=14336, N=8 experts,
top-2 renormalised, bf16, T=16384 tokens).  Inputs and weights are seeded
synthetic data already resident in HBM when the timed region starts.  One
step is one whole moe_forward (route, dispatch, expert gate/up, expert down,
combine).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU; % bf16 MFMA peak (prefill), % HBM BW (decode)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral_prefill_t16384")
    p.add_argument("--decode-workload", default="mixtral_decode_t32",
                   help="second workload reported beside the main one ('' to skip)")
    p.add_argument("--fp8-decode-workload", default="mixtral_decode_t32_fp8",
                   help="the decode workload with FP8 E4M3 expert weights ('' to skip)")
    p.add_argument("--mxfp4-decode-workload", default="mixtral_decode_t32_mxfp4",
                   help="the decode workload with MXFP4 expert weights ('' to skip)")
    p.add_argument("--switch-workload", default="switch_top1_skewed_t16384",
                   help="the skewed top-1 workload with a capacity limit, reported with its "
                        "balance statistics and drop ledger ('' to skip)")
    p.add_argument("--latent-workload", default="latent_t8192",
                   help="the LatentMoE workload ('' to skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-backward", action="store_true",
                   help="skip the backward-pass timings (forward and its stages only)")
    p.add_argument("--cpu-sample-tokens", type=int, default=1536,
                   help="pilot sample of the CPU baseline (the timed sample aims at ~15 s)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device-to-device copy (3 times) so that "
                        "hardware byte counters can be scaled against a known size")
    return p.parse_args()


def algorithmic(cfg, counts_kept):
    """Algorithmic work of one forward: expert FLOPs on kept rows, and the
    bytes of the selected experts' weights (each touched expert read once)."""
    R = int(sum(counts_kept))
    xw = cfg.x_width
    # bytes per weight, and scale bytes per weight row of K elements
    wb = {"bf16": 2, "f32": 4, "fp8": 1, "mxfp4": 0.5}[cfg.w_dtype]
    def sb(K):
        return {"fp8": 4, "mxfp4": K // 32}.get(cfg.w_dtype, 0)
    gu_flops = 2.0 * R * xw * 2 * cfg.h
    down_flops = 2.0 * R * cfg.h * xw
    touched = sum(1 for c in counts_kept if c > 0)
    gu_bytes = touched * 2 * cfg.h * (xw * wb + sb(xw))
    down_bytes = touched * xw * (cfg.h * wb + sb(cfg.h))
    return {"rows": R, "gu_flops": gu_flops, "down_flops": down_flops, "gu_bytes": gu_bytes,
            "down_bytes": down_bytes, "touched": touched}


def tile_rows(cfg):
    """m-tile height the library uses for the routed expert GEMMs (for the
    kernel label only): whichever of 256 and 192 pads the mean kept rows per
    expert least."""
    import math
    kept = cfg.T * cfg.k if cfg.capacity_factor is None else min(
        cfg.T * cfg.k, cfg.N * math.ceil(cfg.capacity_factor * cfg.k * cfg.T / cfg.N))
    e = kept / cfg.N
    w = {bm: math.ceil(e / bm) * bm - e for bm in (256, 192)}
    return 192 if w[192] < w[256] else 256


def measured_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel, from the
    rocprofv3 counter runs recorded in profiles/hbm_traffic.json, or None when
    there is no record or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)["workloads"].get(workload)
    if rec is None:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes"]


class SclkSampler:
    """Samples the GPU's shader clock (the active level of the amdgpu
    driver's pp_dpm_sclk table) from a host thread while queued work runs."""

    def __init__(self, period_s=0.002):
        import glob
        self.path = next((p for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
                          if os.access(p, os.R_OK)), None)
        self.period = period_s
        self.samples = []

    def _read(self):
        try:
            with open(self.path) as f:
                for ln in f:
                    if ln.rstrip().endswith("*"):
                        return float(ln.split(":")[1].strip().split("M")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _loop(self):
        while not self.stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self.stop.wait(self.period)

    def __enter__(self):
        import threading
        self.stop = threading.Event()
        self.thread = None
        if self.path is not None:
            self.thread = threading.Thread(target=self._loop, daemon=True)
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.thread is not None:
            self.thread.join()

    def summary(self):
        if not self.samples:
            return None
        import numpy as np
        s = np.array(self.samples)
        return {"median": float(np.median(s)), "min": float(s.min()), "max": float(s.max()),
                "samples": int(s.size), "source": self.path}


def run_workload(cfg, steps, warmup, backward=True):
    import numpy as np
    import torch

    import sparse_mixture_experts_11_amd as moe
    from tests import harness as H

    desc = H.desc_for(cfg)
    w = H.upload_layer(cfg)
    u = H.to_device(cfg.u())
    y = H.y_buffer(cfg)
    out = H.out_buffers(cfg)
    ws = moe.workspace(desc)
    stages = moe.moe_stage_names(desc)
    stream = torch.cuda.current_stream()

    def mk():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]

    for _ in range(warmup):
        moe.moe_forward(desc, w, u, y, out, ws)
    torch.cuda.synchronize()
    # Timed region: `steps` plain forwards (no markers inside a step).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(steps):
        moe.moe_forward(desc, w, u, y, out, ws)
    t_end.record(stream)
    with SclkSampler() as sclk:   # while the queued steps run
        torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # Stage breakdown: the same number of forwards again, each with HIP events
    # recorded between its stages on the same stream.  The markers cost a few
    # microseconds each, so these steps run a little longer than the timed
    # ones; each stage's own duration is what the events bracket.
    ev = [mk() for _ in range(steps)]
    for i in range(steps):
        moe.moe_forward_traced(desc, w, u, y, out, ws, ev[i])
    torch.cuda.synchronize()
    per_stage = {s: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
                 for j, s in enumerate(stages)}
    per_step = [ev[i][0].elapsed_time(ev[i][-1]) for i in range(steps)]
    kept = np.diff(H.to_host(out["kept_offsets"]))
    graph_ms = None
    if cfg.T <= 64:
        # Launch-bound decode: the same forward captured once in a HIP graph
        # and replayed (the library allocates nothing and never syncs).
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            moe.moe_forward(desc, w, u, y, out, ws)
        stream.wait_stream(cs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            moe.moe_forward(desc, w, u, y, out, ws)
        graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / steps
        del graph
    r = {"ms_per_step": total_ms / steps, "stages_ms": per_stage,
         "traced_step_ms": {"median": float(np.median(per_step)), "min": float(np.min(per_step)),
                            "mean": float(np.mean(per_step))},
         "alg": algorithmic(cfg, kept), "desc": desc, "graph_ms_per_step": graph_ms,
         "sclk_mhz": sclk.summary(), "counts": H.to_host(out["counts"]), "kept": kept, "stats": H.to_host(out["stats"])}
    if cfg.act_dtype == "bf16" and cfg.router_dtype == "bf16":
        r["quantile_balancing"] = time_qb(moe, desc, u, w["W_route"], ws, cfg, steps)
        if not backward:
            pass
        elif not cfg.latent:
            r["route_backward"] = time_route_backward(moe, H, desc, u, w, y, out, ws, cfg, steps)
            if cfg.w_dtype == "bf16":
                r["experts_backward"] = time_experts_backward(moe, H, desc, u, w, out, cfg,
                                                              max(3, steps // 4))
        elif cfg.w_dtype == "bf16":
            r["latent_backward"] = time_latent_backward(moe, H, desc, u, w, y, out, ws, cfg,
                                                        max(3, steps // 4))
    return r


def time_latent_backward(moe, H, desc, u, w, y, out, ws, cfg, steps):
    """moe_latent_backward (every gradient) after a forward that hands out its
    expert outputs, with a seeded dy; averaged over `steps`.  Algorithmic
    work: the routed experts' 8 products of R x l x H and the shared experts'
    8 of T x d x h_s (2 m n k flops each), five T x d x l products (x_l
    recomputed, dn, dW_lup, du through W_ldown, dW_ldown) and three T x N x d
    (logits, dW_route, the router's du)."""
    import torch

    import synth as S

    kept = int(H.to_host(out["kept_offsets"])[-1])
    y_perm = torch.empty((max(kept, 1), cfg.l), dtype=torch.float32, device="cuda")
    out = dict(out, y_perm=y_perm)
    moe.moe_forward(desc, w, u, y, out, ws)
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()
    dy = H.to_device(S.normal_stored(cfg.seed + 1, 96, cfg.T * cfg.d, 0.5, "bf16")
                     .reshape(cfg.T, cfg.d))
    f = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")  # noqa: E731
    g = {"du": f(cfg.T, cfg.d), "dz": f(cfg.T, cfg.N), "dW_route": f(cfg.N, cfg.d),
         "dW_ldown": f(cfg.l, cfg.d), "dW_lup": f(cfg.d, cfg.l),
         "dW_gate": f(cfg.N, cfg.h, cfg.l), "dW_up": f(cfg.N, cfg.h, cfg.l),
         "dW_down": f(cfg.N, cfg.l, cfg.h)}
    if cfg.n_shared:
        g.update(dWs_gate=f(cfg.n_shared, cfg.h_shared, cfg.d),
                 dWs_up=f(cfg.n_shared, cfg.h_shared, cfg.d),
                 dWs_down=f(cfg.n_shared, cfg.d, cfg.h_shared))
    bws = moe.backward_workspace(desc)

    def timed(fwd):
        moe.moe_latent_backward(desc, w, u, fwd, dy, g, bws, aux_scale=1.0)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            moe.moe_latent_backward(desc, w, u, fwd, dy, g, bws, aux_scale=1.0)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms = timed(out)
    T, d, l = cfg.T, cfg.d, cfg.l
    flops = (16.0 * kept * l * cfg.h + 16.0 * cfg.n_shared * T * d * cfg.h_shared
             + 10.0 * T * d * l + 6.0 * T * cfg.N * d)
    res = {"ms": ms, "algorithmic_tflop": flops / 1e12, "tflops": flops / (ms / 1e3) / 1e12,
           "mfma_frac": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
           "workspace_gb": moe.moe_backward_workspace_bytes(desc) / 1e9}
    # With the forward keeping the routed experts' G | U.
    gu = torch.empty((max(kept, 1), 2 * cfg.h), dtype=torch.bfloat16, device="cuda")
    fws = moe.workspace(desc)
    out_gu = dict(out, gate_up=gu)
    moe.moe_forward(desc, w, u, y, out_gu, fws)
    torch.cuda.synchronize()
    del fws
    res["saved_gate_up_ms"] = timed(out_gu)
    del bws, g, gu
    torch.cuda.empty_cache()
    return res


def time_experts_backward(moe, H, desc, u, w, out, cfg, steps):
    """moe_experts_backward (dx and all three weight gradients) after a
    forward, with a seeded dy; averaged over `steps`.  Algorithmic work:
    8 GEMM-sized products of R x d x h (gate/up recompute 2, dH 1, dx 2,
    dW_down 1, dW_gate + dW_up 2), 2 R d h flops each."""
    import torch

    import synth as S

    kept = int(H.to_host(out["kept_offsets"])[-1])
    ws = moe.backward_workspace(desc)
    dy = H.to_device(S.normal_stored(cfg.seed + 1, 95, cfg.T * cfg.d, 0.5, "bf16")
                     .reshape(cfg.T, cfg.d))
    dx = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    dW = {"dW_gate": torch.empty((cfg.N, cfg.h, cfg.d), dtype=torch.float32, device="cuda"),
          "dW_up": torch.empty((cfg.N, cfg.h, cfg.d), dtype=torch.float32, device="cuda"),
          "dW_down": torch.empty((cfg.N, cfg.d, cfg.h), dtype=torch.float32, device="cuda")}
    args = (desc, w, u, out["topk_w"], out["offsets"], out["kept_offsets"], out["perm"],
            out["row_of"], dy, dx, ws)

    def timed(fn):
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms = timed(lambda: moe.moe_experts_backward(*args, **dW))
    flops = 16.0 * kept * cfg.d * cfg.h
    res = {"ms": ms, "algorithmic_tflop": flops / 1e12,
           "tflops": flops / (ms / 1e3) / 1e12,
           "mfma_frac": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
           "workspace_gb": moe.moe_backward_workspace_bytes(desc) / 1e9}
    # With the forward keeping G | U (moe_outputs_t.gate_up): the backward
    # skips the recompute (6 of the 8 products remain); the forward pays for
    # writing the 2 R h bf16 values.
    if cfg.T > 64:
        gu = torch.empty((max(kept, 1), 2 * cfg.h), dtype=torch.bfloat16, device="cuda")
        fws = moe.workspace(desc)
        y = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
        out_gu = dict(out, gate_up=gu)
        f_plain = timed(lambda: moe.moe_forward(desc, w, u, y, out, fws))
        f_save = timed(lambda: moe.moe_forward(desc, w, u, y, out_gu, fws))
        ms_s = timed(lambda: moe.moe_experts_backward(*args, gate_up=gu, **dW))
        flops_s = 12.0 * kept * cfg.d * cfg.h
        res["saved_gate_up"] = {"ms": ms_s, "algorithmic_tflop": flops_s / 1e12,
                                "tflops": flops_s / (ms_s / 1e3) / 1e12,
                                "mfma_frac": flops_s / (ms_s / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                                "forward_ms_plain": f_plain, "forward_ms_saving": f_save}
        del gu, fws
    del ws, dW
    return res


def time_route_backward(moe, H, desc, u, w, y, out, ws, cfg, steps):
    """moe_route_backward after a forward that hands out its expert outputs,
    with a seeded upstream gradient dy; averaged over `steps`.  Algorithmic
    bytes: u twice (logits GEMM, dW_route), dy, the kept expert-output rows
    (fp32), du written (fp32), dz and the logits (T x N fp32, three passes)."""
    import torch

    import synth as S

    kept = int(H.to_host(out["kept_offsets"])[-1])
    y_perm = torch.empty((max(kept, 1), cfg.d), dtype=torch.float32, device="cuda")
    out = dict(out, y_perm=y_perm)
    moe.moe_forward(desc, w, u, y, out, ws)
    dy = H.to_device(S.normal_stored(cfg.seed + 1, 96, cfg.T * cfg.d, 0.5, "bf16")
                     .reshape(cfg.T, cfg.d))
    dz = torch.empty((cfg.T, cfg.N), dtype=torch.float32, device="cuda")
    dw = torch.empty((cfg.N, cfg.d), dtype=torch.float32, device="cuda")
    du = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    args = (desc, u, w["W_route"], out["topk_idx"], out["row_of"], out["stats"], y_perm, dy, dz,
            dw, du, ws)
    for _ in range(5):
        moe.moe_route_backward(*args, aux_scale=1.0)
    # A call is ~0.4 ms: one batch of `steps` calls is short enough for a
    # clock transient to dominate it, so three batches are timed and the
    # median batch is reported.
    batches = []
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            moe.moe_route_backward(*args, aux_scale=1.0)
        b.record()
        torch.cuda.synchronize()
        batches.append(a.elapsed_time(b) / steps)
    ms = sorted(batches)[1]
    T, d, N = cfg.T, cfg.d, cfg.N
    alg = 2 * T * d * 2 + T * d * 2 + kept * d * 4 + T * d * 4 + 3 * T * N * 4
    return {"ms": ms, "batch_ms": batches, "algorithmic_bytes": alg,
            "gb_s": alg / (ms / 1e3) / 1e9, "hbm_frac": alg / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}


def time_qb(moe, desc, u, w_route, ws, cfg, steps):
    """One Quantile Balancing bias update (router logits, cutoffs, per-expert
    quantile) from zero bias, exact and histogram, averaged over `steps`."""
    import torch

    nb = torch.empty(cfg.N, dtype=torch.float32, device="cuda")
    res = {}
    for name, method in (("exact_ms", moe.QB_EXACT), ("histogram_ms", moe.QB_HISTOGRAM)):
        for _ in range(2):
            moe.moe_qb_update(desc, u, w_route, None, nb, ws, method=method)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            moe.moe_qb_update(desc, u, w_route, None, nb, ws, method=method)
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / steps
    res["q"] = int((2 * cfg.k * cfg.T + cfg.N) // (2 * cfg.N))
    return res


def _host_info():
    from threadpoolctl import threadpool_info
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return int(threads), model


def _oracle_sample(cfg, n, expert_budget_bytes):
    """Inputs of one oracle forward over the first n tokens of the workload
    (the layer taken at T = n, so a capacity limit is recomputed for n), with
    every weight the sample touches generated and expanded to fp64 up front,
    so that the timed region holds the oracle's arithmetic only.  For the
    latent layer n shrinks until the touched routed experts fit the budget."""
    import numpy as np

    import oracle as O

    while True:
        sub = cfg.with_(T=n)
        u = sub.u()
        wr = sub.w_route()
        idx = O.route(O.expand(u), O.expand(wr), sub.k, sub.gate)["idx"]
        touched = sorted(set(int(e) for e in np.unique(idx)))
        per = 3 * sub.h * sub.x_width * 8
        if not cfg.latent or len(touched) * per <= expert_budget_bytes or n == 1:
            break
        n = max(1, n // 2)
    experts = {e: tuple(O.expand(m) for m in sub.expert(e)) for e in touched}

    def kw(T):
        cap = None if cfg.capacity_factor is None else O.capacity_from_factor(
            T, sub.N, sub.k, sub.capacity_factor)
        return dict(k=sub.k, gate=sub.gate, act=sub.act, capacity=cap, beta_g=sub.beta_g,
                    beta_u=sub.beta_u, alpha=sub.aux_alpha)

    if cfg.latent:
        shared = [tuple(O.expand(m) for m in sub.shared(j)) for j in range(sub.n_shared)]
        wld, wlu = O.expand(sub.w_ldown()), O.expand(sub.w_lup())

        def run(rows=None):
            uu = u if rows is None else u[rows]
            return O.latent_forward(uu, wr, experts.__getitem__, wld, wlu, shared.__getitem__,
                                    sub.n_shared, rms_eps=sub.rms_eps, **kw(uu.shape[0]))
    else:
        def run(rows=None):
            uu = u if rows is None else u[rows]
            return O.forward(uu, wr, experts.__getitem__, **kw(uu.shape[0]))
    return n, run


def cpu_baseline(cfg, n_tokens, target_s=15.0, expert_budget_bytes=24e9):
    """The fp64 oracle, as it stands, on the host: a forward over the first n
    tokens of the workload with its weights already generated and expanded
    (the generator is not timed).  A pilot on n_tokens sizes the timed
    sample to about target_s seconds (at most the whole workload).  A second
    figure runs the oracle on one thread over a deterministic 1/64 subsample
    of the timed tokens (every 64th) and scales it up to the whole sample:
    an extrapolation, labelled as one."""
    from threadpoolctl import threadpool_limits

    def timed(n):
        n, run = _oracle_sample(cfg, n, expert_budget_bytes)
        t0 = time.perf_counter()
        run()
        return n, run, time.perf_counter() - t0

    n, run, dt = timed(n_tokens)
    for _ in range(3):
        if dt >= 0.6 * target_s or n >= cfg.T or cfg.latent:
            break
        n, run, dt = timed(int(min(cfg.T, max(n + 1, n * target_s / dt))))
    threads, model = _host_info()
    # Single thread on every 64th token of the sample (the layer taken at the
    # subsample's size: routing, dispatch and experts over those tokens).
    rows = list(range(0, n, 64))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        run(rows)
        dt1 = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"fp64 oracle forward of the first {n} of {cfg.T} tokens, {dt:.1f} s; "
                      "weights generated and expanded to fp64 before timing",
            "single_thread_extrapolated": {
                "value": len(rows) / dt1, "unit": "tokens/s", "cores": 1,
                "sample": f"every 64th of those {n} tokens ({len(rows)} tokens) on one thread, "
                          f"{dt1:.2f} s; extrapolation: the {n}-token sample would take "
                          f"{dt1 * n / len(rows):.1f} s"}}


def cpu_baseline_balance_stats(cfg):
    """The oracle's balance statistics of a whole workload (routing only, all
    T tokens), for comparison with the GPU's."""
    import oracle as O

    r = O.route(O.expand(cfg.u()), O.expand(cfg.w_route()), cfg.k, cfg.gate)
    s = O.balance_stats(r["p"], cfg.aux_alpha)
    return {"f": [float(x) for x in s["f"]], "P": [float(x) for x in s["P"]],
            "n_sum_fP": float(s["n_sum_fP"]), "aux": float(s["aux"])}


def switch_section(cfg, r):
    """A top-1 layer with a capacity limit: throughput, the gate/up kernel on
    its kept rows, the balance statistics f_i, P_i, N sum f P and the
    auxiliary loss alpha N sum f P (page "MoE: how sparse activation saves
    compute", section 3.4), and the capacity ledger of section 3.8 (tokens
    over capacity, empty slots)."""
    from tests import harness as H

    N = cfg.N
    a = r["alg"]
    cap = H.capacity_of(cfg)
    counts = [int(c) for c in r["counts"]]
    st = r["stats"]
    t_gu = r["stages_ms"]["expert_gate_up"] / 1e3
    return {
        "workload": cfg.name, "T": cfg.T, "k": cfg.k, "gate": cfg.gate,
        "tokens_per_s": cfg.T / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
        "stages_ms": r["stages_ms"], "sclk_mhz": r["sclk_mhz"],
        "expert_gate_up_kept_rows": {"rows": a["rows"], "tflop": a["gu_flops"] / 1e12,
                                     "tflops": a["gu_flops"] / t_gu / 1e12,
                                     "mfma_frac": a["gu_flops"] / t_gu / 1e12 / PEAK_BF16_TFLOPS},
        "capacity": cap, "loads": counts, "kept": [int(c) for c in r["kept"]],
        "dropped": int(sum(max(c - cap, 0) for c in counts)),
        "empty_slots": int(sum(max(cap - c, 0) for c in counts)),
        "f": [float(x) for x in st[:N]], "P": [float(x) for x in st[N:2 * N]],
        "n_sum_fP": float(st[2 * N]), "aux_alpha": cfg.aux_alpha, "aux": float(st[2 * N + 1]),
    }


def latent_section(cfg, r):
    """The LatentMoE layer: throughput, stages, and the routed expert GEMMs
    against HBM (their weights, 146 rows per expert on average, make them
    bandwidth-bound)."""
    a = r["alg"]
    t_gu = r["stages_ms"]["expert_gate_up"] / 1e3
    t_dn = r["stages_ms"]["expert_down"] / 1e3
    sec = {
        "workload": cfg.name, "T": cfg.T, "d": cfg.d, "l": cfg.l, "H": cfg.h, "E": cfg.N,
        "k": cfg.k, "n_shared": cfg.n_shared, "expert_weights": cfg.w_dtype,
        "tokens_per_s": cfg.T / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
        "stages_ms": r["stages_ms"], "sclk_mhz": r["sclk_mhz"],
        "routed_gate_up": {"weight_bytes": a["gu_bytes"], "gb_s": a["gu_bytes"] / t_gu / 1e9,
                           "hbm_frac": a["gu_bytes"] / t_gu / 1e9 / PEAK_HBM_GBS},
        "routed_down": {"weight_bytes": a["down_bytes"], "gb_s": a["down_bytes"] / t_dn / 1e9,
                        "hbm_frac": a["down_bytes"] / t_dn / 1e9 / PEAK_HBM_GBS},
        "experts_touched": a["touched"], "rows": a["rows"],
    }
    if "latent_backward" in r:
        sec["latent_backward"] = r["latent_backward"]
    return sec


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this layer has no "
              "multi-GPU path here", file=sys.stderr)
        sys.exit(2)
    import torch

    from synth import configs as C

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = C.ALL[args.workload]
    print(f"[bench] {cfg.name}: uploading weights", file=sys.stderr, flush=True)
    r = run_workload(cfg, args.steps, args.warmup, backward=not args.no_backward)
    tok_s = cfg.T / (r["ms_per_step"] / 1e3)
    alg = r["alg"]
    total_flops = alg["gu_flops"] + alg["down_flops"]
    # Dominant kernel: the expert gate/up stage (one launch).  Its bound is
    # set by arithmetic intensity against the ridge (peak flop/s / peak B/s).
    t = r["stages_ms"]["expert_gate_up"] / 1e3
    intensity = alg["gu_flops"] / alg["gu_bytes"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if cfg.act_dtype != "bf16":
        kernel = "simt_gu_kernel (fp32 expert gate/up)"
    elif cfg.T <= 64:
        wf = {"bf16": 0, "fp8": 1, "mxfp4": 2}[cfg.w_dtype]
        tg = 1 if cfg.T <= 32 else 2   # token groups a workgroup holds
        kernel = f"decode_kernel<true, {tg}, {wf}> (expert gate/up)"
    else:
        kernel = (f"grouped_gemm_kernel<EP_GLU, {tile_rows(cfg)}"
                  f"{', true' if cfg.w_dtype == 'fp8' else ''}> (expert gate/up)")
    if intensity < ridge:
        achieved = alg["gu_bytes"] / t / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(cfg.name),
                "kernel": kernel}
    else:
        achieved = alg["gu_flops"] / t / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(cfg.name), "kernel": kernel}
    roof["algorithmic_per_launch"] = {"flops": alg["gu_flops"], "bytes": alg["gu_bytes"],
                                      "rows": alg["rows"], "experts_touched": alg["touched"]}
    line = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "traced_step_ms": r["traced_step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.act_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "h": cfg.h, "N": cfg.N,
                   "k": cfg.k, "expert_weights": cfg.w_dtype, "parallelism": "single GPU"},
        "tflops": total_flops / (r["ms_per_step"] / 1e3) / 1e12,
        "expert_stage_tflops": total_flops / (
            (r["stages_ms"]["expert_gate_up"] + r["stages_ms"]["expert_down"]) / 1e3) / 1e12,
        "stages_ms": r["stages_ms"],
        "sclk_mhz": r["sclk_mhz"],
        "roofline": roof,
    }
    if r.get("graph_ms_per_step") is not None:
        line["graph_ms_per_step"] = r["graph_ms_per_step"]
    if "quantile_balancing" in r:
        line["quantile_balancing"] = r["quantile_balancing"]
    if "route_backward" in r:
        line["route_backward"] = r["route_backward"]
    if "experts_backward" in r:
        line["experts_backward"] = r["experts_backward"]
    if "latent_backward" in r:
        line["latent_backward"] = r["latent_backward"]
    for key, name in (("decode", args.decode_workload), ("decode_fp8", args.fp8_decode_workload),
                      ("decode_mxfp4", args.mxfp4_decode_workload)):
        if not name:
            continue
        dc = C.ALL[name]
        print(f"[bench] {dc.name}", file=sys.stderr, flush=True)
        rd = run_workload(dc, args.steps, args.warmup, backward=False)
        a = rd["alg"]
        wbytes = a["gu_bytes"] + a["down_bytes"]
        line[key] = {
            "workload": dc.name, "expert_weights": dc.w_dtype,
            "tokens_per_s": dc.T / (rd["ms_per_step"] / 1e3),
            "ms_per_step": rd["ms_per_step"], "graph_ms_per_step": rd["graph_ms_per_step"],
            "stages_ms": rd["stages_ms"], "sclk_mhz": rd["sclk_mhz"],
            "selected_expert_weight_bytes": wbytes,
            "hbm_frac_whole_forward": wbytes / (rd["ms_per_step"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "hbm_frac_expert_kernels": wbytes / ((rd["stages_ms"]["expert_gate_up"] +
                                                  rd["stages_ms"]["expert_down"]) / 1e3)
            / 1e9 / PEAK_HBM_GBS,
        }
        del rd
    if args.switch_workload and args.switch_workload != args.workload:
        sc = C.ALL[args.switch_workload]
        print(f"[bench] {sc.name}", file=sys.stderr, flush=True)
        line["switch_top1"] = switch_section(sc, run_workload(sc, args.steps, args.warmup,
                                                              backward=False))
    if args.latent_workload and args.latent_workload != args.workload:
        lc = C.ALL[args.latent_workload]
        print(f"[bench] {lc.name}: uploading weights", file=sys.stderr, flush=True)
        line["latent"] = latent_section(lc, run_workload(lc, args.steps, args.warmup,
                                                         backward=not args.no_backward))
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_sample_tokens, cfg.T))
        if "switch_top1" in line:
            ref = cpu_baseline_balance_stats(C.ALL[args.switch_workload])
            gpu = line["switch_top1"]
            ref["aux_rel_diff_gpu"] = abs(gpu["aux"] - ref["aux"]) / ref["aux"]
            ref["f_equal_gpu"] = bool(all(abs(a - b) * gpu["T"] < 0.5
                                          for a, b in zip(gpu["f"], ref["f"])))
            line["cpu_baseline"]["switch_top1_balance_stats"] = ref
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
