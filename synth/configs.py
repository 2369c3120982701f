"""Workload recipes: shapes, dtypes, seeds and the synthetic input recipe.

Each recipe says how to draw every tensor of one MoE layer from the seeded
generator in ``synth``. Nothing here computes any part of the layer; the
capacity is stated as a factor and each side converts it itself.

Init convention: every weight matrix is drawn from N(0, 1/fan_in), with
fan_in the length of the dimension it contracts over; activations u ~ N(0,1).
Values are sampled in fp64 and rounded to the stored dtype, nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

import synth as S


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    T: int
    d: int
    h: int                      # expert hidden (H for the latent layer)
    N: int                      # routed experts (E for the latent layer)
    k: int
    act_dtype: str = "bf16"     # "f32" | "bf16"
    w_dtype: str = "bf16"      # routed experts: "f32" | "bf16" | "fp8" (E4M3 rows) | "mxfp4"
    router_dtype: str = "bf16"
    gate: str = "renorm"        # "renorm" (a = p / sum_S p) | "prob" (a = p)
    act: str = "swiglu"         # "swiglu" | "situ"
    beta_g: float = 4.0
    beta_u: float = 25.0
    capacity_factor: Optional[float] = None   # None: unlimited
    l: int = 0                  # latent width, 0 for the plain layer
    n_shared: int = 0
    h_shared: int = 0
    rms_eps: float = 1e-6
    aux_alpha: float = 0.01
    seed: int = 0
    hot_rows: Sequence[int] = ()   # router rows scaled after sampling
    hot_scale: float = 1.0
    planted: Optional[Sequence[int]] = None   # planted top-1 assignment per token
    planted_gain: float = 8.0
    planted_noise: float = 0.01

    # ---- derived shapes -------------------------------------------------
    @property
    def latent(self) -> bool:
        return self.l > 0

    @property
    def x_width(self) -> int:
        """Width of the vectors the routed experts read and write."""
        return self.l if self.latent else self.d

    def with_(self, **kw) -> "Layer":
        return dataclasses.replace(self, **kw)

    # ---- stored tensors ---------------------------------------------------
    def u(self, rows: Optional[np.ndarray] = None) -> np.ndarray:
        """Activations [T, d] (or the given token rows) in act_dtype."""
        if self.planted is not None:
            return self._planted_u(rows)
        if rows is None:
            return S.normal_stored(self.seed, S.TID_U, self.T * self.d, 1.0,
                                   self.act_dtype).reshape(self.T, self.d)
        rows = np.asarray(rows, dtype=np.int64)
        out = np.empty((rows.size, self.d),
                       dtype=np.uint16 if self.act_dtype == "bf16" else np.float32)
        for i, t in enumerate(rows):
            out[i] = S.normal_stored(self.seed, S.TID_U, self.d, 1.0, self.act_dtype,
                                     start=int(t) * self.d)
        return out

    def w_route(self) -> np.ndarray:
        """Router matrix [N, d] in router_dtype."""
        if self.planted is not None:
            # Planted router: expert i reads coordinate i with a large gain.
            w = np.zeros((self.N, self.d))
            for i in range(self.N):
                w[i, i] = self.planted_gain
            return S.round_to(w, self.router_dtype)
        w = S.normal_f64(self.seed, S.TID_W_ROUTE, self.N * self.d,
                         1.0 / math.sqrt(self.d)).reshape(self.N, self.d)
        for r in self.hot_rows:
            w[r] *= self.hot_scale
        return S.round_to(w, self.router_dtype)

    def _planted_u(self, rows):
        a = np.asarray(self.planted)
        assert a.size == self.T
        noise = S.normal_f64(self.seed, S.TID_U_NOISE, self.T * self.d,
                             self.planted_noise).reshape(self.T, self.d)
        u = noise.copy()
        u[np.arange(self.T), a] += 1.0
        u = S.round_to(u, self.act_dtype)
        return u if rows is None else u[np.asarray(rows)]

    # Routed expert e: gate/up [h, x_width], down [x_width, h].  With
    # w_dtype "fp8" each is an Fp8Rows drawn from the same values.
    def _expert_matrix(self, tid, rows, cols, std, start):
        if self.w_dtype == "fp8":
            return S.normal_fp8_rows(self.seed, tid, rows, cols, std, start=start)
        if self.w_dtype == "mxfp4":
            return S.normal_mxfp4_rows(self.seed, tid, rows, cols, std, start=start)
        return S.normal_stored(self.seed, tid, rows * cols, std, self.w_dtype,
                               start=start).reshape(rows, cols)

    def expert(self, e: int):
        xw, h = self.x_width, self.h
        n = h * xw
        g = self._expert_matrix(S.TID_W_GATE, h, xw, 1.0 / math.sqrt(xw), e * n)
        u = self._expert_matrix(S.TID_W_UP, h, xw, 1.0 / math.sqrt(xw), e * n)
        dn = self._expert_matrix(S.TID_W_DOWN, xw, h, 1.0 / math.sqrt(h), e * n)
        return g, u, dn

    def expert_tensor(self, which: str, out: Optional[np.ndarray] = None):
        """Whole stacked routed-expert tensor: gate/up [N,h,xw], down [N,xw,h]
        (fp8: an Fp8Rows of codes [N,rows,cols] and scales [N,rows])."""
        xw, h = self.x_width, self.h
        n = self.N * h * xw
        tid, std, shape = {
            "gate": (S.TID_W_GATE, 1.0 / math.sqrt(xw), (self.N, h, xw)),
            "up": (S.TID_W_UP, 1.0 / math.sqrt(xw), (self.N, h, xw)),
            "down": (S.TID_W_DOWN, 1.0 / math.sqrt(h), (self.N, xw, h)),
        }[which]
        if self.w_dtype == "fp8":
            m = S.normal_fp8_rows(self.seed, tid, self.N * shape[1], shape[2], std,
                                  codes=None if out is None else out.reshape(-1))
            return S.Fp8Rows(m.codes.reshape(shape), m.scale.reshape(shape[:2]))
        if self.w_dtype == "mxfp4":
            m = S.normal_mxfp4_rows(self.seed, tid, self.N * shape[1], shape[2], std)
            return S.MxFp4Rows(m.packed.reshape(shape[:2] + (shape[2] // 2,)),
                               m.block_scale.reshape(shape[:2] + (shape[2] // 32,)))
        flat = None if out is None else out.reshape(-1)
        return S.normal_stored(self.seed, tid, n, std, self.w_dtype, out=flat).reshape(shape)

    # Latent projections and shared experts are stored in the activation
    # dtype when the routed experts are fp8.
    @property
    def dense_w_dtype(self) -> str:
        return self.act_dtype if self.w_dtype in ("fp8", "mxfp4") else self.w_dtype

    def w_ldown(self) -> np.ndarray:   # [l, d]
        return S.normal_stored(self.seed, S.TID_W_LDOWN, self.l * self.d,
                               1.0 / math.sqrt(self.d), self.dense_w_dtype).reshape(self.l, self.d)

    def w_lup(self) -> np.ndarray:     # [d, l]
        return S.normal_stored(self.seed, S.TID_W_LUP, self.d * self.l,
                               1.0 / math.sqrt(self.l), self.dense_w_dtype).reshape(self.d, self.l)

    def shared_tensor(self, which: str) -> np.ndarray:
        """Shared experts: gate/up [S,h_s,d], down [S,d,h_s]."""
        Sx, hs, d = self.n_shared, self.h_shared, self.d
        n = Sx * hs * d
        if which == "gate":
            return S.normal_stored(self.seed, S.TID_WS_GATE, n, 1.0 / math.sqrt(d),
                                   self.dense_w_dtype).reshape(Sx, hs, d)
        if which == "up":
            return S.normal_stored(self.seed, S.TID_WS_UP, n, 1.0 / math.sqrt(d),
                                   self.dense_w_dtype).reshape(Sx, hs, d)
        return S.normal_stored(self.seed, S.TID_WS_DOWN, n, 1.0 / math.sqrt(hs),
                               self.dense_w_dtype).reshape(Sx, d, hs)

    def shared(self, j: int):
        Sx, hs, d = self.n_shared, self.h_shared, self.d
        n = hs * d
        g = S.normal_stored(self.seed, S.TID_WS_GATE, n, 1.0 / math.sqrt(d), self.dense_w_dtype,
                            start=j * n).reshape(hs, d)
        u = S.normal_stored(self.seed, S.TID_WS_UP, n, 1.0 / math.sqrt(d), self.dense_w_dtype,
                            start=j * n).reshape(hs, d)
        dn = S.normal_stored(self.seed, S.TID_WS_DOWN, n, 1.0 / math.sqrt(hs), self.dense_w_dtype,
                             start=j * n).reshape(d, hs)
        return g, u, dn


# ---------------------------------------------------------------------------
# The five workloads. Each is a layer shape from the pages' discussion with
# synthetic weights drawn as above.
# ---------------------------------------------------------------------------
PLANTED_ASSIGNMENT = [0] * 10 + [1] * 3 + [2] * 2 + [3]

TINY = Layer("tiny_f32_top2", T=16, d=64, h=128, N=4, k=2, act_dtype="f32",
             w_dtype="f32", router_dtype="f32", seed=0)
TINY_PLANTED = TINY.with_(name="tiny_f32_planted_top1", k=1, gate="prob",
                          planted=tuple(PLANTED_ASSIGNMENT), capacity_factor=1.0)
MCU_BATCH = Layer("mcu_t4096", T=4096, d=512, h=128, N=8, k=2,
                  router_dtype="f32", seed=1)
MCU_DECODE = MCU_BATCH.with_(name="mcu_t1", T=1)
MIXTRAL_PREFILL = Layer("mixtral_prefill_t16384", T=16384, d=4096, h=14336, N=8, k=2,
                        seed=2)
MIXTRAL_DECODE = MIXTRAL_PREFILL.with_(name="mixtral_decode_t32", T=32)
SWITCH_SKEWED = Layer("switch_top1_skewed_t16384", T=16384, d=4096, h=14336, N=8, k=1,
                      gate="prob", capacity_factor=1.25, hot_rows=(0, 1), hot_scale=6.0,
                      seed=3)
LATENT = Layer("latent_t8192", T=8192, d=4096, h=3072, N=896, k=16, act="situ",
               l=3584, n_shared=2, h_shared=3072, seed=4)

# FP8 E4M3 routed-expert weights (row-scaled), same draws as the bf16 layers.
MIXTRAL_DECODE_FP8 = MIXTRAL_DECODE.with_(name="mixtral_decode_t32_fp8", w_dtype="fp8")
MIXTRAL_PREFILL_FP8 = MIXTRAL_PREFILL.with_(name="mixtral_prefill_t16384_fp8", w_dtype="fp8")
LATENT_FP8 = LATENT.with_(name="latent_t8192_fp8", w_dtype="fp8")
# MXFP4 routed-expert weights (E2M1 in blocks of 32 with E8M0 scales): the
# Mixtral decode and prefill workloads and the LatentMoE layer.
MIXTRAL_DECODE_MXFP4 = MIXTRAL_DECODE.with_(name="mixtral_decode_t32_mxfp4", w_dtype="mxfp4")
MIXTRAL_PREFILL_MXFP4 = MIXTRAL_PREFILL.with_(name="mixtral_prefill_t16384_mxfp4",
                                              w_dtype="mxfp4")
LATENT_MXFP4 = LATENT.with_(name="latent_t8192_mxfp4", w_dtype="mxfp4")

ALL = {c.name: c for c in (TINY, TINY_PLANTED, MCU_BATCH, MCU_DECODE, MIXTRAL_PREFILL,
                           MIXTRAL_DECODE, SWITCH_SKEWED, LATENT, MIXTRAL_DECODE_FP8,
                           MIXTRAL_PREFILL_FP8, LATENT_FP8, MIXTRAL_DECODE_MXFP4,
                           MIXTRAL_PREFILL_MXFP4, LATENT_MXFP4)}
