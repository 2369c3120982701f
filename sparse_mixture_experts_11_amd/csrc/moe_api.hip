// C ABI of the MoE layer: descriptor validation, workspace layout and the
// stage sequence.  Every call validates first (no launch on error), then
// enqueues kernels on the caller's stream and returns without synchronising.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr int32_t kUnsetI32 = INT32_MIN;
constexpr int64_t kUnsetI64 = INT64_MIN;
constexpr int kMaxExperts = 1024;
constexpr int kMaxK = 32;
constexpr int kRouteWaveMaxN = 64;
constexpr uint64_t k4G = 1ull << 32;

bool unset_f(float x) { return isnan(x); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte regions of the workspace.  Offsets are relative to ws; a size of 0
// means the region is not used by this layer.
struct Layout {
  size_t idx, w, stats, part_p, part_cnt, logits;
  size_t counts, offsets, kept_offsets, perm, row_of, drop, blk_counts, tile_start;
  size_t x_l, hid, y_perm, rn, hs, ys;
  size_t qb_logits, qb_req;  // Quantile Balancing: logits [T, N], required [N, T]
  size_t rb_part;             // router backward: fp32 partial sums of dW_route
  size_t total;
};

int64_t kept_rows_bound(const moe_desc_t &d) {
  const int64_t E = d.T * d.k;
  if (d.capacity >= 0) {
    const int64_t cap = (int64_t)d.capacity * d.N;
    return cap < E ? cap : E;
  }
  return E;
}

bool is_latent(const moe_desc_t &d) { return d.l > 0; }
int xwidth(const moe_desc_t &d) { return is_latent(d) ? d.l : d.d; }
bool bf16_path(const moe_desc_t &d) { return d.act_dtype == MOE_BF16; }
// Decode kernels: at most kDecodeMaxRows tokens, and token matrices (x
// [T, w] into the gate/up, the hidden rows [R, h] into the down) within the
// kDecodeXBytes their buffer resources address; larger layers take the
// tiled GEMM.
bool decode_path(const moe_desc_t &d) {
  const int64_t w = d.l > 0 ? d.l : d.d;
  return bf16_path(d) && d.T <= kDecodeMaxRows && d.T * w * 2 < (int64_t)kDecodeXBytes &&
         kept_rows_bound(d) * (int64_t)d.h * 2 < (int64_t)kDecodeXBytes;
}
// MXFP4 expert weights: on the decode kernels (T <= 64 tokens) their
// 4-byte block-scale loads need each contraction width (the expert input
// width and h) below one 2048-wide window set or a multiple of 512; the
// tiled GEMM takes any width (multiples of 128, as validated).
bool mxfp4_ok(const moe_desc_t &d) {
  if (d.w_dtype != MOE_MXFP4) return true;
  const int w = d.l > 0 ? d.l : d.d;
  if (!bf16_path(d)) return false;
  if (!decode_path(d)) return true;
  auto width_ok = [](int k) { return k < 2048 || k % 512 == 0; };
  return width_ok(w) && width_ok(d.h);
}
bool router_gemm(const moe_desc_t &d) { return d.N > kRouteWaveMaxN; }
// The router GEMM in two K-halves (two [T, N] partial products that the
// top-k adds) when its 256 x 256 tiles would fill under three quarters of
// the 256 CUs (LatentMoE at T = 8192: 128 tiles).
bool router_split(const moe_desc_t &d) {
  const int64_t tiles = ((int64_t)d.T + 255) / 256 * (((int64_t)d.N + 255) / 256);
  return router_gemm(d) && tiles < 192 && d.d % 256 == 0 && d.d >= 512;
}
bool fp8_experts(const moe_desc_t &d) { return d.w_dtype == MOE_FP8_E4M3; }
bool mxfp4_experts(const moe_desc_t &d) { return d.w_dtype == MOE_MXFP4; }
// Routed-expert weights that come with scales.
bool scaled_experts(const moe_desc_t &d) { return fp8_experts(d) || mxfp4_experts(d); }
int weight_format(const moe_desc_t &d) {
  return fp8_experts(d) ? WFMT_FP8 : (mxfp4_experts(d) ? WFMT_MXFP4 : WFMT_BF16);
}

// Partial rows of the balance statistics the router writes for this layer.
int route_rows(const moe_desc_t &d) {
  return route_waves(d.T, d.N, d.d, d.act_dtype == MOE_BF16, d.router_dtype == MOE_BF16);
}

Layout layout(const moe_desc_t &d) {
  Layout L;
  memset(&L, 0, sizeof(L));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const int64_t E = d.T * d.k;
  const int64_t R = kept_rows_bound(d);
  const size_t act = bf16_path(d) ? 2 : 4;
  const int waves = route_rows(d);
  L.idx = take(E * 4);
  L.w = take(E * 4);
  L.stats = take((2 * (size_t)d.N + 2) * 4);
  L.part_p = take((size_t)waves * d.N * 4);
  L.part_cnt = take((size_t)waves * d.N * 4);
  L.logits = router_gemm(d) ? take((router_split(d) ? 2 : 1) * (size_t)d.T * d.N * 4) : 0;
  L.counts = take((size_t)d.N * 4);
  L.offsets = take(((size_t)d.N + 1) * 4);
  L.kept_offsets = take(((size_t)d.N + 1) * 4);
  L.perm = take(E * 4);
  L.row_of = take(E * 4);
  L.drop = take(E);
  L.blk_counts = take((size_t)dispatch_blocks(E) * d.N * 4);
  L.tile_start = take(((size_t)d.N + 1) * 4);
  if (is_latent(d)) L.x_l = take((size_t)d.T * d.l * 2);
  L.hid = take((size_t)R * d.h * act);
  L.y_perm = take((size_t)R * xwidth(d) * 4);
  if (is_latent(d)) {
    L.rn = take((size_t)d.T * d.l * 2);
    if (d.n_shared > 0) {
      L.hs = take((size_t)d.n_shared * d.T * d.h_shared * 2);
      L.ys = take((size_t)d.n_shared * d.T * d.d * 4);
    }
  }
  L.qb_logits = take((size_t)d.T * d.N * 4);
  L.qb_req = take((size_t)d.T * d.N * 4);
  L.rb_part = is_latent(d) ? 0
                           : take((size_t)route_bwd_chunks(d.T, d.N, d.d) * d.N * d.d * 4);
  L.total = off;
  return L;
}

moe_status_t validate(const moe_desc_t *dp) {
  if (dp == nullptr) return MOE_ERR_ARG;
  const moe_desc_t &d = *dp;
  // Every field must have been set.
  if (d.T == kUnsetI64 || d.d == kUnsetI32 || d.h == kUnsetI32 || d.N == kUnsetI32 ||
      d.k == kUnsetI32 || d.capacity == kUnsetI32 || d.act_dtype == kUnsetI32 ||
      d.w_dtype == kUnsetI32 || d.router_dtype == kUnsetI32 || d.gate == kUnsetI32 ||
      d.act == kUnsetI32 || unset_f(d.beta_g) || unset_f(d.beta_u) || d.l == kUnsetI32 ||
      d.n_shared == kUnsetI32 || d.h_shared == kUnsetI32 || unset_f(d.rms_eps) ||
      unset_f(d.aux_alpha))
    return MOE_ERR_ARG;
  // Ranges.
  if (d.T < 1 || d.d < 1 || d.h < 1 || d.N < 1 || d.N > kMaxExperts || d.k < 1 || d.k > d.N ||
      d.k > kMaxK || d.capacity < -1)
    return MOE_ERR_ARG;
  if ((d.act_dtype != MOE_F32 && d.act_dtype != MOE_BF16) ||
      (d.w_dtype != MOE_F32 && d.w_dtype != MOE_BF16 && d.w_dtype != MOE_FP8_E4M3 &&
       d.w_dtype != MOE_MXFP4) ||
      (d.router_dtype != MOE_F32 && d.router_dtype != MOE_BF16))
    return MOE_ERR_ARG;
  if ((d.gate != MOE_GATE_RENORM && d.gate != MOE_GATE_PROB) ||
      (d.act != MOE_ACT_SWIGLU && d.act != MOE_ACT_SITU_GLU))
    return MOE_ERR_ARG;
  if (!isfinite(d.beta_g) || !isfinite(d.beta_u) || !isfinite(d.rms_eps) ||
      !isfinite(d.aux_alpha) || d.rms_eps < 0.f)
    return MOE_ERR_ARG;
  if (d.act == MOE_ACT_SITU_GLU && (d.beta_g <= 0.f || d.beta_u <= 0.f)) return MOE_ERR_ARG;
  if (d.l < 0 || d.n_shared < 0 || d.h_shared < 0) return MOE_ERR_ARG;
  if (d.l == 0 && (d.n_shared != 0 || d.h_shared != 0)) return MOE_ERR_ARG;
  if (d.n_shared > 0 && d.h_shared < 1) return MOE_ERR_ARG;
  if (d.T * (int64_t)d.k > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;

  // What the kernels implement (no fallback path).
  // Expert weights in the activation dtype, or fp8 / MXFP4 under bf16 activations.
  if (d.act_dtype != d.w_dtype && !(scaled_experts(d) && d.act_dtype == MOE_BF16))
    return MOE_ERR_UNSUPPORTED;
  if (d.d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (d.act_dtype == MOE_F32) {
    if (d.router_dtype != MOE_F32 || d.l != 0 || router_gemm(d)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  if (router_gemm(d) && (d.router_dtype != MOE_BF16 || d.d % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  if (d.d % 128 != 0 || d.h % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t R = kept_rows_bound(d);
  if (is_latent(d)) {
    if (d.l % 128 != 0 || d.l > 4096 || d.n_shared > 2) return MOE_ERR_UNSUPPORTED;
    if (d.n_shared > 0 && d.h_shared % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if ((uint64_t)d.T * d.l * 2 >= k4G) return MOE_ERR_UNSUPPORTED;
    if ((uint64_t)d.n_shared * d.T * d.h_shared * 2 >= k4G) return MOE_ERR_UNSUPPORTED;
  }
  if (d.d > 16384) return MOE_ERR_UNSUPPORTED;
  // 32-bit buffer addressing of gathered / streamed operands.
  if ((uint64_t)d.T * d.d * 2 >= k4G || (uint64_t)R * d.h * 2 >= k4G ||
      (uint64_t)d.h * xwidth(d) * 2 >= k4G || (uint64_t)d.N * d.d * 2 >= k4G)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

template <typename T>
T *region(void *ws, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                          \
  do {                                         \
    const hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

// ---- the experts' backward: its own workspace ---------------------------------
// One group of experts: N experts of input width w and hidden h, k entries
// per token, at most R kept rows.  The plain layer's routed experts are one
// such group; the latent layer has two (routed at width l, shared at d).
int routed_bm(const moe_desc_t &d);

struct BwdDims {
  int64_t T, R;
  int N, k, w, h, act, bm;
  float bg, bu;
};

// dH and dx read W_down and W_gate | W_up either as stored (the GEMM's
// transposed-B mode) or from K-contiguous copies made first.  The copies
// cost a read and a write of every weight; the transposed-B mode costs
// about a fifth more GEMM time (measured on gfx950).  Per weight element
// that is 4 bytes of copy traffic against about 6 flops per kept row, so
// the copies pay only for experts with many rows: above 1024 rows per
// expert on average (the Mixtral prefill shape has 4096; the LatentMoE
// shape 146, where the copies would also take 59 GB of workspace).
bool bwd_weight_copies(const BwdDims &D) { return D.R > 1024ll * D.N; }

BwdDims routed_dims(const moe_desc_t &d) {
  return BwdDims{d.T, kept_rows_bound(d), d.N, d.k, xwidth(d), d.h, d.act, routed_bm(d),
                 d.beta_g, d.beta_u};
}

// The latent layer's shared experts: every token takes each of them.
BwdDims shared_dims(const moe_desc_t &d) {
  return BwdDims{d.T, d.T * d.n_shared, d.n_shared, d.n_shared, d.d, d.h_shared,
                 MOE_ACT_SWIGLU, gemm_pick_bm((double)d.T), 1.f, 1.f};
}

struct BwdLayout {
  size_t tile_start, kseg, dy_perm, g, u, dgu, dx_perm, wdt, wgut, dyt, ht, xt, dgt, dut;
  int64_t Rpad;
  size_t total;
};

BwdLayout bwd_layout(const BwdDims &D, size_t base = 0) {
  BwdLayout L;
  memset(&L, 0, sizeof(L));
  size_t off = base;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t R = (size_t)D.R, N = D.N, W = D.w, H = D.h;
  // each expert's rows padded to a multiple of 64, at least 128 (so under
  // m + 128 per expert); the total a multiple of 64
  const size_t Rpad = (R + 128 * N + 63) / 64 * 64;
  L.Rpad = (int64_t)Rpad;
  L.tile_start = take((N + 1) * 4);
  L.kseg = take((N + 1) * 4);
  L.dy_perm = take(R * W * 2);
  L.g = take(R * H * 2);
  L.u = take(R * H * 2);
  L.dgu = take(R * 2 * H * 2);
  L.dx_perm = take(R * W * 4);
  if (bwd_weight_copies(D)) {
    L.wdt = take(N * H * W * 2);
    L.wgut = take(N * W * 2 * H * 2);
  }
  L.dyt = take(W * Rpad * 2);
  L.ht = take(H * Rpad * 2);
  L.xt = take(W * Rpad * 2);
  L.dgt = take(H * Rpad * 2);
  L.dut = take(H * Rpad * 2);
  L.total = off - base;
  return L;
}

// 32-bit offsets into the group's transposed and row-major operands.
bool bwd_dims_ok(const BwdDims &D) {
  const uint64_t R = (uint64_t)D.R, Rpad = (R + 128ull * D.N + 63) / 64 * 64;
  const uint64_t wmax = (uint64_t)(D.w > D.h ? D.w : D.h);
  return wmax * Rpad * 2 < k4G && R * 2ull * D.h * 2 < k4G && 2ull * D.h * D.w * 2 < k4G &&
         R * (uint64_t)D.w * 4 < k4G;
}

// What the backward supports: bf16 activations, bf16 expert weights (and a
// bf16 router for the latent layer, whose router backward runs here too),
// 32-bit offsets into its transposed operands.
moe_status_t bwd_supported(const moe_desc_t &d) {
  if (d.act_dtype != MOE_BF16 || d.w_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!bwd_dims_ok(routed_dims(d))) return MOE_ERR_UNSUPPORTED;
  if (is_latent(d)) {
    if (d.router_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d.n_shared > 0 && !bwd_dims_ok(shared_dims(d))) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// ---- stages (no validation; callers validated) ------------------------------

hipError_t do_route(const moe_desc_t &d, const Layout &L, const void *u, const void *W_route,
                    const float *bias, int32_t *idx, float *w, float *stats, void *ws,
                    hipStream_t st) {
  float *pp = region<float>(ws, L.part_p);
  int32_t *pc = region<int32_t>(ws, L.part_cnt);
  hipError_t e;
  if (router_gemm(d)) {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = static_cast<const uint16_t *>(u);
    a.lda = d.d;
    a.B = static_cast<const uint16_t *>(W_route);
    a.K = d.d;
    a.ncols = d.N;
    a.mode = GM_DENSE;
    a.G = 1;
    a.M_dense = d.T;
    a.out = region<float>(ws, L.logits);
    a.ldo = d.N;
    const bool split = router_split(d);
    if (split) {
      a.G = 2;
      a.kchunk = d.d / 2;
      a.ldb = d.d;
      a.out_group_stride = d.T;
    }
    e = launch_gemm(a, EP_F32, 0, st);
    if (e != hipSuccess) return e;
    const float *z = region<float>(ws, L.logits);
    e = launch_topk_logits(z, split ? z + (size_t)d.T * d.N : nullptr, d.T, d.N, d.k, d.gate, bias,
                           idx, w, pp, pc, st);
  } else {
    e = launch_route_wave(u, d.act_dtype == MOE_BF16, W_route, d.router_dtype == MOE_BF16, d.T,
                          d.d, d.N, d.k, d.gate, bias, idx, w, pp, pc, st);
  }
  if (e != hipSuccess || stats == nullptr) return e;
  return launch_stats_finalize(pp, pc, route_rows(d), d.T, d.N, d.aux_alpha, stats, st);
}

// At most 1024 (token, slot) entries: one single-block launch does the
// dispatch, and inside a forward also the balance statistics the router
// left as partial rows (the router then skips its own two-launch finish).
bool small_tail(const moe_desc_t &d) { return small_tail_fits(d.T * d.k, d.N); }

// stats != nullptr only when the router deferred its statistics to here.
hipError_t do_dispatch(const moe_desc_t &d, const Layout &L, const int32_t *idx, int32_t *counts,
                       int32_t *offsets, int32_t *kept_offsets, int32_t *perm, int32_t *row_of,
                       uint8_t *drop, float *stats, void *ws, hipStream_t st) {
  if (small_tail(d))
    return launch_small_tail(region<float>(ws, L.part_p), region<int32_t>(ws, L.part_cnt),
                             route_rows(d), d.T, d.aux_alpha, stats, idx, d.k, d.N,
                             d.capacity, counts, offsets, kept_offsets, perm, row_of, drop, st);
  return launch_dispatch(idx, d.T, d.k, d.N, d.capacity, counts, offsets, kept_offsets, perm,
                         row_of, drop, region<int32_t>(ws, L.blk_counts),
                         region<float>(ws, L.part_p), region<int32_t>(ws, L.part_cnt),
                         route_rows(d), d.aux_alpha, stats, st);
}

// Expert-projection kernel family for a layer: fp32 on the vector ALUs,
// decode-sized T streams the selected experts' weights, otherwise the tiled
// grouped GEMM.
enum FfnPath { FFN_SIMT, FFN_DECODE, FFN_TILED };

FfnPath ffn_path(const moe_desc_t &d) {
  if (!bf16_path(d)) return FFN_SIMT;
  if (decode_path(d)) return FFN_DECODE;
  return FFN_TILED;
}

// m-tile height of the routed expert GEMMs, from the mean kept rows per
// expert (known on the host without waiting for the routing).
int routed_bm(const moe_desc_t &d) {
  return gemm_pick_bm((double)kept_rows_bound(d) / (double)d.N);
}

// The tiled path finds its work from a per-expert prefix of m-tiles.
hipError_t do_tile_prefix(const moe_desc_t &d, const Layout &L, const int32_t *kept_offsets,
                          void *ws, hipStream_t st) {
  if (ffn_path(d) != FFN_TILED) return hipSuccess;
  return launch_tile_prefix(kept_offsets, d.N, routed_bm(d), region<int32_t>(ws, L.tile_start),
                            st);
}

// sg, su, sd: fp8 row scales or MXFP4 block scales (null for bf16 / fp32).
// gate_up: null, or [R, 2h] bf16 rows receiving G | U as well (tiled path,
// bf16 weights; validated by the caller).
hipError_t do_ffn_gate_up(const moe_desc_t &d, const Layout &L, const void *x, const int32_t *perm,
                          const int32_t *offsets, const int32_t *kept_offsets, const void *Wg,
                          const void *Wu, const void *sg, const void *su, void *ws,
                          hipStream_t st, void *gate_up = nullptr) {
  const int w = xwidth(d);
  if (!bf16_path(d))
    return launch_simt_gu(static_cast<const float *>(x), perm, offsets, kept_offsets, d.k,
                          static_cast<const float *>(Wg), static_cast<const float *>(Wu), w, d.h,
                          d.N, d.act, d.beta_g, d.beta_u, region<float>(ws, L.hid), st);
  if (decode_path(d))
    return launch_decode_gu(static_cast<const uint16_t *>(x), d.T, w, perm, offsets, kept_offsets,
                            d.k, Wg, Wu, sg, su, weight_format(d), d.h, d.N, d.act, d.beta_g,
                            d.beta_u, region<uint16_t>(ws, L.hid), st);
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = static_cast<const uint16_t *>(x);
  a.lda = w;
  a.B = Wg;
  a.B2 = Wu;
  a.bscale = static_cast<const float *>(sg);
  a.bscale2 = static_cast<const float *>(su);
  a.mx4 = mxfp4_experts(d) ? 1 : 0;
  a.strideB = (int64_t)d.h * w;
  a.K = w;
  a.ncols = d.h;
  a.mode = GM_GATHER;
  a.G = d.N;
  a.kslots = d.k;
  a.perm = perm;
  a.offsets = offsets;
  a.kept_offsets = kept_offsets;
  a.tile_start = region<int32_t>(ws, L.tile_start);
  a.out = region<uint16_t>(ws, L.hid);
  a.ldo = d.h;
  a.act = d.act;
  a.beta_g = d.beta_g;
  a.beta_u = d.beta_u;
  a.bm = routed_bm(d);
  if (gate_up != nullptr) {
    a.out2 = gate_up;
    a.ldg = 2 * (int64_t)d.h;
  }
  return launch_gemm(a, gate_up != nullptr ? EP_GLU_SAVE : EP_GLU,
                     gemm_mtile_bound(kept_rows_bound(d), d.N, a.bm), st);
}

hipError_t do_ffn_down(const moe_desc_t &d, const Layout &L, const int32_t *kept_offsets,
                       const void *Wd, const void *sd, float *y_perm, void *ws, hipStream_t st) {
  const int w = xwidth(d);
  if (!bf16_path(d))
    return launch_simt_down(region<float>(ws, L.hid), kept_offsets,
                            static_cast<const float *>(Wd), d.h, w, d.N, y_perm, st);
  if (decode_path(d))
    return launch_decode_down(region<uint16_t>(ws, L.hid), d.T, kept_offsets, Wd, sd,
                              weight_format(d), d.h, w, d.N, y_perm, st);
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = region<uint16_t>(ws, L.hid);
  a.lda = d.h;
  a.B = Wd;
  a.bscale = static_cast<const float *>(sd);
  a.mx4 = mxfp4_experts(d) ? 1 : 0;
  a.strideB = (int64_t)w * d.h;
  a.K = d.h;
  a.ncols = w;
  a.mode = GM_SEGMENT;
  a.G = d.N;
  a.kept_offsets = kept_offsets;
  a.tile_start = region<int32_t>(ws, L.tile_start);
  a.out = y_perm;
  a.ldo = w;
  a.bm = routed_bm(d);
  return launch_gemm(a, EP_F32, gemm_mtile_bound(kept_rows_bound(d), d.N, a.bm), st);
}

// Dense (one or few groups) projection: out[g*T + r] = A[g*a_rows + r] . B_g
hipError_t dense_gemm(const uint16_t *A, int64_t lda, int64_t a_group_rows, const uint16_t *B,
                      const uint16_t *B2, int64_t strideB, int K, int ncols, int G, int64_t M,
                      void *out, int64_t ldo, int epi, const float *add0, const float *add1,
                      int act, hipStream_t st) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = A;
  a.lda = lda;
  a.a_group_rows = a_group_rows;
  a.B = B;
  a.B2 = B2;
  a.strideB = strideB;
  a.K = K;
  a.ncols = ncols;
  a.mode = GM_DENSE;
  a.G = G;
  a.M_dense = M;
  a.out = out;
  a.ldo = ldo;
  a.out_group_stride = M;
  a.add0 = add0;
  a.add1 = add1;
  a.act = act;
  a.beta_g = 1.f;
  a.beta_u = 1.f;
  return launch_gemm(a, epi, 0, st);
}

struct Tracer {
  void *const *ev;
  int n;
  int next;
  hipStream_t st;
  hipError_t mark() {
    if (next < n) {
      const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(ev[next]), st);
      ++next;
      return e;
    }
    return hipSuccess;
  }
};

const char *const kPlainStages[] = {"route", "dispatch", "expert_gate_up", "expert_down",
                                    "combine"};
const char *const kLatentStages[] = {"route",         "dispatch",        "latent_down_proj",
                                     "expert_gate_up", "expert_down",     "combine_rmsnorm",
                                     "shared_gate_up", "shared_down",     "latent_up_proj"};

moe_status_t forward_impl(const moe_desc_t *desc, const moe_weights_t *wts, const void *u, void *y,
                          const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t st,
                          void *const *events, int n_events) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  const moe_desc_t &d = *desc;
  if (wts == nullptr || u == nullptr || y == nullptr || wts->W_route == nullptr ||
      wts->W_gate == nullptr || wts->W_up == nullptr || wts->W_down == nullptr)
    return MOE_ERR_ARG;
  if (is_latent(d) && (wts->W_ldown == nullptr || wts->W_lup == nullptr)) return MOE_ERR_ARG;
  // Scales: all three with fp8 / MXFP4 expert weights, none otherwise.
  const bool any_scale = wts->gate_scale || wts->up_scale || wts->down_scale;
  const bool all_scales = wts->gate_scale && wts->up_scale && wts->down_scale;
  if (scaled_experts(d) ? !all_scales : any_scale) return MOE_ERR_ARG;
  if (!mxfp4_ok(d)) return MOE_ERR_UNSUPPORTED;
  if (is_latent(d) && d.n_shared > 0 &&
      (wts->Ws_gate == nullptr || wts->Ws_up == nullptr || wts->Ws_down == nullptr))
    return MOE_ERR_ARG;
  const Layout L = layout(d);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (n_events > 0 && events == nullptr) return MOE_ERR_ARG;

  moe_outputs_t o;
  memset(&o, 0, sizeof(o));
  if (out != nullptr) o = *out;
  // Saved gate/up sums come from the tiled GEMM's epilogue (bf16 weights).
  if (o.gate_up != nullptr && (ffn_path(d) != FFN_TILED || d.w_dtype != MOE_BF16))
    return MOE_ERR_UNSUPPORTED;
  int32_t *idx = o.topk_idx ? o.topk_idx : region<int32_t>(ws, L.idx);
  float *tw = o.topk_w ? o.topk_w : region<float>(ws, L.w);
  float *stats = o.stats ? o.stats : region<float>(ws, L.stats);
  int32_t *counts = o.counts ? o.counts : region<int32_t>(ws, L.counts);
  int32_t *offsets = o.offsets ? o.offsets : region<int32_t>(ws, L.offsets);
  int32_t *kept_offsets = o.kept_offsets ? o.kept_offsets : region<int32_t>(ws, L.kept_offsets);
  int32_t *perm = o.perm ? o.perm : region<int32_t>(ws, L.perm);
  int32_t *row_of = o.row_of ? o.row_of : region<int32_t>(ws, L.row_of);
  uint8_t *drop = o.drop ? o.drop : region<uint8_t>(ws, L.drop);
  float *y_perm = o.y_perm ? o.y_perm : region<float>(ws, L.y_perm);

  Tracer tr{events, n_events, 0, st};
  MOE_TRY(tr.mark());
  // The dispatch launches finish the balance statistics from the router's
  // partial rows.
  MOE_TRY(do_route(d, L, u, wts->W_route, wts->selection_bias, idx, tw, nullptr, ws, st));
  MOE_TRY(tr.mark());
  MOE_TRY(do_dispatch(d, L, idx, counts, offsets, kept_offsets, perm, row_of, drop, stats, ws,
                      st));
  MOE_TRY(do_tile_prefix(d, L, kept_offsets, ws, st));
  MOE_TRY(tr.mark());
  const void *x = u;
  if (is_latent(d)) {
    uint16_t *xl = region<uint16_t>(ws, L.x_l);
    MOE_TRY(dense_gemm(static_cast<const uint16_t *>(u), d.d, 0,
                       static_cast<const uint16_t *>(wts->W_ldown), nullptr, 0, d.d, d.l, 1, d.T,
                       xl, d.l, EP_BF16, nullptr, nullptr, 0, st));
    MOE_TRY(tr.mark());
    x = xl;
  }
  MOE_TRY(do_ffn_gate_up(d, L, x, perm, offsets, kept_offsets, wts->W_gate, wts->W_up,
                         wts->gate_scale, wts->up_scale, ws, st, o.gate_up));
  MOE_TRY(tr.mark());
  MOE_TRY(do_ffn_down(d, L, kept_offsets, wts->W_down, wts->down_scale, y_perm, ws, st));
  MOE_TRY(tr.mark());
  if (!is_latent(d)) {
    MOE_TRY(launch_combine(y_perm, row_of, tw, d.T, d.k, d.d, bf16_path(d), false, 0.f, y, st));
    MOE_TRY(tr.mark());
  } else {
    uint16_t *rn = region<uint16_t>(ws, L.rn);
    MOE_TRY(launch_combine(y_perm, row_of, tw, d.T, d.k, d.l, true, true, d.rms_eps, rn, st));
    MOE_TRY(tr.mark());
    const float *add0 = nullptr, *add1 = nullptr;
    if (d.n_shared > 0) {
      uint16_t *hs = region<uint16_t>(ws, L.hs);
      float *ys = region<float>(ws, L.ys);
      MOE_TRY(dense_gemm(static_cast<const uint16_t *>(u), d.d, 0,
                         static_cast<const uint16_t *>(wts->Ws_gate),
                         static_cast<const uint16_t *>(wts->Ws_up), (int64_t)d.h_shared * d.d, d.d,
                         d.h_shared, d.n_shared, d.T, hs, d.h_shared, EP_GLU, nullptr, nullptr,
                         MOE_ACT_SWIGLU, st));
      MOE_TRY(tr.mark());
      MOE_TRY(dense_gemm(hs, d.h_shared, d.T, static_cast<const uint16_t *>(wts->Ws_down), nullptr,
                         (int64_t)d.d * d.h_shared, d.h_shared, d.d, d.n_shared, d.T, ys, d.d,
                         EP_F32, nullptr, nullptr, 0, st));
      MOE_TRY(tr.mark());
      add0 = ys;
      add1 = d.n_shared > 1 ? ys + (int64_t)d.T * d.d : nullptr;
    } else {
      MOE_TRY(tr.mark());
      MOE_TRY(tr.mark());
    }
    MOE_TRY(dense_gemm(rn, d.l, 0, static_cast<const uint16_t *>(wts->W_lup), nullptr, 0, d.l, d.d,
                       1, d.T, y, d.d, add0 ? EP_ADD_BF16 : EP_BF16, add0, add1, 0, st));
    MOE_TRY(tr.mark());
  }
  while (tr.next < tr.n) MOE_TRY(tr.mark());
  return MOE_OK;
}

// The experts' backward for one group of experts (see BwdDims): dx [T, w]
// fp32 (written, not accumulated) and, when dWg is not null, the three weight
// gradients.  L's regions are offsets into ws.
// gate_up: the forward's saved [G | U] rows ([R, 2h] bf16), or null to
// recompute them.
hipError_t experts_bwd_core(const BwdDims &D, const BwdLayout &L, void *ws, const uint16_t *x,
                            const uint16_t *Wg, const uint16_t *Wu, const uint16_t *Wd,
                            const float *topk_w, const int32_t *offsets,
                            const int32_t *kept_offsets, const int32_t *perm,
                            const int32_t *row_of, const uint16_t *gate_up, const uint16_t *dy,
                            float *dx, float *dWg, float *dWu, float *dWd, hipStream_t st) {
  const int bm = D.bm;
  const int64_t mt = gemm_mtile_bound(D.R, D.N, bm);
  int32_t *tile_start = region<int32_t>(ws, L.tile_start);
  uint16_t *dy_perm = region<uint16_t>(ws, L.dy_perm);
  const uint16_t *G = gate_up ? gate_up : region<uint16_t>(ws, L.g);
  const uint16_t *U = gate_up ? gate_up + D.h : region<uint16_t>(ws, L.u);
  const int64_t ldgu = gate_up ? 2 * (int64_t)D.h : (int64_t)D.h;
  uint16_t *dgu = region<uint16_t>(ws, L.dgu);
  float *dx_perm = region<float>(ws, L.dx_perm);
  const int64_t W = D.w, H = D.h;
  hipError_t e;
#define MOE_BWD_TRY(expr)              \
  do {                                 \
    e = (expr);                        \
    if (e != hipSuccess) return e;     \
  } while (0)
  MOE_BWD_TRY(launch_tile_prefix(kept_offsets, D.N, bm, tile_start, st));
  // dY = a dy_t per kept row.
  MOE_BWD_TRY(launch_bwd_gather_dy(dy, D.T, D.w, D.k, row_of, topk_w, dy_perm, st));
  // G, U recomputed (bf16) unless the forward kept them.
  if (gate_up == nullptr) {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = x;
    a.lda = W;
    a.B = Wg;
    a.B2 = Wu;
    a.strideB = H * W;
    a.K = D.w;
    a.ncols = D.h;
    a.mode = GM_GATHER;
    a.G = D.N;
    a.kslots = D.k;
    a.perm = perm;
    a.offsets = offsets;
    a.kept_offsets = kept_offsets;
    a.tile_start = tile_start;
    a.out = region<uint16_t>(ws, L.g);
    a.out2 = region<uint16_t>(ws, L.u);
    a.ldo = H;
    a.bm = bm;
    MOE_BWD_TRY(launch_gemm(a, EP_GU, mt, st));
  }
  // W_down and W_gate | W_up as the K-contiguous operands of dH and dx:
  // copies [N][h][w] and [N][w][2h], or the weights as stored.
  const bool copies = bwd_weight_copies(D);
  uint16_t *wdt = copies ? region<uint16_t>(ws, L.wdt) : nullptr;
  uint16_t *wgut = copies ? region<uint16_t>(ws, L.wgut) : nullptr;
  if (copies) {
    MOE_BWD_TRY(launch_transpose_bf16(Wd, D.N, D.w, D.h, wdt, W, 0, st));
    MOE_BWD_TRY(launch_transpose_bf16(Wg, D.N, D.h, D.w, wgut, 2 * H, 0, st));
    MOE_BWD_TRY(launch_transpose_bf16(Wu, D.N, D.h, D.w, wgut, 2 * H, D.h, st));
  }
  // dH = W_down^T dY, and in the epilogue (dG, dU) = act'(G, U) dH.
  {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = dy_perm;
    a.lda = W;
    if (copies) {
      a.B = wdt;
    } else {
      a.B = Wd;
      a.bt = 1;
      a.ldbt = H;
    }
    a.strideB = H * W;
    a.K = D.w;
    a.ncols = D.h;
    a.mode = GM_SEGMENT;
    a.G = D.N;
    a.kept_offsets = kept_offsets;
    a.tile_start = tile_start;
    a.out = dgu;
    a.out2 = dgu + H;
    a.ldo = 2 * H;
    a.gsrc = G;
    a.usrc = U;
    a.ldg = ldgu;
    a.act = D.act;
    a.beta_g = D.bg;
    a.beta_u = D.bu;
    a.bm = bm;
    MOE_BWD_TRY(launch_gemm(a, EP_GLU_BWD, mt, st));
  }
  // dx rows = [dG | dU] [W_gate ; W_up], then summed per token.
  {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = dgu;
    a.lda = 2 * H;
    if (copies) {
      a.B = wgut;
      a.strideB = W * 2 * H;
    } else {
      a.B = Wg;
      a.B2 = Wu;
      a.bt = 1;
      a.ldbt = W;
      a.ksplit = D.h;
      a.strideB = W * H;
    }
    a.K = 2 * D.h;
    a.ncols = D.w;
    a.mode = GM_SEGMENT;
    a.G = D.N;
    a.kept_offsets = kept_offsets;
    a.tile_start = tile_start;
    a.out = dx_perm;
    a.ldo = W;
    a.bm = bm;
    MOE_BWD_TRY(launch_gemm(a, EP_F32, mt, st));
  }
  MOE_BWD_TRY(launch_rows_sum(dx_perm, D.T, D.w, D.k, row_of, dx, st));
  if (dWg == nullptr) return hipSuccess;
  // Weight gradients: per-expert K segments over the expert's own rows.
  int32_t *kseg = region<int32_t>(ws, L.kseg);
  uint16_t *dyt = region<uint16_t>(ws, L.dyt), *ht = region<uint16_t>(ws, L.ht);
  uint16_t *xt = region<uint16_t>(ws, L.xt), *dgt = region<uint16_t>(ws, L.dgt);
  uint16_t *dut = region<uint16_t>(ws, L.dut);
  const int64_t Rp = L.Rpad;
  MOE_BWD_TRY(launch_kseg(kept_offsets, D.N, kseg, st));
  MOE_BWD_TRY(launch_seg_transpose(dy_perm, nullptr, W, D.w, kept_offsets, offsets, nullptr, D.k,
                                   kseg, D.N, 0, 1.f, 1.f, dyt, Rp, st));
  MOE_BWD_TRY(launch_seg_transpose(G, U, ldgu, D.h, kept_offsets, offsets, nullptr, D.k, kseg,
                                   D.N, D.act, D.bg, D.bu, ht, Rp, st));
  MOE_BWD_TRY(launch_seg_transpose(x, nullptr, W, D.w, kept_offsets, offsets, perm, D.k, kseg,
                                   D.N, 0, 1.f, 1.f, xt, Rp, st));
  MOE_BWD_TRY(launch_seg_transpose(dgu, nullptr, 2 * H, D.h, kept_offsets, offsets, nullptr, D.k,
                                   kseg, D.N, 0, 1.f, 1.f, dgt, Rp, st));
  MOE_BWD_TRY(launch_seg_transpose(dgu + H, nullptr, 2 * H, D.h, kept_offsets, offsets, nullptr,
                                   D.k, kseg, D.N, 0, 1.f, 1.f, dut, Rp, st));
  auto kseg_gemm = [&](const uint16_t *A, int M, const uint16_t *B, int ncols, float *out) {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = A;
    a.lda = Rp;
    a.B = B;
    a.strideB = 0;
    a.K = 128;  // the k range comes from kseg
    a.ncols = ncols;
    a.mode = GM_DENSE;
    a.G = D.N;
    a.M_dense = M;
    a.a_group_rows = 0;
    a.out = out;
    a.ldo = ncols;
    a.out_group_stride = M;
    a.kseg = kseg;
    a.ldb = Rp;
    a.bm = 256;
    return launch_gemm(a, EP_F32, 0, st);
  };
  MOE_BWD_TRY(kseg_gemm(dyt, D.w, ht, D.h, dWd));
  MOE_BWD_TRY(kseg_gemm(dgt, D.h, xt, D.w, dWg));
  MOE_BWD_TRY(kseg_gemm(dut, D.h, xt, D.w, dWu));
#undef MOE_BWD_TRY
  return hipSuccess;
}

// ---- the latent layer's backward: its workspace ---------------------------------
// The experts' regions (sized for the larger of the routed and shared
// groups, used by one then the other) come first, then the latent steps'.
struct LatBwdLayout {
  size_t core;                                 // experts' regions, at offset 0
  size_t xl, dn, dr, nb, wlupt, wldt, dyt, nt;  // latent steps
  size_t dxl, dxlb, dxlt, ut, tmp, logits, rb_part;
  size_t sh_w, sh_perm, sh_row, sh_off, sh_koff;
  int64_t Tp;  // T padded: the K of the T-long contractions
  size_t total;
};

LatBwdLayout lat_bwd_layout(const moe_desc_t &d) {
  LatBwdLayout L;
  memset(&L, 0, sizeof(L));
  size_t core = bwd_layout(routed_dims(d)).total;
  if (d.n_shared > 0) {
    const size_t cs = bwd_layout(shared_dims(d)).total;
    if (cs > core) core = cs;
  }
  L.core = core;
  size_t off = align256(core);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t T = (size_t)d.T, l = (size_t)d.l, D = (size_t)d.d, S = (size_t)d.n_shared;
  const int64_t Tp = ((d.T + 63) / 64) * 64;
  L.Tp = Tp < 128 ? 128 : Tp;
  const size_t tp = (size_t)L.Tp;
  L.xl = take(T * l * 2);
  L.dn = take(T * l * 4);
  L.dr = take(T * l * 2);
  L.nb = take(T * l * 2);
  L.wlupt = take(l * D * 2);
  L.wldt = take(D * l * 2);
  L.dyt = take(D * tp * 2);
  L.nt = take(l * tp * 2);
  L.dxl = take(T * l * 4);
  L.dxlb = take(T * l * 2);
  L.dxlt = take(l * tp * 2);
  L.ut = take(D * tp * 2);
  L.tmp = take(T * D * 4);
  L.logits = take(T * (size_t)d.N * 4);
  L.rb_part = take((size_t)route_bwd_chunks(d.T, d.N, d.d) * d.N * d.d * 4);
  L.sh_w = take(T * S * 4);
  L.sh_perm = take(T * S * 4);
  L.sh_row = take(T * S * 4);
  L.sh_off = take((S + 1) * 4);
  L.sh_koff = take((S + 1) * 4);
  L.total = off;
  return L;
}

}  // namespace

// ---- the static scratch of moe_forward_noalloc ------------------------------
// One array per GPU, created with the code object on each device.  In host
// code its name only stands in for the symbol: the device address of a
// device's copy comes from hipGetSymbolAddress with that device current,
// looked up on the first call on the device and kept per device.  Nothing in
// the forward reads a workspace byte it has not written earlier in the same
// call (its histograms are LDS integer atomics, every partial row and
// dispatch array is written whole), so the array needs no clearing.
__device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the device that runs `st`.
moe_status_t static_scratch(hipStream_t st, void **ptr) {
  int dev = -1;
  if (st != nullptr) {
    if (hipStreamGetDevice(st, &dev) != hipSuccess) return MOE_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

void moe_desc_init(moe_desc_t *d) {
  if (d == nullptr) return;
  d->T = kUnsetI64;
  d->d = d->h = d->N = d->k = d->capacity = kUnsetI32;
  d->act_dtype = d->w_dtype = d->router_dtype = d->gate = d->act = kUnsetI32;
  d->beta_g = d->beta_u = NAN;
  d->l = d->n_shared = d->h_shared = kUnsetI32;
  d->rms_eps = NAN;
  d->aux_alpha = NAN;
}

const char *moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "layer not supported by these kernels";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

moe_status_t moe_workspace_bytes(const moe_desc_t *desc, size_t *bytes) {
  if (bytes == nullptr) return MOE_ERR_ARG;
  *bytes = 0;
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  *bytes = layout(*desc).total;
  return MOE_OK;
}

int32_t moe_capacity_from_factor(int64_t T, int32_t N, int32_t k, double c) {
  if (T < 1 || N < 1 || k < 1 || !isfinite(c) || c <= 0.0) return -1;
  const double v = ceil((c * (double)k * (double)T) / (double)N);
  if (v > (double)INT32_MAX) return -1;
  return (int32_t)v;
}

moe_status_t moe_route_biased(const moe_desc_t *desc, const void *u, const void *W_route,
                              const float *bias, int32_t *topk_idx, float *topk_w,
                              float *stats, void *ws, size_t ws_bytes, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  if (u == nullptr || W_route == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return MOE_ERR_ARG;
  const Layout L = layout(*desc);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return hip_status(do_route(*desc, L, u, W_route, bias, topk_idx, topk_w, stats, ws,
                             reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_route(const moe_desc_t *desc, const void *u, const void *W_route,
                       int32_t *topk_idx, float *topk_w, float *stats, void *ws, size_t ws_bytes,
                       moe_stream_t stream) {
  return moe_route_biased(desc, u, W_route, nullptr, topk_idx, topk_w, stats, ws, ws_bytes,
                          stream);
}

moe_status_t moe_qb_update(const moe_desc_t *desc, const void *u, const void *W_route,
                           const float *bias, int32_t q, int32_t method, float *new_bias,
                           void *ws, size_t ws_bytes, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  const moe_desc_t &d = *desc;
  if (u == nullptr || W_route == nullptr || new_bias == nullptr) return MOE_ERR_ARG;
  if (method != 0 && method != 1) return MOE_ERR_ARG;
  if (q > d.T) return MOE_ERR_ARG;
  // The logits come from the bf16 MFMA GEMM (d is a multiple of 128 here).
  if (d.act_dtype != MOE_BF16 || d.router_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const Layout L = layout(d);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  // q <= 0: round(k T / N) = floor((2 k T + N) / (2 N)), clamped to [1, T].
  int64_t qq = q;
  if (qq <= 0) {
    qq = (2 * (int64_t)d.k * d.T + d.N) / (2 * (int64_t)d.N);
    if (qq < 1) qq = 1;
    if (qq > d.T) qq = d.T;
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float *logits = region<float>(ws, L.qb_logits);
  MOE_TRY(dense_gemm(static_cast<const uint16_t *>(u), d.d, 0,
                     static_cast<const uint16_t *>(W_route), nullptr, 0, d.d, d.N, 1, d.T, logits,
                     d.N, EP_F32, nullptr, nullptr, 0, st));
  return hip_status(launch_qb_update(logits, d.T, d.N, d.k, bias, (int)qq, method,
                                     region<float>(ws, L.qb_req), new_bias, st));
}

moe_status_t moe_backward_workspace_bytes(const moe_desc_t *desc, size_t *bytes) {
  if (bytes == nullptr) return MOE_ERR_ARG;
  *bytes = 0;
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  const moe_status_t s = bwd_supported(*desc);
  if (s != MOE_OK) return s;
  *bytes = is_latent(*desc) ? lat_bwd_layout(*desc).total : bwd_layout(routed_dims(*desc)).total;
  return MOE_OK;
}

moe_status_t moe_experts_backward(const moe_desc_t *desc, const moe_weights_t *wts, const void *u,
                                  const float *topk_w, const int32_t *offsets,
                                  const int32_t *kept_offsets, const int32_t *perm,
                                  const int32_t *row_of, const void *gate_up, const void *dy,
                                  float *dx, float *dW_gate, float *dW_up, float *dW_down,
                                  void *ws, size_t ws_bytes, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  const moe_desc_t &d = *desc;
  if (wts == nullptr || wts->W_gate == nullptr || wts->W_up == nullptr ||
      wts->W_down == nullptr || u == nullptr || topk_w == nullptr || offsets == nullptr ||
      kept_offsets == nullptr || perm == nullptr || row_of == nullptr || dy == nullptr ||
      dx == nullptr)
    return MOE_ERR_ARG;
  const bool any_w = dW_gate || dW_up || dW_down, all_w = dW_gate && dW_up && dW_down;
  if (any_w && !all_w) return MOE_ERR_ARG;
  if (is_latent(d)) return MOE_ERR_UNSUPPORTED;  // moe_latent_backward
  const moe_status_t s = bwd_supported(d);
  if (s != MOE_OK) return s;
  const BwdDims D = routed_dims(d);
  const BwdLayout L = bwd_layout(D);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return hip_status(experts_bwd_core(
      D, L, ws, static_cast<const uint16_t *>(u), static_cast<const uint16_t *>(wts->W_gate),
      static_cast<const uint16_t *>(wts->W_up), static_cast<const uint16_t *>(wts->W_down), topk_w,
      offsets, kept_offsets, perm, row_of, static_cast<const uint16_t *>(gate_up),
      static_cast<const uint16_t *>(dy), dx, dW_gate, dW_up, dW_down,
      reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_latent_backward(const moe_desc_t *desc, const moe_weights_t *wts, const void *u,
                                 const moe_outputs_t *fwd, const void *dy, float aux_scale,
                                 const moe_latent_grads_t *g, void *ws, size_t ws_bytes,
                                 moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  const moe_desc_t &d = *desc;
  if (!is_latent(d)) return MOE_ERR_UNSUPPORTED;  // moe_route_backward + moe_experts_backward
  if (wts == nullptr || u == nullptr || fwd == nullptr || dy == nullptr || g == nullptr)
    return MOE_ERR_ARG;
  if (wts->W_route == nullptr || wts->W_gate == nullptr || wts->W_up == nullptr ||
      wts->W_down == nullptr || wts->W_ldown == nullptr || wts->W_lup == nullptr)
    return MOE_ERR_ARG;
  if (d.n_shared > 0 &&
      (wts->Ws_gate == nullptr || wts->Ws_up == nullptr || wts->Ws_down == nullptr))
    return MOE_ERR_ARG;
  if (fwd->topk_idx == nullptr || fwd->topk_w == nullptr || fwd->stats == nullptr ||
      fwd->offsets == nullptr || fwd->kept_offsets == nullptr || fwd->perm == nullptr ||
      fwd->row_of == nullptr || fwd->y_perm == nullptr)
    return MOE_ERR_ARG;
  if (g->du == nullptr || g->dz == nullptr || g->dW_route == nullptr || g->dW_ldown == nullptr ||
      g->dW_lup == nullptr || g->dW_gate == nullptr || g->dW_up == nullptr ||
      g->dW_down == nullptr)
    return MOE_ERR_ARG;
  if (d.n_shared > 0 && (g->dWs_gate == nullptr || g->dWs_up == nullptr || g->dWs_down == nullptr))
    return MOE_ERR_ARG;
  if (!isfinite(aux_scale)) return MOE_ERR_ARG;
  const moe_status_t s = bwd_supported(d);
  if (s != MOE_OK) return s;
  const LatBwdLayout L = lat_bwd_layout(d);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t *U = static_cast<const uint16_t *>(u);
  const uint16_t *DY = static_cast<const uint16_t *>(dy);
  const uint16_t *Wldown = static_cast<const uint16_t *>(wts->W_ldown);
  const uint16_t *Wlup = static_cast<const uint16_t *>(wts->W_lup);
  const int64_t T = d.T, Tp = L.Tp;
  const int l = d.l, D = d.d;
  uint16_t *xl = region<uint16_t>(ws, L.xl), *dr = region<uint16_t>(ws, L.dr);
  uint16_t *nb = region<uint16_t>(ws, L.nb), *wlupt = region<uint16_t>(ws, L.wlupt);
  uint16_t *wldt = region<uint16_t>(ws, L.wldt), *dyt = region<uint16_t>(ws, L.dyt);
  uint16_t *nt = region<uint16_t>(ws, L.nt), *dxlb = region<uint16_t>(ws, L.dxlb);
  uint16_t *dxlt = region<uint16_t>(ws, L.dxlt), *ut = region<uint16_t>(ws, L.ut);
  float *dn = region<float>(ws, L.dn), *dxl = region<float>(ws, L.dxl);
  float *tmp = region<float>(ws, L.tmp), *logits = region<float>(ws, L.logits);
  // x_l = W_ldown u, recomputed as the forward rounded it.
  MOE_TRY(dense_gemm(U, D, 0, Wldown, nullptr, 0, D, l, 1, T, xl, l, EP_BF16, nullptr, nullptr, 0,
                     st));
  // dn = dy W_lup (W_lup^T as the K-contiguous operand), then dr and n.
  MOE_TRY(launch_transpose_bf16(Wlup, 1, D, l, wlupt, D, 0, st));
  MOE_TRY(dense_gemm(DY, D, 0, wlupt, nullptr, 0, D, l, 1, T, dn, l, EP_F32, nullptr, nullptr, 0,
                     st));
  MOE_TRY(launch_rms_backward(fwd->y_perm, fwd->row_of, fwd->topk_w, T, d.k, l, d.rms_eps, dn, dr,
                              nb, st));
  // dW_lup = dy^T n: a contraction over the tokens (both operands transposed,
  // T padded with zeros).
  MOE_TRY(launch_fill_zero(dyt, (size_t)D * Tp * 2, st));
  MOE_TRY(launch_fill_zero(nt, (size_t)l * Tp * 2, st));
  MOE_TRY(launch_transpose_bf16(DY, 1, (int)T, D, dyt, Tp, 0, st));
  MOE_TRY(launch_transpose_bf16(nb, 1, (int)T, l, nt, Tp, 0, st));
  MOE_TRY(dense_gemm(dyt, Tp, 0, nt, nullptr, 0, (int)Tp, l, 1, D, g->dW_lup, l, EP_F32, nullptr,
                     nullptr, 0, st));
  // The routed experts at width l, driven by dr.
  {
    const BwdDims Dr = routed_dims(d);
    const BwdLayout Lr = bwd_layout(Dr);
    MOE_TRY(experts_bwd_core(Dr, Lr, ws, xl, static_cast<const uint16_t *>(wts->W_gate),
                             static_cast<const uint16_t *>(wts->W_up),
                             static_cast<const uint16_t *>(wts->W_down), fwd->topk_w,
                             fwd->offsets, fwd->kept_offsets, fwd->perm, fwd->row_of,
                             static_cast<const uint16_t *>(fwd->gate_up), dr, dxl, g->dW_gate,
                             g->dW_up, g->dW_down, st));
  }
  // The router, driven by dr and the expert outputs at width l; writes du.
  MOE_TRY(dense_gemm(U, D, 0, static_cast<const uint16_t *>(wts->W_route), nullptr, 0, D, d.N, 1,
                     T, logits, d.N, EP_F32, nullptr, nullptr, 0, st));
  const float aux_coef = aux_scale * d.aux_alpha * (float)d.N / (float)d.T;
  MOE_TRY(launch_route_backward(logits, T, d.N, d.k, D, l, d.gate == MOE_GATE_RENORM ? 1 : 0,
                                fwd->topk_idx, fwd->row_of, fwd->y_perm, dr, fwd->stats, aux_coef,
                                U, static_cast<const uint16_t *>(wts->W_route),
                                region<float>(ws, L.rb_part), g->dz, g->dW_route, g->du, st));
  // Through W_ldown: du += dx_l W_ldown; dW_ldown = dx_l^T u.
  MOE_TRY(launch_cast_bf16(dxl, T * l, dxlb, st));
  MOE_TRY(launch_transpose_bf16(Wldown, 1, l, D, wldt, l, 0, st));
  MOE_TRY(dense_gemm(dxlb, l, 0, wldt, nullptr, 0, l, D, 1, T, tmp, D, EP_F32, nullptr, nullptr, 0,
                     st));
  MOE_TRY(launch_add_f32(g->du, tmp, T * D, st));
  MOE_TRY(launch_fill_zero(dxlt, (size_t)l * Tp * 2, st));
  MOE_TRY(launch_fill_zero(ut, (size_t)D * Tp * 2, st));
  MOE_TRY(launch_transpose_bf16(dxlb, 1, (int)T, l, dxlt, Tp, 0, st));
  MOE_TRY(launch_transpose_bf16(U, 1, (int)T, D, ut, Tp, 0, st));
  MOE_TRY(dense_gemm(dxlt, Tp, 0, ut, nullptr, 0, (int)Tp, D, 1, l, g->dW_ldown, D, EP_F32,
                     nullptr, nullptr, 0, st));
  // The shared experts: every token, weight 1, on u and dy.
  if (d.n_shared > 0) {
    const BwdDims Ds = shared_dims(d);
    const BwdLayout Ls = bwd_layout(Ds);
    float *sw = region<float>(ws, L.sh_w);
    int32_t *sperm = region<int32_t>(ws, L.sh_perm), *srow = region<int32_t>(ws, L.sh_row);
    int32_t *soff = region<int32_t>(ws, L.sh_off), *skoff = region<int32_t>(ws, L.sh_koff);
    MOE_TRY(launch_shared_route(T, d.n_shared, sw, sperm, srow, soff, skoff, st));
    MOE_TRY(experts_bwd_core(Ds, Ls, ws, U, static_cast<const uint16_t *>(wts->Ws_gate),
                             static_cast<const uint16_t *>(wts->Ws_up),
                             static_cast<const uint16_t *>(wts->Ws_down), sw, soff, skoff, sperm,
                             srow, nullptr, DY, tmp, g->dWs_gate, g->dWs_up, g->dWs_down, st));
    MOE_TRY(launch_add_f32(g->du, tmp, T * D, st));
  }
  return MOE_OK;
}

moe_status_t moe_route_backward(const moe_desc_t *desc, const void *u, const void *W_route,
                                const int32_t *topk_idx, const int32_t *row_of,
                                const float *stats, const float *y_perm, const void *dy,
                                float aux_scale, float *dz, float *dW_route, float *du, void *ws,
                                size_t ws_bytes, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  const moe_desc_t &d = *desc;
  if (u == nullptr || W_route == nullptr || topk_idx == nullptr || row_of == nullptr ||
      stats == nullptr || y_perm == nullptr || dy == nullptr || dz == nullptr ||
      dW_route == nullptr || du == nullptr)
    return MOE_ERR_ARG;
  if (!isfinite(aux_scale)) return MOE_ERR_ARG;
  // Plain layer; the logits come from the bf16 MFMA GEMM.
  if (is_latent(d) || d.act_dtype != MOE_BF16 || d.router_dtype != MOE_BF16)
    return MOE_ERR_UNSUPPORTED;
  const Layout L = layout(d);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float *logits = region<float>(ws, L.qb_logits);
  MOE_TRY(dense_gemm(static_cast<const uint16_t *>(u), d.d, 0,
                     static_cast<const uint16_t *>(W_route), nullptr, 0, d.d, d.N, 1, d.T, logits,
                     d.N, EP_F32, nullptr, nullptr, 0, st));
  const float aux_coef = aux_scale * d.aux_alpha * (float)d.N / (float)d.T;
  return hip_status(launch_route_backward(
      logits, d.T, d.N, d.k, d.d, d.d, d.gate == MOE_GATE_RENORM ? 1 : 0, topk_idx, row_of, y_perm,
      static_cast<const uint16_t *>(dy), stats, aux_coef, static_cast<const uint16_t *>(u),
      static_cast<const uint16_t *>(W_route), region<float>(ws, L.rb_part), dz, dW_route, du,
      st));
}

moe_status_t moe_dispatch(const moe_desc_t *desc, const int32_t *topk_idx, int32_t *counts,
                          int32_t *offsets, int32_t *kept_offsets, int32_t *perm, int32_t *row_of,
                          uint8_t *drop, void *ws, size_t ws_bytes, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  if (topk_idx == nullptr || counts == nullptr || offsets == nullptr || kept_offsets == nullptr ||
      perm == nullptr || row_of == nullptr || drop == nullptr)
    return MOE_ERR_ARG;
  const Layout L = layout(*desc);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return hip_status(do_dispatch(*desc, L, topk_idx, counts, offsets, kept_offsets, perm, row_of,
                                drop, nullptr, ws, reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_ffn_scaled(const moe_desc_t *desc, const void *x, const int32_t *perm,
                                   const int32_t *offsets, const int32_t *kept_offsets,
                                   const void *W_gate, const void *W_up, const void *W_down,
                                   const void *gate_scale, const void *up_scale,
                                   const void *down_scale, float *y_perm, void *ws,
                                   size_t ws_bytes, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  if (x == nullptr || perm == nullptr || offsets == nullptr || kept_offsets == nullptr ||
      W_gate == nullptr || W_up == nullptr || W_down == nullptr || y_perm == nullptr)
    return MOE_ERR_ARG;
  const bool any_scale = gate_scale || up_scale || down_scale;
  const bool all_scales = gate_scale && up_scale && down_scale;
  if (scaled_experts(*desc) ? !all_scales : any_scale) return MOE_ERR_ARG;
  if (!mxfp4_ok(*desc)) return MOE_ERR_UNSUPPORTED;
  const Layout L = layout(*desc);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MOE_TRY(do_tile_prefix(*desc, L, kept_offsets, ws, st));
  MOE_TRY(do_ffn_gate_up(*desc, L, x, perm, offsets, kept_offsets, W_gate, W_up, gate_scale,
                         up_scale, ws, st));
  MOE_TRY(do_ffn_down(*desc, L, kept_offsets, W_down, down_scale, y_perm, ws, st));
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_desc_t *desc, const void *x, const int32_t *perm,
                            const int32_t *offsets, const int32_t *kept_offsets,
                            const void *W_gate, const void *W_up, const void *W_down,
                            float *y_perm, void *ws, size_t ws_bytes, moe_stream_t stream) {
  return moe_expert_ffn_scaled(desc, x, perm, offsets, kept_offsets, W_gate, W_up, W_down,
                               nullptr, nullptr, nullptr, y_perm, ws, ws_bytes, stream);
}

moe_status_t moe_combine(const moe_desc_t *desc, const float *y_perm, const int32_t *row_of,
                         const float *topk_w, void *y, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  if (y_perm == nullptr || row_of == nullptr || topk_w == nullptr || y == nullptr)
    return MOE_ERR_ARG;
  const moe_desc_t &d = *desc;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (is_latent(d))
    return hip_status(
        launch_combine(y_perm, row_of, topk_w, d.T, d.k, d.l, true, true, d.rms_eps, y, st));
  return hip_status(
      launch_combine(y_perm, row_of, topk_w, d.T, d.k, d.d, bf16_path(d), false, 0.f, y, st));
}

moe_status_t moe_forward(const moe_desc_t *desc, const moe_weights_t *w, const void *u, void *y,
                         const moe_outputs_t *out, void *ws, size_t ws_bytes,
                         moe_stream_t stream) {
  return forward_impl(desc, w, u, y, out, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                      nullptr, 0);
}

moe_status_t moe_forward_noalloc(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                                 void *y, const moe_outputs_t *out, moe_stream_t stream) {
  const moe_status_t v = validate(desc);
  if (v != MOE_OK) return v;
  if (layout(*desc).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  const moe_status_t s = static_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
  if (s != MOE_OK) return s;
  return forward_impl(desc, w, u, y, out, ws, (size_t)MOE_STATIC_SCRATCH_BYTES,
                      reinterpret_cast<hipStream_t>(stream), nullptr, 0);
}

moe_status_t moe_forward_traced(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                                void *y, const moe_outputs_t *out, void *ws, size_t ws_bytes,
                                moe_stream_t stream, void *const *events, int32_t n_events) {
  return forward_impl(desc, w, u, y, out, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                      events, n_events < 0 ? 0 : n_events);
}

const char *moe_stage_name(const moe_desc_t *desc, int32_t i, int32_t *n_stages) {
  if (n_stages) *n_stages = 0;
  if (validate(desc) != MOE_OK) return nullptr;
  const bool lat = is_latent(*desc);
  const int n = lat ? 9 : 5;
  if (n_stages) *n_stages = n;
  if (i < 1 || i > n) return nullptr;
  return lat ? kLatentStages[i - 1] : kPlainStages[i - 1];
}

}  // extern "C"
