// Router kernels: scores z = W_route u, fp32 softmax, top-k selection and
// combine weights (page "MoE: how sparse activation saves compute", section
// 3.2), plus per-wave partials of the balance statistics f_i and P_i
// (section 3.4).  No floating-point atomics: every sum has a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRouteBlock = 256;       // 4 waves
constexpr int kRouteMaxWaves = 8192;   // wave router, per launch (sizes the stats partials)
constexpr int kLogitsMaxWaves = 8192;  // top-k over materialised logits (N up to 1024): a wave per token up to 8192 tokens
constexpr int kRouteSmallT = 256;      // at or below: one block per token (N <= 64)
constexpr int kSmallBlock = 512;       // 8 waves: d = 4096 in one load round

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t off, float (&x)[8]) {
  if constexpr (BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const bf16_t *>(base) + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off);
    const float4 b =
        *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Selection and weights for one token whose N scores z[] every lane holds.
// Lane s < k ends with the s-th selected expert (descending z, or descending
// z + bias with a selection bias; ties to the lower index) and writes it; the
// weights come from the unbiased softmax.  Lane n < N accumulates the
// statistics of expert n (f counts the unbiased arg-max).
template <int NMAX>
__device__ __forceinline__ void select_and_write(const float (&z)[NMAX], int N, int k, int gate,
                                                 const float *bias, int64_t t, int lane,
                                                 int32_t *idx, float *w, float &acc_p,
                                                 int &acc_cnt) {
  float m = -INFINITY;
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    if (n < N) m = fmaxf(m, z[n]);
  float e[NMAX];
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    e[n] = (n < N) ? expf(z[n] - m) : 0.f;
    s += e[n];
  }
  const float inv = 1.0f / s;
  float mine_p = 0.f;
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    if (n == lane) mine_p = e[n] * inv;
  float zs[NMAX];  // selection scores
#pragma unroll
  for (int n = 0; n < NMAX; ++n) zs[n] = (bias != nullptr && n < N) ? z[n] + bias[n] : z[n];
  int first = 0;  // unbiased arg-max (ties: lower index), for f
  if (bias != nullptr) {
    float bz = -INFINITY;
    int best = -1;
#pragma unroll
    for (int n = 0; n < NMAX; ++n)
      if (n < N && (best < 0 || z[n] > bz)) {
        best = n;
        bz = z[n];
      }
    first = best;
  }
  uint64_t taken = 0;
  int my_idx = 0;
  float my_p = 0.f;
  for (int sl = 0; sl < k; ++sl) {
    int best = -1;
    float bz = -INFINITY;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      if (n < N && !((taken >> n) & 1ull) && (best < 0 || zs[n] > bz)) {
        best = n;
        bz = zs[n];
      }
    }
    float bp = 0.f;
#pragma unroll
    for (int n = 0; n < NMAX; ++n)
      if (n == best) bp = e[n] * inv;
    taken |= 1ull << best;
    if (sl == 0 && bias == nullptr) first = best;
    if (lane == sl) {
      my_idx = best;
      my_p = bp;
    }
  }
  const float psum = wave_sum(lane < k ? my_p : 0.f);
  if (lane < k) {
    idx[t * k + lane] = my_idx;
    w[t * k + lane] = (gate == 0) ? my_p / psum : my_p;
  }
  acc_p += mine_p;
  acc_cnt += (lane == first) ? 1 : 0;
}

template <bool UB, bool WB, int NMAX, int TPW>
__global__ __launch_bounds__(kRouteBlock) void route_wave_kernel(
    const void *__restrict__ u, const void *__restrict__ W, int64_t T, int d, int N, int k,
    int gate, const float *__restrict__ bias, int32_t *__restrict__ idx, float *__restrict__ w,
    float *__restrict__ part_p, int32_t *__restrict__ part_cnt) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kRouteBlock / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kRouteBlock / 64);
  float acc_p = 0.f;
  int acc_cnt = 0;
  const int64_t groups = (T + TPW - 1) / TPW;
  for (int64_t g = wave; g < groups; g += nwaves) {
    const int64_t t0 = g * TPW;
    float acc[TPW][NMAX];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int n = 0; n < NMAX; ++n) acc[i][n] = 0.f;
    for (int base = lane * 8; base < d; base += 512) {
      float x[TPW][8];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int64_t t = (t0 + i < T) ? t0 + i : T - 1;
        load8<UB>(u, t * d + base, x[i]);
      }
#pragma unroll
      for (int n = 0; n < NMAX; ++n) {
        if (n < N) {
          float wv[8];
          load8<WB>(W, (int64_t)n * d + base, wv);
#pragma unroll
          for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][n] = fmaf(x[i][j], wv[j], acc[i][n]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      float z[NMAX];
#pragma unroll
      for (int n = 0; n < NMAX; ++n) z[n] = (n < N) ? wave_sum(acc[i][n]) : 0.f;
      if (t0 + i < T)
        select_and_write<NMAX>(z, N, k, gate, bias, t0 + i, lane, idx, w, acc_p, acc_cnt);
    }
  }
  if (part_p != nullptr && lane < N) {
    part_p[(int64_t)wave * N + lane] = acc_p;
    part_cnt[(int64_t)wave * N + lane] = acc_cnt;
  }
}

// Small T: one 8-wave block per token.  Each thread accumulates its share of
// the d-loop for every expert; the 8 wave partials meet in LDS and wave 0
// adds them in a fixed order, then selects.  Stats partials are per token.
template <bool UB, bool WB, int NMAX>
__global__ __launch_bounds__(kSmallBlock) void route_small_kernel(
    const void *__restrict__ u, const void *__restrict__ W, int64_t T, int d, int N, int k,
    int gate, const float *__restrict__ bias, int32_t *__restrict__ idx, float *__restrict__ w,
    float *__restrict__ part_p, int32_t *__restrict__ part_cnt) {
  __shared__ float red[kSmallBlock / 64][NMAX];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  float acc[NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) acc[n] = 0.f;
  for (int base = threadIdx.x * 8; base < d; base += kSmallBlock * 8) {
    float x[8];
    load8<UB>(u, t * d + base, x);
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      if (n < N) {
        float wv[8];
        load8<WB>(W, (int64_t)n * d + base, wv);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[n] = fmaf(x[j], wv[j], acc[n]);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    const float v = (n < N) ? wave_sum(acc[n]) : 0.f;
    if (lane == 0) red[wave][n] = v;
  }
  __syncthreads();
  if (wave != 0) return;
  float z[NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    z[n] = ((((((red[0][n] + red[1][n]) + red[2][n]) + red[3][n]) + red[4][n]) + red[5][n]) +
            red[6][n]) +
           red[7][n];
  float acc_p = 0.f;
  int acc_cnt = 0;
  select_and_write<NMAX>(z, N, k, gate, bias, t, lane, idx, w, acc_p, acc_cnt);
  if (part_p != nullptr && lane < N) {
    part_p[t * N + lane] = acc_p;
    part_cnt[t * N + lane] = acc_cnt;
  }
}

// One wave per token over materialised logits, N <= 64 * NPL.
template <int NPL>
__global__ __launch_bounds__(kRouteBlock) void topk_logits_kernel(
    const float *__restrict__ logits, int64_t T, int N, int k, int gate,
    const float *__restrict__ bias, int32_t *__restrict__ idx, float *__restrict__ w,
    float *__restrict__ part_p, int32_t *__restrict__ part_cnt) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kRouteBlock / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kRouteBlock / 64);
  float acc_p[NPL];
  int acc_c[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    acc_p[j] = 0.f;
    acc_c[j] = 0;
  }
  for (int64_t t = wave; t < T; t += nwaves) {
    float z[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = lane + 64 * j;
      z[j] = (n < N) ? logits[t * N + n] : -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) m = fmaxf(m, z[j]);
    m = wave_max(m);
    float e[NPL];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      e[j] = (lane + 64 * j < N) ? expf(z[j] - m) : 0.f;
      s += e[j];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
    float zs[NPL];  // selection scores
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = lane + 64 * j;
      zs[j] = (bias != nullptr && n < N) ? z[j] + bias[n] : z[j];
    }
    int first = 0;  // unbiased arg-max (ties: lower index), for f
    if (bias != nullptr) {
      float bz = -INFINITY;
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        if (n < N && (bn == 0x7FFFFFFF || z[j] > bz)) {
          bz = z[j];
          bn = n;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float oz = __shfl_xor(bz, o, 64);
        const int on = __shfl_xor(bn, o, 64);
        if (oz > bz || (oz == bz && on < bn)) {
          bz = oz;
          bn = on;
        }
      }
      first = bn;
    }
    uint32_t taken = 0;
    int my_idx = 0;
    float my_p = 0.f;
    for (int sl = 0; sl < k; ++sl) {
      // Local best among this lane's untaken experts (ties: lower index).
      float bz = -INFINITY;
      int bn = 0x7FFFFFFF;
      float bp = 0.f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        if (n < N && !((taken >> j) & 1u) && (bn == 0x7FFFFFFF || zs[j] > bz)) {
          bz = zs[j];
          bn = n;
          bp = e[j] * inv;
        }
      }
      // Wave arg-max: larger z wins, equal z -> lower expert index.
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float oz = __shfl_xor(bz, o, 64);
        const int on = __shfl_xor(bn, o, 64);
        const float op = __shfl_xor(bp, o, 64);
        if (oz > bz || (oz == bz && on < bn)) {
          bz = oz;
          bn = on;
          bp = op;
        }
      }
      if ((bn & 63) == lane) taken |= 1u << (bn >> 6);
      if (sl == 0 && bias == nullptr) first = bn;
      if (lane == sl) {
        my_idx = bn;
        my_p = bp;
      }
    }
    const float psum = wave_sum(lane < k ? my_p : 0.f);
    if (lane < k) {
      idx[t * k + lane] = my_idx;
      w[t * k + lane] = (gate == 0) ? my_p / psum : my_p;
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      acc_p[j] += e[j] * inv;
      acc_c[j] += (lane + 64 * j == first) ? 1 : 0;
    }
  }
  if (part_p != nullptr) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = lane + 64 * j;
      if (n < N) {
        part_p[(int64_t)wave * N + n] = acc_p[j];
        part_cnt[(int64_t)wave * N + n] = acc_c[j];
      }
    }
  }
}

// stats = [f(N), P(N), N sum f P, alpha N sum f P] (page "MoE: how sparse
// activation saves compute", section 3.4: f_i the share of tokens whose top
// expert is i, P_i the mean router probability of expert i), in two
// fixed-order passes over the per-wave partial rows [waves][N]:
//  1. block (c, s) sums rows [256 s, 256 s + 256) of a band of EW experts
//     (EW lanes a row, 256 / EW rows at a time: reads coalesced along the
//     experts) and leaves the sums in the slice's first row;
//  2. one block adds the slices' first rows per expert, writes f and P and
//     sums f_i P_i.
constexpr int kStatsSliceRows = 256;

__global__ __launch_bounds__(256) void stats_slice_kernel(float *__restrict__ part_p,
                                                          int32_t *__restrict__ part_cnt,
                                                          int waves, int N, int EW) {
  __shared__ float sp[256];
  __shared__ int sc[256];
  const int rr = threadIdx.x / EW, e = threadIdx.x % EW;
  const int rpp = 256 / EW;
  const int n = blockIdx.x * EW + e;
  const int w0 = blockIdx.y * kStatsSliceRows;
  const int w1 = w0 + kStatsSliceRows < waves ? w0 + kStatsSliceRows : waves;
  float p = 0.f;
  int c = 0;
  if (n < N) {
    for (int wv = w0 + rr; wv < w1; wv += rpp) {
      p += part_p[(int64_t)wv * N + n];
      c += part_cnt[(int64_t)wv * N + n];
    }
  }
  sp[threadIdx.x] = p;
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int s = rpp / 2; s > 0; s >>= 1) {
    if (rr < s) {
      sp[threadIdx.x] += sp[threadIdx.x + s * EW];
      sc[threadIdx.x] += sc[threadIdx.x + s * EW];
    }
    __syncthreads();
  }
  // Only this block reads these columns of this slice, and it has finished.
  if (rr == 0 && n < N) {
    part_p[(int64_t)w0 * N + n] = sp[e];
    part_cnt[(int64_t)w0 * N + n] = sc[e];
  }
}

__global__ __launch_bounds__(1024) void stats_total_kernel(const float *__restrict__ part_p,
                                                           const int32_t *__restrict__ part_cnt,
                                                           int slices, int64_t T, int N,
                                                           float alpha, float *__restrict__ stats) {
  __shared__ float red[1024];
  float local = 0.f;
  for (int n = threadIdx.x; n < N; n += 1024) {
    float p = 0.f;
    int64_t c = 0;
    for (int s = 0; s < slices; ++s) {
      p += part_p[(int64_t)s * kStatsSliceRows * N + n];
      c += part_cnt[(int64_t)s * kStatsSliceRows * N + n];
    }
    const float f = (float)((double)c / (double)T);
    const float P = p / (float)T;
    stats[n] = f;
    stats[N + n] = P;
    local += f * P;
  }
  red[threadIdx.x] = local;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float v = (float)N * red[0];
    stats[2 * N] = v;
    stats[2 * N + 1] = alpha * v;
  }
}

template <bool UB, bool WB, int NMAX, int TPW>
hipError_t launch_rw(const void *u, const void *W, int64_t T, int d, int N, int k, int gate,
                     const float *bias, int32_t *idx, float *w, float *pp, int32_t *pc, hipStream_t st) {
  const int waves = route_waves(T, N);
  hipLaunchKernelGGL((route_wave_kernel<UB, WB, NMAX, TPW>), dim3(waves / 4), dim3(kRouteBlock), 0,
                     st, u, W, T, d, N, k, gate, bias, idx, w, pp, pc);
  return hipGetLastError();
}

template <bool UB, bool WB, int NMAX>
hipError_t launch_rs(const void *u, const void *W, int64_t T, int d, int N, int k, int gate,
                     const float *bias, int32_t *idx, float *w, float *pp, int32_t *pc, hipStream_t st) {
  hipLaunchKernelGGL((route_small_kernel<UB, WB, NMAX>), dim3((unsigned)T), dim3(kSmallBlock), 0,
                     st, u, W, T, d, N, k, gate, bias, idx, w, pp, pc);
  return hipGetLastError();
}

template <bool UB, bool WB>
hipError_t launch_rw_n(const void *u, const void *W, int64_t T, int d, int N, int k, int gate,
                       const float *bias, int32_t *idx, float *w, float *pp, int32_t *pc, hipStream_t st) {
  if (T <= kRouteSmallT) {
    if (N <= 8) return launch_rs<UB, WB, 8>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
    if (N <= 16) return launch_rs<UB, WB, 16>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
    if (N <= 32) return launch_rs<UB, WB, 32>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
    return launch_rs<UB, WB, 64>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  }
  if (N <= 8) return launch_rw<UB, WB, 8, 4>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  if (N <= 16) return launch_rw<UB, WB, 16, 2>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  if (N <= 32) return launch_rw<UB, WB, 32, 1>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  return launch_rw<UB, WB, 64, 1>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
}

}  // namespace

int route_waves(int64_t T, int N) {
  if (N <= 64 && T <= kRouteSmallT) return (int)T;  // one partial row per token
  const int tpw = N <= 8 ? 4 : (N <= 16 ? 2 : 1);
  int64_t groups = (T + tpw - 1) / tpw;
  int64_t cap = kRouteMaxWaves;
  if (N > 64) {
    groups = T;
    cap = kLogitsMaxWaves;
  }
  int64_t waves = groups < cap ? groups : cap;
  waves = (waves + 3) / 4 * 4;  // whole blocks of 4 waves
  return (int)waves;
}

hipError_t launch_route_wave(const void *u, bool u_bf16, const void *W, bool w_bf16, int64_t T,
                             int d, int N, int k, int gate, const float *bias, int32_t *idx,
                             float *w, float *part_p, int32_t *part_cnt, hipStream_t st) {
  if (u_bf16 && w_bf16) return launch_rw_n<true, true>(u, W, T, d, N, k, gate, bias, idx, w, part_p, part_cnt, st);
  if (u_bf16) return launch_rw_n<true, false>(u, W, T, d, N, k, gate, bias, idx, w, part_p, part_cnt, st);
  if (w_bf16) return launch_rw_n<false, true>(u, W, T, d, N, k, gate, bias, idx, w, part_p, part_cnt, st);
  return launch_rw_n<false, false>(u, W, T, d, N, k, gate, bias, idx, w, part_p, part_cnt, st);
}

hipError_t launch_topk_logits(const float *logits, int64_t T, int N, int k, int gate,
                              const float *bias, int32_t *idx, float *w, float *part_p,
                              int32_t *part_cnt, hipStream_t st) {
  const int waves = route_waves(T, N);
  const dim3 grid(waves / 4), block(kRouteBlock);
  if (N <= 256)
    hipLaunchKernelGGL(topk_logits_kernel<4>, grid, block, 0, st, logits, T, N, k, gate, bias, idx, w,
                       part_p, part_cnt);
  else if (N <= 512)
    hipLaunchKernelGGL(topk_logits_kernel<8>, grid, block, 0, st, logits, T, N, k, gate, bias, idx, w,
                       part_p, part_cnt);
  else
    hipLaunchKernelGGL(topk_logits_kernel<16>, grid, block, 0, st, logits, T, N, k, gate, bias, idx, w,
                       part_p, part_cnt);
  return hipGetLastError();
}

hipError_t launch_stats_finalize(float *part_p, int32_t *part_cnt, int waves, int64_t T, int N,
                                 float alpha, float *stats, hipStream_t st) {
  int ew = 8;  // expert band: a power of two, 8 .. 64
  while (ew < 64 && ew < N) ew *= 2;
  const int slices = (waves + kStatsSliceRows - 1) / kStatsSliceRows;
  hipLaunchKernelGGL(stats_slice_kernel, dim3((N + ew - 1) / ew, slices), dim3(256), 0, st,
                     part_p, part_cnt, waves, N, ew);
  hipLaunchKernelGGL(stats_total_kernel, dim3(1), dim3(1024), 0, st, part_p, part_cnt, slices, T,
                     N, alpha, stats);
  return hipGetLastError();
}

}  // namespace moe
