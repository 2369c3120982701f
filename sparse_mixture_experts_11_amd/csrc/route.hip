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
constexpr int kTopkBlock = 256;       // top-k over materialised logits (N up to 1024): 4 waves
constexpr int kTopkMaxBlocks = 512;   // 2048 waves: all resident at once, a few tokens each
constexpr int kRouteSmallT = 256;      // at or below: one block per token (N <= 64)
constexpr int kSmallBlock = 512;       // 8 waves: d = 4096 in one load round

// Lane exchange with lane ^ M.
template <int M>
__device__ __forceinline__ float xchg(float v) {
  if constexpr (M == 1) return lane_xor1(v);
  else if constexpr (M == 2) return lane_xor2(v);
  else if constexpr (M < 32) return lane_xor_swz<M>(v);
  else return __shfl_xor(v, 32, kWave);
}

// The low log2(V) bits of x in reverse order.
template <int V>
__device__ __forceinline__ int bit_reverse(int x) {
  int r = 0;
#pragma unroll
  for (int b = 1; b < V; b <<= 1) {
    r <<= 1;
    r |= (x & b) ? 1 : 0;
  }
  return r;
}

// One step of a transposed reduction: pairs (r[i], r[i + H]) split between
// this lane and lane ^ M -- the lane with bit M set keeps the upper member
// and sends the lower one -- and each kept member adds the partner's.
template <int H, int M>
__device__ __forceinline__ void transpose_step(float *r, int lane) {
  const bool hi = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float a = r[i], b = r[i + H];
    const float send = hi ? a : b;
    r[i] = (hi ? b : a) + xchg<M>(send);
  }
}

// Sum over the 64 lanes of each of V per-lane values (V a power of two up
// to 64) in log2(V) transposed steps plus 6 - log2(V) plain ones, instead of
// V separate wave reductions.  Lane l returns the total of value
// bit_reverse<V>(l mod V); r is overwritten.  The steps run on lane
// distances 1, 2, ... so the largest ones (V/2 exchanges) are DPP moves.
template <int V>
__device__ __forceinline__ float transpose_reduce(float (&r)[V], int lane) {
  if constexpr (V >= 2) transpose_step<V / 2, 1>(r, lane); else r[0] += xchg<1>(r[0]);
  if constexpr (V >= 4) transpose_step<V / 4, 2>(r, lane); else r[0] += xchg<2>(r[0]);
  if constexpr (V >= 8) transpose_step<V / 8, 4>(r, lane); else r[0] += xchg<4>(r[0]);
  if constexpr (V >= 16) transpose_step<V / 16, 8>(r, lane); else r[0] += xchg<8>(r[0]);
  if constexpr (V >= 32) transpose_step<V / 32, 16>(r, lane); else r[0] += xchg<16>(r[0]);
  if constexpr (V >= 64) transpose_step<1, 32>(r, lane); else r[0] += xchg<32>(r[0]);
  return r[0];
}

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
  float zs[NMAX];  // selection scores (a NaN ranks as -inf)
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    const float v = (bias != nullptr && n < N) ? z[n] + bias[n] : z[n];
    zs[n] = (v == v) ? v : -INFINITY;
  }
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
  float psum = 0.f;  // every lane holds every z: the selection is uniform
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
    psum += bp;
    if (sl == 0 && bias == nullptr) first = best;
    if (lane == sl) {
      my_idx = best;
      my_p = bp;
    }
  }
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
  // Lane l ends with the wave's total of expert bitrev(l mod NMAX).
  const float tot = transpose_reduce<NMAX>(acc, lane);
  if (lane < NMAX) red[wave][bit_reverse<NMAX>(lane)] = tot;
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

// Wave reductions over DPP moves inside rows of 16 lanes, then the rows
// folded into row 3 by row_bcast:15 and row_bcast:31 and read from lane 63
// (a fixed order: deterministic).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, lane_xor1(v));
  v = fmaxf(v, lane_xor2(v));
  v = fmaxf(v, lane_half_mirror(v));
  v = fmaxf(v, lane_mirror(v));
  v = fmaxf(v, __int_as_float(dpp_bcast15(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_bcast31(__float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += lane_xor1(v);
  v += lane_xor2(v);
  v += lane_half_mirror(v);
  v += lane_mirror(v);
  // rows 1 and 3 add rows 0 and 2; then rows 2 and 3 add rows 0 + 1
  const float a = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += ((threadIdx.x & 16) != 0) ? a : 0.f;
  const float b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  v += ((threadIdx.x & 32) != 0) ? b : 0.f;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave minimum of an int (readlane 63 after the DPP steps).
__device__ __forceinline__ int wave_min_dpp(int v) {
  v = min(v, lane_xor1(v));
  v = min(v, lane_xor2(v));
  v = min(v, lane_half_mirror(v));
  v = min(v, lane_mirror(v));
  v = min(v, dpp_bcast15(v));
  v = min(v, dpp_bcast31(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k over materialised logits (N <= 64 * NPL, the router GEMM's output,
// or the sum of its two K-halves when SPLIT): a wave per token at a time,
// consecutive tokens per wave; lane l holds experts l, l + 64, ...  Each
// lane keeps its three best untaken scores (ties: lower expert index
// first).  A selection round takes the wave maximum of the lanes' heads (one
// DPP max), finds the lanes holding it with a ballot (several only on an
// exact tie, then the lowest expert index wins) and pops the winner's head;
// a lane whose three entries are all taken while rounds remain triggers a
// rebuild of every lane's list from its untaken scores (rare: one lane must
// win three of the k rounds).  The probabilities of the chosen experts are
// recomputed from their logits with the same operations as the softmax
// (same values).  The statistics partials of a block's waves are added in
// LDS (wave order), so each block writes one partial row.
template <int NPL, bool SPLIT>
__global__ __launch_bounds__(kTopkBlock) void topk_logits_kernel(
    const float *__restrict__ logits, const float *__restrict__ logits2, int64_t T, int N, int k,
    int gate, const float *__restrict__ bias, int32_t *__restrict__ idx, float *__restrict__ w,
    float *__restrict__ part_p, int32_t *__restrict__ part_cnt) {
  constexpr int kW = kTopkBlock / 64;
  constexpr int kEmpty = 0x7FFFFFFF;
  __shared__ float sp[kW][64 * NPL];
  __shared__ int sc[kW][64 * NPL];
  const int lane = threadIdx.x & 63;
  const int wib = threadIdx.x >> 6;
  const int wave = blockIdx.x * kW + wib;
  const int nwaves = gridDim.x * kW;
  // The wave's statistics partials accumulate in its own LDS rows (lane l
  // owns columns l, l + 64, ...): registers held across the token loop cost
  // waves per SIMD.
  float *my_sp = sp[wib];
  int *my_sc = sc[wib];
  // Loads are unconditional at clamped indices (a load under a per-element
  // condition becomes its own branch, and the loads then issue one by one);
  // entries past N are replaced by -inf after the load.
  auto ncl = [&](int j) {
    const int n = lane + 64 * j;
    return n < N ? n : N - 1;
  };
  float bj[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    my_sp[lane + 64 * j] = 0.f;
    my_sc[lane + 64 * j] = 0;
    bj[j] = (bias != nullptr) ? bias[ncl(j)] : 0.f;
  }
  auto logit = [&](float a, float b) { return SPLIT ? a + b : a; };
  for (int64_t t = wave; t < T; t += nwaves) {
    // The token's logits (no prefetch of the next token: the registers it
    // would hold cost waves per SIMD, which hide these loads better).
    float z[NPL];
    {
      float za[NPL], zb[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        za[j] = logits[t * N + ncl(j)];
        zb[j] = SPLIT ? logits2[t * N + ncl(j)] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        // A NaN logit takes part as -inf: every selection below then has a
        // total order, so it always yields k distinct experts below N.
        const float v = logit(za[j], zb[j]);
        z[j] = (lane + 64 * j < N && v == v) ? v : -INFINITY;
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) m = fmaxf(m, z[j]);
    m = wave_max_dpp(m);
    float e[NPL];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      e[j] = (lane + 64 * j < N) ? __expf(z[j] - m) : 0.f;
      s += e[j];
    }
    s = wave_sum_dpp(s);
    const float inv = 1.0f / s;
    // Unbiased arg-max (ties: lower index), for f: the lowest index whose
    // logit equals the maximum.
    int first;
    {
      int fl = kEmpty;
#pragma unroll
      for (int j = NPL - 1; j >= 0; --j) fl = (z[j] == m && lane + 64 * j < N) ? lane + 64 * j : fl;
      first = wave_min_dpp(fl);
    }
    // This token's share of the statistics partials (z and e are not needed
    // past here).
#pragma unroll
    for (int j = 0; j < NPL; ++j) my_sp[lane + 64 * j] += e[j] * inv;
    if (lane == (first & 63)) my_sc[first] += 1;
    float zs[NPL];  // selection scores
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float v = (bias != nullptr) ? z[j] + bj[j] : z[j];
      zs[j] = (v == v) ? v : -INFINITY;
    }
    // The lane's three best untaken scores, c[0] first (valid entries form
    // a prefix of j, and j runs in index order, so a strict > keeps ties in
    // index order).
    uint32_t taken = 0;
    float c[3];
    int nn[3];
    // Insert score v of expert n; slot i takes it if it is empty (when
    // CHECK_EMPTY) or v beats it; the lower slots shift down.
    auto insert = [&](float v, int n, bool ok, bool check_empty) {
      bool t[3];
#pragma unroll
      for (int i = 0; i < 3; ++i)
        t[i] = ok & ((check_empty & (nn[i] == kEmpty)) | (v > c[i]));
      c[2] = t[1] ? c[1] : (t[2] ? v : c[2]);
      nn[2] = t[1] ? nn[1] : (t[2] ? n : nn[2]);
      c[1] = t[0] ? c[0] : (t[1] ? v : c[1]);
      nn[1] = t[0] ? nn[0] : (t[1] ? n : nn[1]);
      c[0] = t[0] ? v : c[0];
      nn[0] = t[0] ? n : nn[0];
    };
    auto clear = [&]() {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        c[i] = -INFINITY;
        nn[i] = kEmpty;
      }
    };
    clear();
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = lane + 64 * j;
      // From j = 3 on every slot of a lane with a valid entry j is full,
      // and entries past N (-inf) beat nothing.
      insert(zs[j], n, n < N, j < 3);
    }
    // After a lane's three entries are taken while rounds remain, every
    // lane rebuilds from its untaken scores.
    auto rebuild = [&]() {
      clear();
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        insert(zs[j], n, (n < N) & !((taken >> j) & 1u), true);
      }
    };
    int my_idx = 0;
    for (int sl = 0; sl < k; ++sl) {
      const float hm = wave_max_dpp(c[0]);
      const uint64_t at = __builtin_amdgcn_ballot_w64(c[0] == hm);
      int win;
      if (__builtin_popcountll(at) == 1) {
        win = __builtin_amdgcn_readlane(nn[0], __builtin_ctzll(at));
      } else {
        // An exact tie between lanes (or only -inf left): the lowest index.
        win = wave_min_dpp(c[0] == hm ? nn[0] : kEmpty);
      }
      if (lane == sl) my_idx = win;
      if (lane == (win & 63)) {
        taken |= 1u << (win >> 6);
        c[0] = c[1];
        nn[0] = nn[1];
        c[1] = c[2];
        nn[1] = nn[2];
        c[2] = -INFINITY;
        nn[2] = kEmpty;
      }
      if (sl + 1 < k && __builtin_amdgcn_readlane(nn[0], win & 63) == kEmpty) rebuild();
    }
    // Chosen experts' probabilities: the softmax's own arithmetic on the
    // same logits.
    float my_p = 0.f;
    if (lane < k) {
      const float zz = logit(logits[t * N + my_idx], SPLIT ? logits2[t * N + my_idx] : 0.f);
      my_p = __expf(zz - m) * inv;
    }
    const float psum = wave_sum_dpp(my_p);
    if (lane < k) {
      idx[t * k + lane] = my_idx;
      w[t * k + lane] = (gate == 0) ? my_p / psum : my_p;
    }
  }
  if (part_p == nullptr) return;
  __syncthreads();
  for (int n = threadIdx.x; n < N; n += kTopkBlock) {
    float p = sp[0][n];
    int c = sc[0][n];
#pragma unroll
    for (int q = 1; q < kW; ++q) {
      p += sp[q][n];
      c += sc[q][n];
    }
    part_p[(int64_t)blockIdx.x * N + n] = p;
    part_cnt[(int64_t)blockIdx.x * N + n] = c;
  }
}

// Large T, N <= 8, bf16 u with d = 512 CH: the whole router matrix sits in
// each block's LDS (rows past N zero; at most 64 KiB), read once per block,
// and each wave routes 4 tokens at a time with all 4 x CH of its 16-byte
// u loads in flight together (lane l reads columns 512 c + 8 l .. + 7).  The
// lane's 4 x 8 partial scores meet in one transposed reduction, the two
// wave halves' sums pass through LDS, and lane (t, n) of the first 32
// (token t of the 4, expert n) finishes the selection for its own expert
// from its token's 8 scores.  bf16 router weights take packed bf16 dot
// products (v_dot2_f32_bf16, products exact in fp32); fp32 weights
// widen u and use fp32 fmas.  One partial row of the statistics per block.
constexpr int kTileTok = 4;
constexpr int kTileMaxBlocks = 512;  // two blocks (8 waves) per CU

template <bool WB, int CH>
__global__ __launch_bounds__(kRouteBlock, 2) void route_tile_kernel(
    const bf16_t *__restrict__ u, const void *__restrict__ W, int64_t T, int d, int N, int k,
    int gate, const float *__restrict__ bias, int32_t *__restrict__ idx, float *__restrict__ w,
    float *__restrict__ part_p, int32_t *__restrict__ part_cnt) {
  constexpr int WES = WB ? 2 : 4;  // bytes per router weight
  static_assert(8 * 512 * CH * WES <= 65536, "router matrix within 64 KiB");
  __shared__ __attribute__((aligned(16))) char smem[8 * 512 * CH * WES + kRouteBlock * 4];
  const int wrow = d * WES;        // bytes per router row in LDS (d = 512 CH)
  float *zx = reinterpret_cast<float *>(smem + 8 * wrow) + (threadIdx.x >> 6) * 64;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kRouteBlock / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kRouteBlock / 64);
  const int64_t groups = (T + kTileTok - 1) / kTileTok;
  // The router matrix goes straight to LDS (16-byte direct loads, all in
  // flight together; rows past N read as zeros beyond the buffer's end),
  // and the wave's first 4 x CH u loads follow them before any wait.
  {
    typedef __attribute__((address_space(3))) void *lds_ptr_t;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (uint32_t)(N * wrow));
    constexpr int kFill = 8 * 512 * CH * WES / (kRouteBlock * 16);
#pragma unroll
    for (int i = 0; i < kFill; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (lds_ptr_t)(smem + (i * kRouteBlock + (threadIdx.x & ~63)) * 16), 16,
          (uint32_t)((i * kRouteBlock + threadIdx.x) * 16), 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 x[kTileTok][CH];
  auto load_x = [&](int64_t g) {
    const int64_t t0 = g * kTileTok;
#pragma unroll
    for (int t = 0; t < kTileTok; ++t) {
      const int64_t tt = (t0 + t < T) ? t0 + t : T - 1;
#pragma unroll
      for (int c = 0; c < CH; ++c)
        x[t][c] = *reinterpret_cast<const u32x4 *>(u + tt * d + c * 512 + lane * 8);
    }
  };
  if (wave < groups) {
    load_x(wave);
    __builtin_amdgcn_sched_barrier(0);
    // In-order load counting: once at most the 4 x CH u loads remain, the
    // router matrix has landed.
    if constexpr (CH == 8) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    else if constexpr (CH == 4) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (CH == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  barrier_keep_loads();  // every wave's share of the matrix is in LDS; u loads keep flying
  const int tl = (lane >> 3) & 3, nl = lane & 7;  // lanes 0..31: (token, expert)
  float bv[8];  // selection bias, 0 without one
#pragma unroll
  for (int j = 0; j < 8; ++j) bv[j] = (bias != nullptr && j < N) ? bias[j] : 0.f;
  float acc_p = 0.f;
  int acc_c = 0;
  for (int64_t g = wave; g < groups; g += nwaves) {
    const int64_t t0 = g * kTileTok;
    if (g != wave) load_x(g);
    __builtin_amdgcn_sched_barrier(0);  // all 4 x CH loads issued before any use
    float acc[kTileTok * 8];
#pragma unroll
    for (int i = 0; i < kTileTok * 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        if constexpr (WB) {
          const u32x4 wv =
              *reinterpret_cast<const u32x4 *>(smem + n * wrow + (c * 512 + lane * 8) * 2);
#pragma unroll
          for (int t = 0; t < kTileTok; ++t) {
            float a = acc[t * 8 + n];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              // (elements taken as scalars first: a bit cast of a vector
              // element inside this loop compiled to element 0 every time)
              const uint32_t xq = x[t][c][q], wq = wv[q];
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq),
                                                  __builtin_bit_cast(bf16x2, wq), a, false);
            }
            acc[t * 8 + n] = a;
          }
        } else {
          const char *wp = smem + n * wrow + (c * 512 + lane * 8) * 4;
          const float4 w0 = *reinterpret_cast<const float4 *>(wp);
          const float4 w1 = *reinterpret_cast<const float4 *>(wp + 16);
          const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int t = 0; t < kTileTok; ++t) {
            float a = acc[t * 8 + n];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              a = fmaf(__uint_as_float(x[t][c][q] << 16), wf[2 * q], a);
              a = fmaf(__uint_as_float(x[t][c][q] & 0xFFFF0000u), wf[2 * q + 1], a);
            }
            acc[t * 8 + n] = a;
          }
        }
      }
    }
    // Lane l (and l ^ 32) now holds half of the sum of value bit_reverse<32>(l mod 32) = t * 8 + n.
    float r[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = acc[i];
    transpose_step<16, 1>(r, lane);
    transpose_step<8, 2>(r, lane);
    transpose_step<4, 4>(r, lane);
    transpose_step<2, 8>(r, lane);
    transpose_step<1, 16>(r, lane);
    zx[(lane & 32) + bit_reverse<32>(lane & 31)] = r[0];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float z[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = zx[tl * 8 + j] + zx[32 + tl * 8 + j];
    __builtin_amdgcn_wave_barrier();  // every lane has read zx before the next group writes it
    const int64_t tt = t0 + tl;
    if (lane < 32 && tt < T && nl < N) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < N) m = fmaxf(m, z[j]);
      float e[8];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[j] = (j < N) ? expf(z[j] - m) : 0.f;
        s += e[j];
      }
      const float inv = 1.0f / s;
      float zs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // NaN scores rank as -inf, so that the ranks below are distinct and
        // every slot receives an expert.
        const float v = z[j] + bv[j];
        zs[j] = (v == v) ? v : -INFINITY;
      }
      // Rank of every expert in the selection order (score descending, ties
      // to the lower index) and the selected probability mass.
      int rank_mine = 0, first_mine = 0;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= N) continue;
        int rj = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < N && i != j && (zs[i] > zs[j] || (zs[i] == zs[j] && i < j))) ++rj;
        if (rj < k) psum += e[j] * inv;
        if (j == nl) rank_mine = rj;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < N && i != nl && (z[i] > z[nl] || (z[i] == z[nl] && i < nl))) ++first_mine;
      const float p = e[nl] * inv;
      if (rank_mine < k) {
        idx[tt * k + rank_mine] = nl;
        w[tt * k + rank_mine] = (gate == 0) ? p / psum : p;
      }
      acc_p += p;
      acc_c += (first_mine == 0) ? 1 : 0;
    }
  }
  if (part_p == nullptr) return;
  // Lanes n, n + 8, n + 16, n + 24 hold expert n's partials; the block's
  // four waves then meet in LDS (wave order): one partial row per block.
  acc_p += xchg<8>(acc_p);
  acc_c += lane_xor_swz<8>(acc_c);
  acc_p += xchg<16>(acc_p);
  acc_c += lane_xor_swz<16>(acc_c);
  __shared__ float bp[kRouteBlock / 64][8];
  __shared__ int bc[kRouteBlock / 64][8];
  if (lane < 8) {
    bp[threadIdx.x >> 6][lane] = acc_p;
    bc[threadIdx.x >> 6][lane] = acc_c;
  }
  __syncthreads();
  if (threadIdx.x < N) {
    const int n = threadIdx.x;
    part_p[(int64_t)blockIdx.x * N + n] = ((bp[0][n] + bp[1][n]) + bp[2][n]) + bp[3][n];
    part_cnt[(int64_t)blockIdx.x * N + n] = bc[0][n] + bc[1][n] + bc[2][n] + bc[3][n];
  }
}

// stats = [f(N), P(N), N sum f P, alpha N sum f P] (page "MoE: how sparse
// activation saves compute", section 3.4: f_i the share of tokens whose top
// expert is i, P_i the mean router probability of expert i), in two
// fixed-order passes over the per-wave partial rows [waves][N]:
//  1. block (c, s) sums rows [32 s, 32 s + 32) of a band of EW experts
//     (EW lanes a row, 256 / EW rows at a time: reads coalesced along the
//     experts) and leaves the sums in the slice's first row (32-row slices:
//     enough blocks to spread the reads, few slices for pass 2);
//  2. one block adds the slices' first rows per expert, writes f and P and
//     sums f_i P_i.
constexpr int kStatsSliceRows = 32;

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
  const int waves = route_waves(T, N, d, UB, WB);
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

// The tile router: large T, N <= 8, bf16 u, d = 512 CH with CH in {1, 2, 4,
// 8} and the 8-row router matrix within 64 KiB of LDS.
bool route_tile_ok(int64_t T, int N, int d, bool u_bf16, bool w_bf16) {
  const int ch = d / 512;
  return T > kRouteSmallT && N <= 8 && u_bf16 && d % 512 == 0 &&
         (ch == 1 || ch == 2 || ch == 4 || ch == 8) && 8 * d * (w_bf16 ? 2 : 4) <= 65536;
}

int route_tile_blocks(int64_t T) {
  const int64_t groups = (T + kTileTok - 1) / kTileTok;
  const int64_t b = (groups + 3) / 4;
  return (int)(b < kTileMaxBlocks ? b : kTileMaxBlocks);
}

template <bool WB>
hipError_t launch_tile(const void *u, const void *W, int64_t T, int d, int N, int k, int gate,
                       const float *bias, int32_t *idx, float *w, float *pp, int32_t *pc,
                       hipStream_t st) {
  const dim3 grid(route_tile_blocks(T)), block(kRouteBlock);
  const bf16_t *ub = static_cast<const bf16_t *>(u);
  switch (d / 512) {
    case 1:
      hipLaunchKernelGGL((route_tile_kernel<WB, 1>), grid, block, 0, st, ub, W, T, d, N, k, gate,
                         bias, idx, w, pp, pc);
      break;
    case 2:
      hipLaunchKernelGGL((route_tile_kernel<WB, 2>), grid, block, 0, st, ub, W, T, d, N, k, gate,
                         bias, idx, w, pp, pc);
      break;
    case 4:
      hipLaunchKernelGGL((route_tile_kernel<WB, 4>), grid, block, 0, st, ub, W, T, d, N, k, gate,
                         bias, idx, w, pp, pc);
      break;
    default:
      if constexpr (WB)
        hipLaunchKernelGGL((route_tile_kernel<WB, 8>), grid, block, 0, st, ub, W, T, d, N, k,
                           gate, bias, idx, w, pp, pc);
      break;
  }
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
  if (route_tile_ok(T, N, d, UB, WB))
    return launch_tile<WB>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  if (N <= 8) return launch_rw<UB, WB, 8, 4>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  if (N <= 16) return launch_rw<UB, WB, 16, 2>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  if (N <= 32) return launch_rw<UB, WB, 32, 1>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
  return launch_rw<UB, WB, 64, 1>(u, W, T, d, N, k, gate, bias, idx, w, pp, pc, st);
}

// Top-k over logits: blocks of kTopkBlock / 64 waves, a token per wave at a time.
int topk_blocks(int64_t T) {
  const int64_t b = (T + kTopkBlock / 64 - 1) / (kTopkBlock / 64);
  return (int)(b < kTopkMaxBlocks ? b : kTopkMaxBlocks);
}

}  // namespace

int route_waves(int64_t T, int N, int d, bool u_bf16, bool w_bf16) {
  if (N > 64) return topk_blocks(T);                  // one partial row per block
  if (T <= kRouteSmallT) return (int)T;               // one partial row per token
  if (route_tile_ok(T, N, d, u_bf16, w_bf16)) return route_tile_blocks(T);  // per block
  const int tpw = N <= 8 ? 4 : (N <= 16 ? 2 : 1);
  const int64_t groups = (T + tpw - 1) / tpw;
  int64_t waves = groups < kRouteMaxWaves ? groups : kRouteMaxWaves;
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

hipError_t launch_topk_logits(const float *logits, const float *logits2, int64_t T, int N, int k,
                              int gate, const float *bias, int32_t *idx, float *w, float *part_p,
                              int32_t *part_cnt, hipStream_t st) {
  const dim3 grid(topk_blocks(T)), block(kTopkBlock);
#define MOE_TOPK(NPLV)                                                                          \
  if (logits2 != nullptr)                                                                       \
    hipLaunchKernelGGL((topk_logits_kernel<NPLV, true>), grid, block, 0, st, logits, logits2, T, \
                       N, k, gate, bias, idx, w, part_p, part_cnt);                             \
  else                                                                                          \
    hipLaunchKernelGGL((topk_logits_kernel<NPLV, false>), grid, block, 0, st, logits, nullptr,  \
                       T, N, k, gate, bias, idx, w, part_p, part_cnt);
  if (N <= 256) {
    MOE_TOPK(4)
  } else if (N <= 512) {
    MOE_TOPK(8)
  } else {
    MOE_TOPK(16)
  }
#undef MOE_TOPK
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
