// Router backward (page "MoE: how sparse activation saves compute", §3.2
// eqs. z, p, a, y and §3.4 eq. L_aux, differentiated with the selected sets,
// the expert outputs F and the arg-max shares f held fixed), for the loss
// <dy, y> + aux_scale * L_aux:
//   da_{t,s} = dy_t . F_{i_s}(u_t)                 (kept slots; 0 if dropped)
//   renorm:   dp_j = (da_j - sum_s da_s a_s) / sum_S p   (j in S_t)
//   prob:     dp_j = da_j
//   aux:      dp_{t,i} += aux_scale * alpha * N * f_i / T
//   softmax:  dz_t = p_t * (dp_t - p_t . dp_t)
//   dW_route = dz^T u,   du = dz W_route   (the router's share of du)
//
//   rb_dz_kernel:   a wave per token (8 per block): softmax of the logits,
//                   the k dot products dy_t . y_perm[row] (over d, or over l
//                   for the latent layer, whose dy is the gradient at the
//                   aggregated r), the gate and
//                   softmax backward through a per-wave LDS row of p and dp.
//   rb_dw_kernel:   fp32 partial sums of dz^T u over chunks of tokens: a
//                   thread per 8 columns of u (one 16-byte load a token) and
//                   8 experts, the chunk's dz staged in LDS;
//   rb_dw_reduce:   the chunks summed in a fixed order (deterministic): 16
//                   interleaved runs of chunks, then the runs in order.
//   rb_du_kernel:   a thread per 8 columns of W_route and 8 tokens.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRbTokens = 8;     // waves (tokens) per block in rb_dz_kernel
constexpr int kDwExperts = 8;    // experts per rb_dw_kernel block
constexpr int kDwChunk = 64;     // tokens per rb_dw_kernel chunk (at least)
constexpr int kDwStage = 256;    // tokens of dz staged in LDS at a time
constexpr int kDuTokens = 8;     // tokens per rb_du_kernel thread
constexpr int kRbMaxK = 32;      // slots per token (k <= 32)

template <int NPL>
__global__ __launch_bounds__(64 * kRbTokens) void rb_dz_kernel(
    const float *__restrict__ logits, int64_t T, int N, int k, int d, int renorm,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ row_of,
    const float *__restrict__ y_perm, const uint16_t *__restrict__ dy,
    const float *__restrict__ stats, float aux_coef, float *__restrict__ dz) {
  __shared__ float sp[kRbTokens][64 * NPL];   // p of the wave's token
  __shared__ float sdp[kRbTokens][64 * NPL];  // dp of the wave's token
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kRbTokens + wv;
  if (t >= T) return;  // no block-wide barrier below
  // Softmax of the token's logits (max subtracted), fp32.
  float z[NPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = lane + 64 * j;
    z[j] = n < N ? logits[t * N + n] : -INFINITY;
    mx = fmaxf(mx, z[j]);
  }
  mx = wave_max(mx);
  float e[NPL], sum = 0.f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = lane + 64 * j;
    e[j] = n < N ? __expf(z[j] - mx) : 0.f;
    sum += e[j];
  }
  sum = wave_sum(sum);
  const float inv = 1.f / sum;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = lane + 64 * j;
    if (n < N) {
      sp[wv][n] = e[j] * inv;
      sdp[wv][n] = aux_coef * stats[n];  // aux term: aux_scale alpha N f_n / T
    }
  }
  // da_s = dy_t . y_perm[row_of(t, s)]: lanes take 8 consecutive columns per
  // step; k accumulators; wave sums in a fixed order.
  // (Register arrays take constant indices only: every slot loop below runs
  // to kRbMaxK with an s < k test.)
  float da[kRbMaxK];
#pragma unroll
  for (int s = 0; s < kRbMaxK; ++s) da[s] = 0.f;
  const uint16_t *dyt = dy + t * d;
  for (int c = 8 * lane; c < d; c += 512) {
    float x[8];
    const uint4 raw = *reinterpret_cast<const uint4 *>(dyt + c);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = __uint_as_float(wds[q] << 16);
      x[2 * q + 1] = __uint_as_float(wds[q] & 0xFFFF0000u);
    }
#pragma unroll
    for (int s = 0; s < kRbMaxK; ++s) {
      if (s >= k) break;
      const int r = row_of[t * k + s];
      if (r < 0) continue;
      const float4 y0 = *reinterpret_cast<const float4 *>(y_perm + (int64_t)r * d + c);
      const float4 y1 = *reinterpret_cast<const float4 *>(y_perm + (int64_t)r * d + c + 4);
      da[s] += x[0] * y0.x + x[1] * y0.y + x[2] * y0.z + x[3] * y0.w + x[4] * y1.x +
               x[5] * y1.y + x[6] * y1.z + x[7] * y1.w;
    }
  }
#pragma unroll
  for (int s = 0; s < kRbMaxK; ++s)
    if (s < k) da[s] = wave_sum(da[s]);
  __builtin_amdgcn_wave_barrier();
  // Gate backward into dp (lanes s < k own slot s; a token names an expert
  // once, so the adds do not collide).
  float ssum = 0.f, dot_da_a = 0.f;
  if (renorm) {
#pragma unroll
    for (int s = 0; s < kRbMaxK; ++s)
      if (s < k) ssum += sp[wv][idx[t * k + s]];
#pragma unroll
    for (int s = 0; s < kRbMaxK; ++s)
      if (s < k) dot_da_a += da[s] * (sp[wv][idx[t * k + s]] / ssum);
  }
  float mine = 0.f;
#pragma unroll
  for (int s = 0; s < kRbMaxK; ++s)
    if (s < k && s == lane) mine = renorm ? (da[s] - dot_da_a) / ssum : da[s];
  if (lane < k) sdp[wv][idx[t * k + lane]] += mine;
  __builtin_amdgcn_wave_barrier();
  // Softmax backward.
  float pd = 0.f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = lane + 64 * j;
    if (n < N) pd += sp[wv][n] * sdp[wv][n];
  }
  pd = wave_sum(pd);
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = lane + 64 * j;
    if (n < N) dz[t * N + n] = sp[wv][n] * (sdp[wv][n] - pd);
  }
}

// Eight bf16 (one 16-byte load) -> fp32.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 raw, float (&x)[8]) {
  const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = __uint_as_float(wds[q] << 16);
    x[2 * q + 1] = __uint_as_float(wds[q] & 0xFFFF0000u);
  }
}

// part[ch][n][c] = sum over tokens t of chunk ch of dz[t][n] * u[t][c]; a
// thread owns columns 8i .. 8i+7 (d % 8 == 0) and the block's 8 experts.
__global__ __launch_bounds__(256) void rb_dw_kernel(const float *__restrict__ dz,
                                                    const uint16_t *__restrict__ u, int64_t T,
                                                    int N, int d, int64_t chunk,
                                                    float *__restrict__ part) {
  __shared__ float sdz[kDwStage * kDwExperts];  // dz of kDwStage tokens
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  const int n0 = blockIdx.y * kDwExperts;
  const int64_t t0 = blockIdx.z * chunk;
  const int64_t t1 = (t0 + chunk) < T ? (t0 + chunk) : T;
  float acc[kDwExperts][8];
#pragma unroll
  for (int j = 0; j < kDwExperts; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[j][q] = 0.f;
  for (int64_t s0 = t0; s0 < t1; s0 += kDwStage) {
    const int nt = (int)((t1 - s0) < kDwStage ? (t1 - s0) : kDwStage);
    __syncthreads();  // the previous stage's reads are done
    for (int i = threadIdx.x; i < nt * kDwExperts; i += 256) {
      const int tt = i / kDwExperts, j = i % kDwExperts;
      sdz[i] = (n0 + j < N) ? dz[(s0 + tt) * N + n0 + j] : 0.f;
    }
    __syncthreads();
    if (c < d) {
      const uint16_t *up = u + s0 * d + c;
#pragma unroll 4
      for (int tt = 0; tt < nt; ++tt) {
        float x[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4 *>(up + (int64_t)tt * d), x);
#pragma unroll
        for (int j = 0; j < kDwExperts; ++j) {
          const float g = sdz[tt * kDwExperts + j];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[j][q] += g * x[q];
        }
      }
    }
  }
  if (c >= d) return;
#pragma unroll
  for (int j = 0; j < kDwExperts; ++j)
    if (n0 + j < N) {
      float *dst = part + ((int64_t)blockIdx.z * N + n0 + j) * d + c;
      *reinterpret_cast<float4 *>(dst) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      *reinterpret_cast<float4 *>(dst + 4) =
          make_float4(acc[j][4], acc[j][5], acc[j][6], acc[j][7]);
    }
}

// dw[i] = sum over the chunks of part[ch][i] in a fixed order: a block owns
// 256 consecutive outputs (a float4 a lane); wave g sums chunks g, g + 16,
// g + 32, ... in order (1 KiB loads, all of a wave's in flight together) and
// the 16 wave sums are added in wave order.
constexpr int kRedWaves = 16;
__global__ __launch_bounds__(64 * kRedWaves) void rb_dw_reduce_kernel(
    const float *__restrict__ part, int64_t chunks, int64_t nd, float *__restrict__ dw) {
  __shared__ float4 sp[kRedWaves][64];
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t i = ((int64_t)blockIdx.x * 64 + lane) * 4;  // nd % 4 == 0
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < nd) {
#pragma unroll 8
    for (int64_t ch = g; ch < chunks; ch += kRedWaves) {
      const float4 p = *reinterpret_cast<const float4 *>(part + ch * nd + i);
      s.x += p.x;
      s.y += p.y;
      s.z += p.z;
      s.w += p.w;
    }
  }
  sp[g][lane] = s;
  __syncthreads();
  if (g != 0 || i >= nd) return;
  float4 t = sp[0][lane];
#pragma unroll
  for (int q = 1; q < kRedWaves; ++q) {
    const float4 p = sp[q][lane];
    t.x += p.x;
    t.y += p.y;
    t.z += p.z;
    t.w += p.w;
  }
  *reinterpret_cast<float4 *>(dw + i) = t;
}

// du[t][c] = sum_n dz[t][n] * W_route[n][c]: a thread owns columns
// 8i .. 8i+7 of kDuTokens tokens.
__global__ __launch_bounds__(256) void rb_du_kernel(const float *__restrict__ dz,
                                                    const uint16_t *__restrict__ w, int64_t T,
                                                    int N, int d, float *__restrict__ du) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  const int64_t t0 = (int64_t)blockIdx.y * kDuTokens;
  if (c >= d) return;
  float acc[kDuTokens][8];
#pragma unroll
  for (int j = 0; j < kDuTokens; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[j][q] = 0.f;
  for (int n = 0; n < N; ++n) {
    float x[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4 *>(w + (int64_t)n * d + c), x);
#pragma unroll
    for (int j = 0; j < kDuTokens; ++j) {
      const float g = (t0 + j < T) ? dz[(t0 + j) * N + n] : 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[j][q] += g * x[q];
    }
  }
#pragma unroll
  for (int j = 0; j < kDuTokens; ++j)
    if (t0 + j < T) {
      float *dst = du + (t0 + j) * d + c;
      *reinterpret_cast<float4 *>(dst) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      *reinterpret_cast<float4 *>(dst + 4) =
          make_float4(acc[j][4], acc[j][5], acc[j][6], acc[j][7]);
    }
}

}  // namespace

int64_t route_bwd_chunks(int64_t T, int N, int d) {
  // Partial-sum chunks of at least kDwChunk tokens, at most 64 MiB of partials.
  const int64_t by_tokens = (T + kDwChunk - 1) / kDwChunk;
  int64_t by_bytes = ((int64_t)64 << 20) / ((int64_t)N * d * 4);
  if (by_bytes < 1) by_bytes = 1;
  return by_tokens < by_bytes ? by_tokens : by_bytes;
}

hipError_t launch_route_backward(const float *logits, int64_t T, int N, int k, int d, int dyw,
                                 int renorm, const int32_t *idx, const int32_t *row_of,
                                 const float *y_perm, const uint16_t *dy, const float *stats,
                                 float aux_coef, const uint16_t *u, const uint16_t *w_route,
                                 float *part, float *dz, float *dw, float *du, hipStream_t st) {
  const dim3 g1((unsigned)((T + kRbTokens - 1) / kRbTokens)), b1(64 * kRbTokens);
#define MOE_RB_CASE(NPLV)                                                                  \
  hipLaunchKernelGGL(rb_dz_kernel<NPLV>, g1, b1, 0, st, logits, T, N, k, dyw, renorm, idx, \
                     row_of, y_perm, dy, stats, aux_coef, dz)
  if (N <= 64) MOE_RB_CASE(1);
  else if (N <= 256) MOE_RB_CASE(4);
  else MOE_RB_CASE(16);
#undef MOE_RB_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t chunks = route_bwd_chunks(T, N, d);
  const int64_t chunk = (T + chunks - 1) / chunks;
  hipLaunchKernelGGL(rb_dw_kernel, dim3((unsigned)((d / 8 + 255) / 256),
                                        (unsigned)((N + kDwExperts - 1) / kDwExperts),
                                        (unsigned)chunks),
                     dim3(256), 0, st, dz, u, T, N, d, chunk, part);
  const int64_t nd = (int64_t)N * d;
  hipLaunchKernelGGL(rb_dw_reduce_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(64 * kRedWaves),
                     0, st, part, chunks, nd, dw);
  hipLaunchKernelGGL(rb_du_kernel, dim3((unsigned)((d / 8 + 255) / 256),
                                        (unsigned)((T + kDuTokens - 1) / kDuTokens)),
                     dim3(256), 0, st, dz, w_route, T, N, d, du);
  return hipGetLastError();
}

}  // namespace moe
