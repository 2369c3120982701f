// The LatentMoE layer's backward (page "Stable LatentMoE interactive demo":
// the width-separation and RMSNorm passages, differentiated).  With the
// aggregated r = sum_kept a E_i(x_l), n = r / rho, rho = sqrt(mean(r^2) + eps)
// and y = W_lup n + shared experts:
//   dn = dy W_lup;  dr = (dn - n mean(dn * n)) / rho;
// dr then feeds the routed experts' backward (at width l) and the router's.
// The products run on the grouped GEMM; this file holds the per-token and
// elementwise steps around them:
//   rms_bwd_kernel:      one workgroup per token: r from the kept expert
//                        rows (as the forward's combine), rho, n, and dr;
//                        writes dr and n (bf16, n rounded exactly as the
//                        forward rounded it before W_lup);
//   cast_bf16_kernel:    fp32 -> bf16 (round to nearest even);
//   add_f32_kernel:      dst += src;
//   shared_route_kernel: the shared experts as a routing in which every token
//                        takes every shared expert with weight 1, so the
//                        routed experts' backward runs them unchanged.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kVPT = 4;  // float4 per thread: width <= 4096

__device__ __forceinline__ float block_sum(float v, float *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void rms_bwd_kernel(const float *__restrict__ y_perm,
                                                           const int32_t *__restrict__ row_of,
                                                           const float *__restrict__ topk_w,
                                                           int k, int width, float eps,
                                                           const float *__restrict__ dn,
                                                           uint16_t *__restrict__ dr,
                                                           uint16_t *__restrict__ n_out) {
  __shared__ float red[kThreads];
  const int64_t t = blockIdx.x;
  const int nv = width / 4;
  float4 acc[kVPT], g[kVPT];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < kVPT; ++it) {
    const int v = it * kThreads + threadIdx.x;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    g[it] = a;
    if (v < nv) {
      for (int s = 0; s < k; ++s) {
        const int r = row_of[t * k + s];
        if (r < 0) continue;
        const float wt = topk_w[t * k + s];
        const float4 x = *reinterpret_cast<const float4 *>(y_perm + (int64_t)r * width + 4 * v);
        a.x = fmaf(wt, x.x, a.x);
        a.y = fmaf(wt, x.y, a.y);
        a.z = fmaf(wt, x.z, a.z);
        a.w = fmaf(wt, x.w, a.w);
      }
      g[it] = reinterpret_cast<const float4 *>(dn + t * width)[v];
    }
    acc[it] = a;
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  const float scale = 1.0f / sqrtf(block_sum(ss, red) / (float)width + eps);
  float dot = 0.f;
#pragma unroll
  for (int it = 0; it < kVPT; ++it) {
    const float4 a = acc[it], b = g[it];
    dot += (a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w) * scale;
  }
  const float c = block_sum(dot, red) / (float)width;
#pragma unroll
  for (int it = 0; it < kVPT; ++it) {
    const int v = it * kThreads + threadIdx.x;
    if (v >= nv) break;
    const float4 a = acc[it], b = g[it];
    const float n0 = a.x * scale, n1 = a.y * scale, n2 = a.z * scale, n3 = a.w * scale;
    uint2 pk;
    pk.x = pack_bf16x2(n0, n1);
    pk.y = pack_bf16x2(n2, n3);
    reinterpret_cast<uint2 *>(n_out + t * width)[v] = pk;
    pk.x = pack_bf16x2((b.x - n0 * c) * scale, (b.y - n1 * c) * scale);
    pk.y = pack_bf16x2((b.z - n2 * c) * scale, (b.w - n3 * c) * scale);
    reinterpret_cast<uint2 *>(dr + t * width)[v] = pk;
  }
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float *__restrict__ src, int64_t n4,
                                                        uint16_t *__restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4 *>(src)[i];
  uint2 pk;
  pk.x = pack_bf16x2(v.x, v.y);
  pk.y = pack_bf16x2(v.z, v.w);
  reinterpret_cast<uint2 *>(dst)[i] = pk;
}

__global__ __launch_bounds__(256) void add_f32_kernel(float *__restrict__ dst,
                                                      const float *__restrict__ src, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 a = reinterpret_cast<float4 *>(dst)[i];
  const float4 b = reinterpret_cast<const float4 *>(src)[i];
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
  reinterpret_cast<float4 *>(dst)[i] = a;
}

// Entry e = t * S + j (token t, shared expert j): weight 1, row j * T + t.
__global__ __launch_bounds__(256) void shared_route_kernel(int64_t T, int S,
                                                           float *__restrict__ w,
                                                           int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ row_of,
                                                           int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ kept_offsets) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e <= S) {
    offsets[e] = (int32_t)(e * T);
    kept_offsets[e] = (int32_t)(e * T);
  }
  if (e >= T * S) return;
  const int64_t t = e / S, j = e % S;
  w[e] = 1.f;
  row_of[e] = (int32_t)(j * T + t);
  perm[j * T + t] = (int32_t)e;
}

unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_rms_backward(const float *y_perm, const int32_t *row_of, const float *topk_w,
                               int64_t T, int k, int width, float eps, const float *dn,
                               uint16_t *dr, uint16_t *n_out, hipStream_t st) {
  hipLaunchKernelGGL(rms_bwd_kernel, dim3((unsigned)T), dim3(kThreads), 0, st, y_perm, row_of,
                     topk_w, k, width, eps, dn, dr, n_out);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float *src, int64_t n, uint16_t *dst, hipStream_t st) {
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(blocks(n / 4)), dim3(256), 0, st, src, n / 4, dst);
  return hipGetLastError();
}

hipError_t launch_add_f32(float *dst, const float *src, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(add_f32_kernel, dim3(blocks(n / 4)), dim3(256), 0, st, dst, src, n / 4);
  return hipGetLastError();
}

hipError_t launch_shared_route(int64_t T, int S, float *w, int32_t *perm, int32_t *row_of,
                               int32_t *offsets, int32_t *kept_offsets, hipStream_t st) {
  const int64_t n = T * S > S + 1 ? T * S : S + 1;
  hipLaunchKernelGGL(shared_route_kernel, dim3(blocks(n)), dim3(256), 0, st, T, S, w, perm,
                     row_of, offsets, kept_offsets);
  return hipGetLastError();
}

}  // namespace moe
