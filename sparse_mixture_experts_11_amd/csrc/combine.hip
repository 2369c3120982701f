// Weighted combine (page "MoE: how sparse activation saves compute", section
// 3.2 eq. for y_t; section 3.5: an overflowing slot contributes nothing): one
// workgroup per token gathers the token's kept expert rows and sums them in
// slot order in fp32 -- no atomics, so the result is deterministic.
// With rmsnorm set (latent layer, page "Stable LatentMoE interactive demo",
// RMSNorm passage) the sum r is scaled by 1 / sqrt(mean(r^2) + eps) before the
// single rounding to the output dtype.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kVPT = 4;  // float4 per thread kept for the norm: width <= 4096

template <bool BF16OUT, bool RMS>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ y_perm,
                                                           const int32_t *__restrict__ row_of,
                                                           const float *__restrict__ topk_w,
                                                           int k, int width, float eps,
                                                           void *__restrict__ y) {
  __shared__ float red[kThreads];
  const int64_t t = blockIdx.x;
  const int nv = width / 4;
  float4 acc[kVPT];
  float ss = 0.f;
  for (int it = 0; it * kThreads < nv; ++it) {
    const int v = it * kThreads + threadIdx.x;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
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
    }
    if constexpr (RMS) {
      acc[it] = a;
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    } else if (v < nv) {
      if constexpr (BF16OUT) {
        uint2 pk;
        pk.x = pack_bf16x2(a.x, a.y);
        pk.y = pack_bf16x2(a.z, a.w);
        reinterpret_cast<uint2 *>(y)[t * nv + v] = pk;
      } else {
        reinterpret_cast<float4 *>(y)[t * nv + v] = a;
      }
    }
  }
  if constexpr (RMS) {
    red[threadIdx.x] = ss;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
      __syncthreads();
    }
    const float scale = 1.0f / sqrtf(red[0] / (float)width + eps);
    for (int it = 0; it * kThreads < nv; ++it) {
      const int v = it * kThreads + threadIdx.x;
      if (v >= nv) break;
      const float4 a = acc[it];
      if constexpr (BF16OUT) {
        uint2 pk;
        pk.x = pack_bf16x2(a.x * scale, a.y * scale);
        pk.y = pack_bf16x2(a.z * scale, a.w * scale);
        reinterpret_cast<uint2 *>(y)[t * nv + v] = pk;
      } else {
        reinterpret_cast<float4 *>(y)[t * nv + v] =
            make_float4(a.x * scale, a.y * scale, a.z * scale, a.w * scale);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const float *y_perm, const int32_t *row_of, const float *topk_w,
                          int64_t T, int k, int width, bool out_bf16, bool rmsnorm, float eps,
                          void *y, hipStream_t st) {
  const dim3 grid((unsigned)T), block(kThreads);
  if (rmsnorm) {
    if (out_bf16)
      hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, st, y_perm, row_of, topk_w,
                         k, width, eps, y);
    else
      hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, st, y_perm, row_of, topk_w,
                         k, width, eps, y);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, st, y_perm, row_of, topk_w,
                         k, width, eps, y);
    else
      hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, st, y_perm, row_of, topk_w,
                         k, width, eps, y);
  }
  return hipGetLastError();
}

}  // namespace moe
