// fp32 expert projections on the vector ALUs (any shape).  Used when the
// activations and weights are fp32; one thread per (row, column) output,
// sequential fp32 FMA over K.  Same grouping as the MFMA path: expert e works
// on its kept rows, x rows gathered through perm (page "MoE: how sparse
// activation saves compute", sections 3.1 and 3.6).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void simt_gu_kernel(
    const float *__restrict__ x, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ kept_offsets, int kslots,
    const float *__restrict__ Wg, const float *__restrict__ Wu, int w, int h, int act, float bg,
    float bu, float *__restrict__ hid) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int M = kept_offsets[e + 1] - kept_offsets[e];
  if (c >= h) return;
  const float *wg = Wg + ((int64_t)e * h + c) * w;
  const float *wu = Wu + ((int64_t)e * h + c) * w;
  for (int j = threadIdx.x >> 6; j < M; j += 4) {
    const int64_t t = perm[offsets[e] + j] / kslots;
    const float *xr = x + t * w;
    float g = 0.f, v = 0.f;
    for (int kk = 0; kk < w; ++kk) {
      g = fmaf(xr[kk], wg[kk], g);
      v = fmaf(xr[kk], wu[kk], v);
    }
    hid[(int64_t)(kept_offsets[e] + j) * h + c] = glu_act(g, v, act, bg, bu);
  }
}

__global__ __launch_bounds__(256) void simt_down_kernel(const float *__restrict__ hid,
                                                        const int32_t *__restrict__ kept_offsets,
                                                        const float *__restrict__ Wd, int h, int w,
                                                        float *__restrict__ y_perm) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int M = kept_offsets[e + 1] - kept_offsets[e];
  if (c >= w) return;
  const float *wd = Wd + ((int64_t)e * w + c) * h;
  for (int j = threadIdx.x >> 6; j < M; j += 4) {
    const int64_t row = kept_offsets[e] + j;
    const float *hr = hid + row * h;
    float acc = 0.f;
    for (int kk = 0; kk < h; ++kk) acc = fmaf(hr[kk], wd[kk], acc);
    y_perm[row * w + c] = acc;
  }
}

}  // namespace

hipError_t launch_simt_gu(const float *x, const int32_t *perm, const int32_t *offsets,
                          const int32_t *kept_offsets, int kslots, const float *Wg,
                          const float *Wu, int w, int h, int N, int act, float bg, float bu,
                          float *hid, hipStream_t st) {
  hipLaunchKernelGGL(simt_gu_kernel, dim3((h + 63) / 64, N), dim3(256), 0, st, x, perm, offsets,
                     kept_offsets, kslots, Wg, Wu, w, h, act, bg, bu, hid);
  return hipGetLastError();
}

hipError_t launch_simt_down(const float *hid, const int32_t *kept_offsets, const float *Wd,
                            int h, int w, int N, float *y_perm, hipStream_t st) {
  hipLaunchKernelGGL(simt_down_kernel, dim3((w + 63) / 64, N), dim3(256), 0, st, hid,
                     kept_offsets, Wd, h, w, y_perm);
  return hipGetLastError();
}

}  // namespace moe
