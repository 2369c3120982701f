// The experts' backward (page "MoE: how sparse activation saves compute",
// §3.1 eq. F and §3.2 eq. y, differentiated): for each kept row of expert i
// with token t and weight a,
//   dY = a dy_t;  G = W_gate x, U = W_up x (recomputed);
//   dH = W_down^T dY;  (dG, dU) = act'(G, U) dH;
//   dx_t += W_gate^T dG + W_up^T dU;
//   dW_down += dY act(G, U)^T;  dW_gate += dG x^T;  dW_up += dU x^T.
// The products run on the grouped GEMM: dH and (dG, dU) in one launch whose
// epilogue applies the activation's backward, dx rows against W_gate | W_up
// (both of these read the weights as stored, through the GEMM's
// transposed-B mode), and the weight gradients as "K segment" GEMMs that
// reduce over each expert's own rows.  This file holds the data movement
// around them:
//   bwd_gather_dy_kernel: dY rows (a dy_t) in the expert-sorted row order;
//   transpose_bf16_kernel: [B][R][C] -> [B][C][ld] at a column offset, 64x64
//     tiles through LDS with 16-byte loads and stores (the latent layer's
//     token-long operands and projection matrices);
//   kseg_kernel: each expert's rows padded to a multiple of 64 (at least
//     128: two k-steps of the GEMM), as a prefix of column offsets;
//   seg_transpose_kernel: row-major [rows][width] -> [width][Rpad], row r of
//     expert g to column kseg[g] + r - kept_offsets[g] and zeros in the rest
//     of the expert's padded segment (tiled over the destination columns,
//     16-byte loads and stores); optionally gathered token rows (x) or
//     act(G, U) computed on the way;
//   fill_zero_kernel, rows_sum_kernel (dx_t = sum of its kept rows).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void bwd_gather_dy_kernel(const uint16_t *__restrict__ dy,
                                                            int d, int k,
                                                            const int32_t *__restrict__ row_of,
                                                            const float *__restrict__ topk_w,
                                                            uint16_t *__restrict__ dy_perm) {
  const int64_t ent = blockIdx.x;
  const int r = row_of[ent];
  if (r < 0) return;
  const float a = topk_w[ent];
  const uint16_t *src = dy + (ent / k) * (int64_t)d;
  uint16_t *dst = dy_perm + (int64_t)r * d;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(src + c);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint4 o;
    uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ow[q] = pack_bf16x2_hw(a * __uint_as_float(w[q] << 16),
                             a * __uint_as_float(w[q] & 0xFFFF0000u));
    *reinterpret_cast<uint4 *>(dst + c) = o;
  }
}

// dst[b][c][col0 + r] = src[b][r][c]: src [B][R][C], dst rows of length ld
// (C, ld and col0 multiples of 8).  A 64x64 tile per block: 16-byte row
// loads into LDS (pitch 66 halves: the column reads below hit distinct
// banks), 16-byte stores of 8 consecutive source rows of one column.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ src,
                                                             int R, int C,
                                                             uint16_t *__restrict__ dst,
                                                             int64_t ld, int col0) {
  __shared__ uint32_t tile[64 * 33];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t *s = src + (int64_t)b * R * C;
  uint16_t *o = dst + (int64_t)b * C * ld;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + 256 * h;
    const int r = i >> 3, c8 = (i & 7) << 3;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + r < R && c0 + c8 < C)
      v = *reinterpret_cast<const uint4 *>(s + (int64_t)(r0 + r) * C + c0 + c8);
    uint32_t *t = tile + r * 33 + (c8 >> 1);
    t[0] = v.x;
    t[1] = v.y;
    t[2] = v.z;
    t[3] = v.w;
  }
  __syncthreads();
  const uint16_t *th = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + 256 * h;
    const int cc = i >> 3, r8 = (i & 7) << 3;
    if (c0 + cc >= C || r0 + r8 >= R) continue;
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = th[(r8 + j) * 66 + cc];
    uint16_t *out = o + (int64_t)(c0 + cc) * ld + col0 + r0 + r8;
    if (r0 + r8 + 8 <= R) {
      uint4 w;
      w.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
      w.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
      w.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
      w.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
      *reinterpret_cast<uint4 *>(out) = w;
    } else {
      for (int j = 0; j < R - r0 - r8; ++j) out[j] = e[j];
    }
  }
}

// kseg[g] = sum over g' < g of max(128, 64 ceil(m_g' / 64)), m = kept rows (a
// LatentMoE expert's ~146 rows pad to 192, not 256: a quarter fewer MFMAs in
// its weight gradients).
__global__ __launch_bounds__(1024) void kseg_kernel(const int32_t *__restrict__ kept_offsets,
                                                    int G, int32_t *__restrict__ kseg) {
  __shared__ int tmp[1024];
  int run = 0;
  for (int base = 0; base < G; base += 1024) {
    const int g = base + threadIdx.x;
    const int m = (g < G) ? kept_offsets[g + 1] - kept_offsets[g] : 0;
    tmp[threadIdx.x] = (g < G) ? (m > 64 ? 64 * ((m + 63) / 64) : 128) : 0;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int add = (int)threadIdx.x >= o ? tmp[threadIdx.x - o] : 0;
      __syncthreads();
      tmp[threadIdx.x] += add;
      __syncthreads();
    }
    if (g < G) kseg[g + 1] = run + tmp[threadIdx.x];
    run += tmp[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) kseg[0] = 0;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4 *__restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// Rows r of the expert-sorted layout (R rows) to columns of dst [width][ld]:
// expert g = the group with kept_offsets[g] <= r < kept_offsets[g+1], column
// kseg[g] + r - kept_offsets[g].  Source row: r (src, row stride lds), or the
// token row perm[offsets[g] + j] / kslots when perm is given; with src2 the
// value is act(src, src2) (the hidden of the recomputed gate and up).
__global__ __launch_bounds__(256) void seg_transpose_kernel(
    const uint16_t *__restrict__ src, const uint16_t *__restrict__ src2, int64_t lds, int width,
    const int32_t *__restrict__ kept_offsets, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, int kslots, const int32_t *__restrict__ kseg, int G,
    int act, float bg, float bu, uint16_t *__restrict__ dst, int64_t ld) {
  __shared__ uint32_t tile[64 * 33];
  // This block's 64 destination columns lie in one expert's padded segment
  // (segments are multiples of 64 wide).
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (p0 >= kseg[G]) return;
  int lo = 0, hi = G;  // largest g with kseg[g] <= p0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (kseg[mid] <= p0) lo = mid; else hi = mid;
  }
  const int m = kept_offsets[lo + 1] - kept_offsets[lo];
  const int j0 = p0 - kseg[lo];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + 256 * h;
    const int r = i >> 3, c8 = (i & 7) << 3;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (j0 + r < m && c0 + c8 < width) {
      const int j = j0 + r;
      const int64_t row = perm ? (int64_t)(perm[offsets[lo] + j] / kslots)
                               : (int64_t)(kept_offsets[lo] + j);
      const int64_t at = row * lds + c0 + c8;
      v = *reinterpret_cast<const uint4 *>(src + at);
      if (src2 != nullptr) {
        const uint4 w = *reinterpret_cast<const uint4 *>(src2 + at);
        const uint32_t gv[4] = {v.x, v.y, v.z, v.w}, uv[4] = {w.x, w.y, w.z, w.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = pack_bf16x2_hw(
              glu_act(__uint_as_float(gv[q] << 16), __uint_as_float(uv[q] << 16), act, bg, bu),
              glu_act(__uint_as_float(gv[q] & 0xFFFF0000u), __uint_as_float(uv[q] & 0xFFFF0000u),
                      act, bg, bu));
        v = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    uint32_t *t = tile + r * 33 + (c8 >> 1);
    t[0] = v.x;
    t[1] = v.y;
    t[2] = v.z;
    t[3] = v.w;
  }
  __syncthreads();
  const uint16_t *th = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + 256 * h;
    const int cc = i >> 3, r8 = (i & 7) << 3;
    if (c0 + cc >= width) continue;
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = th[(r8 + j) * 66 + cc];
    uint4 w;
    w.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    w.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    w.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    w.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<uint4 *>(dst + (int64_t)(c0 + cc) * ld + p0 + r8) = w;
  }
}

// dx[t][c] = sum over the kept slots of t of rows[row_of[t*k + s]][c], fp32.
__global__ __launch_bounds__(256) void rows_sum_kernel(const float *__restrict__ rows, int d,
                                                       int k, const int32_t *__restrict__ row_of,
                                                       float *__restrict__ dx) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < k; ++s) {
      const int r = row_of[t * k + s];
      if (r < 0) continue;
      const float4 v = *reinterpret_cast<const float4 *>(rows + (int64_t)r * d + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4 *>(dx + t * d + c) = acc;
  }
}

}  // namespace

hipError_t launch_bwd_gather_dy(const uint16_t *dy, int64_t T, int d, int k,
                                const int32_t *row_of, const float *topk_w, uint16_t *dy_perm,
                                hipStream_t st) {
  hipLaunchKernelGGL(bwd_gather_dy_kernel, dim3((unsigned)(T * k)), dim3(256), 0, st, dy, d, k,
                     row_of, topk_w, dy_perm);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t *src, int B, int R, int C, uint16_t *dst,
                                 int64_t ld, int col0, hipStream_t st) {
  if (C % 8 != 0 || ld % 8 != 0 || col0 % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((C + 63) / 64),
                                                 (unsigned)((R + 63) / 64), (unsigned)B),
                     dim3(256), 0, st, src, R, C, dst, ld, col0);
  return hipGetLastError();
}

hipError_t launch_kseg(const int32_t *kept_offsets, int G, int32_t *kseg, hipStream_t st) {
  hipLaunchKernelGGL(kseg_kernel, dim3(1), dim3(1024), 0, st, kept_offsets, G, kseg);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<uint4 *>(p), n16);
  return hipGetLastError();
}

hipError_t launch_seg_transpose(const uint16_t *src, const uint16_t *src2, int64_t lds,
                                int width, const int32_t *kept_offsets,
                                const int32_t *offsets, const int32_t *perm, int kslots,
                                const int32_t *kseg, int G, int act, float bg, float bu,
                                uint16_t *dst, int64_t ld, hipStream_t st) {
  if (width % 8 != 0 || lds % 8 != 0 || ld % 64 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(seg_transpose_kernel, dim3((unsigned)((width + 63) / 64),
                                                (unsigned)(ld / 64)),
                     dim3(256), 0, st, src, src2, lds, width, kept_offsets, offsets, perm,
                     kslots, kseg, G, act, bg, bu, dst, ld);
  return hipGetLastError();
}

hipError_t launch_rows_sum(const float *rows, int64_t T, int d, int k, const int32_t *row_of,
                           float *dx, hipStream_t st) {
  hipLaunchKernelGGL(rows_sum_kernel, dim3((unsigned)T), dim3(256), 0, st, rows, d, k, row_of,
                     dx);
  return hipGetLastError();
}

}  // namespace moe
