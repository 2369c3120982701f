// Quantile Balancing (page "Stable LatentMoE interactive demo", QB passage).
// With token t's cutoff a_t held fixed, expert j admits t exactly when
// z_tj + b_j >= a_t, so the bias that admits q tokens is the q-th smallest
// of required_tj = a_t - z_tj over the tokens.  Here a_t is the k-th largest
// of z_t + b under the current bias and the score is the router logit.
//
//   qb_required_kernel: a block of 16 waves takes 16 tokens (one per wave),
//     finds each cutoff with k rounds of a wave arg-max and writes required
//     expert-major ([N][T]) through an LDS tile, 16 tokens per expert row.
//   qb_quantile_kernel: a block per expert.  Exact: a radix select over
//     order-preserving 32-bit keys, 8 bits per pass.  Histogram: min and max,
//     then 256 equal bins, the q-th value placed by linear interpolation in
//     its bin.  Counts use LDS integer atomics (order-free), so the result
//     does not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kQbTokens = 16;   // tokens (waves) per block
constexpr int kQbMaxN = 1024;
constexpr int kQbThreads = 256; // quantile block
constexpr int kQbBins = 256;

template <int NPL>
__global__ __launch_bounds__(64 * kQbTokens) void qb_required_kernel(
    const float *__restrict__ logits, int64_t T, int N, int k, const float *__restrict__ bias,
    float *__restrict__ req) {
  __shared__ float tile[kQbMaxN][kQbTokens];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kQbTokens;
  const int64_t t = t0 + wv;
  if (t < T) {
    float z[NPL], s[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = lane + 64 * j;
      z[j] = (n < N) ? logits[t * N + n] : 0.f;
      s[j] = (n < N) ? z[j] + (bias != nullptr ? bias[n] : 0.f) : -INFINITY;
    }
    // k-th largest of s: k rounds, each removing the current maximum (ties:
    // lower index; the value of the k-th order statistic does not depend on
    // which of equal scores goes first).
    uint32_t taken = 0;
    float kth = -INFINITY;
    for (int sl = 0; sl < k; ++sl) {
      float bs = -INFINITY;
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        if (n < N && !((taken >> j) & 1u) && (bn == 0x7FFFFFFF || s[j] > bs)) {
          bs = s[j];
          bn = n;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float os = __shfl_xor(bs, o, 64);
        const int on = __shfl_xor(bn, o, 64);
        if (os > bs || (os == bs && on < bn)) {
          bs = os;
          bn = on;
        }
      }
      if ((bn & 63) == lane) taken |= 1u << (bn >> 6);
      kth = bs;
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = lane + 64 * j;
      if (n < N) tile[n][wv] = kth - z[j];
    }
  }
  __syncthreads();
  const int ntok = (T - t0) < kQbTokens ? (int)(T - t0) : kQbTokens;
  for (int i = threadIdx.x; i < N * kQbTokens; i += 64 * kQbTokens) {
    const int n = i / kQbTokens, tl = i % kQbTokens;
    if (tl < ntok) req[(int64_t)n * T + t0 + tl] = tile[n][tl];
  }
}

// Order-preserving key of a float (no NaN): larger float -> larger key.
__device__ __forceinline__ uint32_t fkey(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Wave 0 finds the first bin whose running count reaches `rank` (1-based):
// lanes own 4 bins each, an inclusive scan over the lanes' totals locates
// the lane, the lane walks its bins.  Writes the bin and the count of the
// bins before it to out[0], out[1].
__device__ void find_rank_bin(const int *hist, int rank, int *out) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
            c3 = hist[4 * lane + 3];
  const int mine = c0 + c1 + c2 + c3;
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int excl = incl - mine;
  const uint64_t hit = __ballot(incl >= rank);
  const int owner = __ffsll((unsigned long long)hit) - 1;
  if (lane == owner) {
    int run = excl, bin = 4 * lane;
    const int c[4] = {c0, c1, c2, c3};
    for (int i = 0; i < 4; ++i) {
      if (run + c[i] >= rank) {
        bin = 4 * lane + i;
        break;
      }
      run += c[i];
    }
    out[0] = bin;
    out[1] = run;
  }
}

template <int METHOD>
__global__ __launch_bounds__(kQbThreads) void qb_quantile_kernel(const float *__restrict__ req,
                                                                 int64_t T, int q,
                                                                 float *__restrict__ out) {
  __shared__ int hist[kQbBins];
  __shared__ int found[2];
  __shared__ float red_lo[kQbThreads / 64], red_hi[kQbThreads / 64];
  const int n = blockIdx.x;
  const float *col = req + (int64_t)n * T;
  const int tid = threadIdx.x;
  if constexpr (METHOD == 0) {
    // Exact: the q-th smallest key, one byte per pass from the top.
    uint32_t prefix = 0, pmask = 0;
    int rank = q;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < kQbBins; i += kQbThreads) hist[i] = 0;
      __syncthreads();
      for (int64_t i = tid; i < T; i += kQbThreads) {
        const uint32_t key = fkey(col[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1);
      }
      __syncthreads();
      find_rank_bin(hist, rank, found);
      __syncthreads();
      prefix |= (uint32_t)found[0] << shift;
      pmask |= 0xFFu << shift;
      rank -= found[1];
      __syncthreads();
    }
    if (tid == 0) out[n] = fkey_inv(prefix);
  } else {
    // Histogram estimate over [min, max].
    float lo = INFINITY, hi = -INFINITY;
    for (int64_t i = tid; i < T; i += kQbThreads) {
      const float v = col[i];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o, 64));
      hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    if ((tid & 63) == 0) {
      red_lo[tid >> 6] = lo;
      red_hi[tid >> 6] = hi;
    }
    for (int i = tid; i < kQbBins; i += kQbThreads) hist[i] = 0;
    __syncthreads();
    lo = red_lo[0];
    hi = red_hi[0];
#pragma unroll
    for (int w = 1; w < kQbThreads / 64; ++w) {
      lo = fminf(lo, red_lo[w]);
      hi = fmaxf(hi, red_hi[w]);
    }
    if (!(hi > lo)) {
      if (tid == 0) out[n] = lo;
      return;
    }
    const float width = (hi - lo) / (float)kQbBins;
    for (int64_t i = tid; i < T; i += kQbThreads) {
      int b = (int)floorf((col[i] - lo) / width);
      b = b < 0 ? 0 : (b > kQbBins - 1 ? kQbBins - 1 : b);
      atomicAdd(&hist[b], 1);
    }
    __syncthreads();
    find_rank_bin(hist, q, found);
    __syncthreads();
    if (tid == 0) {
      const int m = found[0], before = found[1];
      out[n] = lo + width * ((float)m + (float)(q - before) / (float)hist[m]);
    }
  }
}

}  // namespace

hipError_t launch_qb_update(const float *logits, int64_t T, int N, int k, const float *bias, int q,
                            int method, float *req, float *new_bias, hipStream_t st) {
  const dim3 g1((unsigned)((T + kQbTokens - 1) / kQbTokens)), b1(64 * kQbTokens);
  if (N <= 256)
    hipLaunchKernelGGL(qb_required_kernel<4>, g1, b1, 0, st, logits, T, N, k, bias, req);
  else if (N <= 512)
    hipLaunchKernelGGL(qb_required_kernel<8>, g1, b1, 0, st, logits, T, N, k, bias, req);
  else
    hipLaunchKernelGGL(qb_required_kernel<16>, g1, b1, 0, st, logits, T, N, k, bias, req);
  if (method == 0)
    hipLaunchKernelGGL(qb_quantile_kernel<0>, dim3(N), dim3(kQbThreads), 0, st, req, T, q,
                       new_bias);
  else
    hipLaunchKernelGGL(qb_quantile_kernel<1>, dim3(N), dim3(kQbThreads), 0, st, req, T, q,
                       new_bias);
  return hipGetLastError();
}

}  // namespace moe
