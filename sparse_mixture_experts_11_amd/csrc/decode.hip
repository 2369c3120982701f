// Decode-sized experts: few tokens per expert, so the projections are bound
// by reading the selected experts' weights once (page "Kestrel-MCU notes #13:
// the MoE deployment gap", section 二: experts are stored grouped and looked
// up by index, and only the selected experts' weights are read).
//
// Each workgroup owns 32 weight rows of one expert and all K; its 4 waves
// split K, stream the rows straight from HBM into MFMA operands
// (v_mfma_f32_16x16x32_bf16: 16 weight rows x up to 16 tokens per group; each
// token fragment feeds both 16-row blocks of the wave), and reduce their
// partial sums through LDS in a fixed order.  Experts with
// no kept token exit before touching their weights.
//   GLU = true : hid[row] = act(W_gate x, W_up x), x rows gathered via perm
//   GLU = false: y_perm[row] = W_down hid[row], fp32
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int NRB = 2;          // 16-row weight blocks per wave (token fragments reused NRB x)
constexpr int RB = 16 * NRB;    // weight rows per workgroup
constexpr int kWaves = 4;       // split-K ways
// k-steps of 32 per unrolled iteration (weight bytes in flight per wave:
// 2 KiB x NRB x matrices x U).
template <bool GLU>
constexpr int unroll_of() { return GLU ? 4 : 8; }

template <bool GLU, int TG>
__global__ __launch_bounds__(256) void decode_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ kept_offsets, int kslots,
    const uint16_t *__restrict__ W1, const uint16_t *__restrict__ W2, int64_t wrows, int K,
    int act, float bg, float bu, void *__restrict__ out, int64_t ldo) {
  constexpr int NM = GLU ? 2 : 1;
  __shared__ f32x4 red[kWaves - 1][NM][NRB][TG][64];
  const int e = blockIdx.y;
  const int M = kept_offsets[e + 1] - kept_offsets[e];
  if (M == 0) return;
  const int row0 = blockIdx.x * RB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;           // weight row within block / token within group
  const int kq = (lane >> 4) * 8;     // k offset of this lane's 8 values
  const int Kw = K / kWaves;
  const int kb = wave * Kw;

  const uint16_t *w1 = W1 + ((int64_t)e * wrows + row0 + li) * K + kb + kq;
  const uint16_t *w2 = GLU ? W2 + ((int64_t)e * wrows + row0 + li) * K + kb + kq : nullptr;
  const int64_t rbs = (int64_t)16 * K;  // next 16-row block
  const uint16_t *xr[TG];
  bool xv[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int j = tg * 16 + li;
    xv[tg] = j < M;
    int64_t row;
    if (GLU) row = xv[tg] ? perm[offsets[e] + j] / kslots : 0;
    else row = kept_offsets[e] + (xv[tg] ? j : 0);
    xr[tg] = x + row * ldx + kb + kq;
  }
  const int ngroups = (M + 15) / 16;

  f32x4 acc[NM][NRB][TG];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) acc[m][r][tg] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  constexpr int U = unroll_of<GLU>();
  int k = 0;
  for (; k + 32 * U <= Kw; k += 32 * U) {
    bf16x8 a[NM][NRB][U], b[TG][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        a[0][r][u] = *reinterpret_cast<const bf16x8 *>(w1 + r * rbs + k + 32 * u);
        if (GLU) a[NM - 1][r][u] = *reinterpret_cast<const bf16x8 *>(w2 + r * rbs + k + 32 * u);
      }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[tg][u] = (tg < ngroups && xv[tg]) ? *reinterpret_cast<const bf16x8 *>(xr[tg] + k + 32 * u)
                                           : zero;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if (tg < ngroups) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < NRB; ++r)
              acc[m][r][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][r][u], b[tg][u],
                                                                     acc[m][r][tg], 0, 0, 0);
      }
    }
  }
  for (; k < Kw; k += 32) {
    bf16x8 a[NM][NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      a[0][r] = *reinterpret_cast<const bf16x8 *>(w1 + r * rbs + k);
      if (GLU) a[NM - 1][r] = *reinterpret_cast<const bf16x8 *>(w2 + r * rbs + k);
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if (tg < ngroups) {
        const bf16x8 b = xv[tg] ? *reinterpret_cast<const bf16x8 *>(xr[tg] + k) : zero;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < NRB; ++r)
            acc[m][r][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][r], b, acc[m][r][tg], 0,
                                                                   0, 0);
      }
    }
  }

  // Fixed-order split-K reduction: wave 0 adds waves 1, 2, 3 in turn.
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) red[wave - 1][m][r][tg][lane] = acc[m][r][tg];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[m][r][tg] += red[w][m][r][tg][lane];
  // Lane holds rows row0 + 16r + 4*(lane/16) + {0..3} of token tg*16 + lane%16.
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int j = tg * 16 + li;
    if (tg >= ngroups || j >= M) continue;
    const int64_t orow = kept_offsets[e] + j;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int col = row0 + 16 * r + 4 * (lane >> 4);
      if constexpr (GLU) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = glu_act_fast(acc[0][r][tg][q], acc[1][r][tg][q], act, bg, bu);
        uint2 pk;
        pk.x = pack_bf16x2_hw(v[0], v[1]);
        pk.y = pack_bf16x2_hw(v[2], v[3]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + orow * ldo + col) = pk;
      } else {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + orow * ldo + col) =
            acc[0][r][tg];
      }
    }
  }
}

template <bool GLU>
hipError_t launch_decode(int tg, dim3 grid, hipStream_t st, const uint16_t *x, int64_t ldx,
                         const int32_t *perm, const int32_t *offsets, const int32_t *kept_offsets,
                         int kslots, const uint16_t *W1, const uint16_t *W2, int64_t wrows, int K,
                         int act, float bg, float bu, void *out, int64_t ldo) {
#define MOE_DECODE_CASE(TGV)                                                                     \
  case TGV:                                                                                      \
    hipLaunchKernelGGL((decode_kernel<GLU, TGV>), grid, dim3(256), 0, st, x, ldx, perm, offsets, \
                       kept_offsets, kslots, W1, W2, wrows, K, act, bg, bu, out, ldo);           \
    break;
  switch (tg) {
    MOE_DECODE_CASE(1)
    MOE_DECODE_CASE(2)
    MOE_DECODE_CASE(3)
    default:
    MOE_DECODE_CASE(4)
  }
#undef MOE_DECODE_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gu(const uint16_t *x, int64_t T, int w, const int32_t *perm,
                            const int32_t *offsets, const int32_t *kept_offsets, int kslots,
                            const uint16_t *Wg, const uint16_t *Wu, int h, int N, int act,
                            float bg, float bu, uint16_t *hid, hipStream_t st) {
  const int64_t maxrows = T < kDecodeMaxRows ? T : kDecodeMaxRows;
  const int tg = (int)((maxrows + 15) / 16);
  return launch_decode<true>(tg, dim3(h / RB, N), st, x, w, perm, offsets, kept_offsets, kslots,
                             Wg, Wu, h, w, act, bg, bu, hid, h);
}

hipError_t launch_decode_down(const uint16_t *hid, int64_t T, const int32_t *kept_offsets,
                              const uint16_t *Wd, int h, int w, int N, float *y_perm,
                              hipStream_t st) {
  const int64_t maxrows = T < kDecodeMaxRows ? T : kDecodeMaxRows;
  const int tg = (int)((maxrows + 15) / 16);
  return launch_decode<false>(tg, dim3(w / RB, N), st, hid, h, nullptr, nullptr,
                              kept_offsets, 1, Wd, nullptr, w, h, 0, 1.f, 1.f, y_perm, w);
}

}  // namespace moe
