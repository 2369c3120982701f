// Decode-sized experts: few tokens per expert, so the projections are bound
// by reading the selected experts' weights once (page "Kestrel-MCU notes #13:
// the MoE deployment gap", section 二: experts are stored grouped and looked
// up by index, and only the selected experts' weights are read).
//
// Each workgroup owns 32 weight rows of one expert and all K; its 4 waves
// split K and reduce their partial sums through LDS in a fixed order.  A wave
// reads its weights in windows of 16 KiB with whole-line loads (8 lanes x 16
// bytes per row, 8 rows per instruction), parks each window in its own LDS
// slice (16-byte chunks XOR-swizzled by row) and reads the
// v_mfma_f32_16x16x32_bf16 operands back from there (16 weight rows x up to
// 16 tokens per group; each token fragment feeds both 16-row blocks).  Loading
// the operand layout directly would touch each 128-byte line in two 64-byte
// halves from two instructions, which streams HBM at roughly two thirds of
// the whole-line rate.  Experts with no kept token exit before touching their
// weights.
//   GLU = true : hid[row] = act(W_gate x, W_up x), x rows gathered via perm
//   GLU = false: y_perm[row] = W_down hid[row], fp32
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int NRB = 2;          // 16-row weight blocks per wave (token fragments reused NRB x)
constexpr int RB = 16 * NRB;    // weight rows per workgroup
constexpr int kWaves = 4;       // split-K ways
// k-steps of 32 per iteration: 16 KiB of weights per wave per iteration
// (GLU: 2 matrices x 32 rows x 256 B; down: 32 rows x 512 B).
template <bool GLU>
constexpr int unroll_of() { return GLU ? 4 : 8; }
// Per-wave LDS slice: one iteration's weights, row pitch U * 64 bytes.
constexpr int kSlice = 16384;

template <bool GLU, int TG>
__global__ __launch_bounds__(256) void decode_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ kept_offsets, int kslots,
    const uint16_t *__restrict__ W1, const uint16_t *__restrict__ W2, int64_t wrows, int K,
    int act, float bg, float bu, void *__restrict__ out, int64_t ldo) {
  constexpr int NM = GLU ? 2 : 1;
  constexpr int U = unroll_of<GLU>();
  constexpr int kPitch = U * 64;          // bytes of one row's window in a slice
  constexpr int kLoads = 2 * U;           // 1 KiB load instructions per matrix
  static_assert(NM * RB * kPitch == kSlice, "slice holds one iteration");
  // After the loop the same LDS holds the partial sums of waves 1 .. 3.
  constexpr int kRedBytes = NM * NRB * TG * 64 * 16;
  constexpr int kLds = kWaves * kSlice > (kWaves - 1) * kRedBytes ? kWaves * kSlice
                                                                  : (kWaves - 1) * kRedBytes;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
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
  // Whole-line loads: instruction i takes rows 8*(i%4) + lane/8 and the
  // 128-byte piece i/4 of the iteration's window; lane%8 picks 16 bytes.
  const int lr = lane >> 3, lc = lane & 7;
  const uint16_t *g1 = W1 + ((int64_t)e * wrows + row0 + lr) * K + kb + 8 * lc;
  const uint16_t *g2 = GLU ? W2 + ((int64_t)e * wrows + row0 + lr) * K + kb + 8 * lc : nullptr;
  char *slice = smem + wave * kSlice;
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
  int k = 0;
  for (; k + 32 * U <= Kw; k += 32 * U) {
    bf16x8 v[NM][kLoads], b[TG][U];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int64_t off = (int64_t)(8 * (i % 4)) * K + 64 * (i / 4) + k;
      v[0][i] = *reinterpret_cast<const bf16x8 *>(g1 + off);
      if (GLU) v[NM - 1][i] = *reinterpret_cast<const bf16x8 *>(g2 + off);
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[tg][u] = (tg < ngroups && xv[tg]) ? *reinterpret_cast<const bf16x8 *>(xr[tg] + k + 32 * u)
                                           : zero;
    // Into the wave's own slice: row r's 16-byte chunk c sits at chunk c ^ (r & 15).
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int r = 8 * (i % 4) + lr;
        const int c = 8 * (i / 4) + lc;
        *reinterpret_cast<bf16x8 *>(slice + m * RB * kPitch + r * kPitch + ((c ^ (r & 15)) << 4)) =
            v[m][i];
      }
    // MFMA operands: lane l takes row 16 rb + l%16, chunk 4u + l/16.
    bf16x8 a[NM][NRB][U];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = 16 * rb + li;
          const int c = 4 * u + (lane >> 4);
          a[m][rb][u] = *reinterpret_cast<const bf16x8 *>(slice + m * RB * kPitch + r * kPitch +
                                                          ((c ^ li) << 4));
        }
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

  // Fixed-order split-K reduction: once every wave is done with its slice,
  // waves 1..3 park their partial sums in LDS and wave 0 adds waves 1, 2, 3
  // in turn.
  typedef f32x4 RedT[NM][NRB][TG][64];
  __syncthreads();
  if (wave > 0) {
    RedT &mine = *reinterpret_cast<RedT *>(smem + (wave - 1) * kRedBytes);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) mine[m][r][tg][lane] = acc[m][r][tg];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    const RedT &theirs = *reinterpret_cast<const RedT *>(smem + (w - 1) * kRedBytes);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[m][r][tg] += theirs[m][r][tg][lane];
  }
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
