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
// FP8 weights (E4M3 codes, one fp32 scale per weight row) use 256-byte row
// windows, 256 k; the operands are widened to bf16 exactly after the LDS
// read, and the row scales multiply the fp32 sums after the split-K
// reduction.  MXFP4 weights (E2M1 codes two a byte, one E8M0 scale per 32 k)
// use 128-byte windows of 256 k for the gate/up and, for the down, 256-byte
// windows of 512 k with one token group a workgroup (128-byte ones with
// two); each k-step's operand is 4 bytes, widened with its block scale
// folded in (v_cvt_scalef32_pk_bf16_fp4, exact).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int NRB = 2;          // 16-row weight blocks per wave (token fragments reused NRB x)
constexpr int RB = 16 * NRB;    // weight rows per workgroup
constexpr int kWaves = 4;       // split-K ways
// Weight formats.
constexpr int WF_BF16 = WFMT_BF16;   // bf16
constexpr int WF_FP8 = WFMT_FP8;     // E4M3, fp32 scale per weight row
constexpr int WF_MX4 = WFMT_MXFP4;   // MXFP4: E2M1 pairs, E8M0 scale per 32 k
// Bytes of one weight row per 32-k step.
template <int WF>
constexpr int kstep_bytes() { return WF == WF_BF16 ? 64 : (WF == WF_FP8 ? 32 : 16); }
// k-steps of 32 per iteration.  bf16: 16 KiB of weights per wave per
// iteration (GLU: 2 matrices x 32 rows x 256 B, U = 4; down: 32 rows x
// 512 B, U = 8).  fp8: 256-byte row windows (U = 8): GLU streams 16 KiB,
// down 8 KiB (a 512-byte fp8 window's operand registers push it past 256
// VGPRs; measured 0.13 vs 0.10 ms at the Mixtral decode shape).  MXFP4
// gate/up: 128-byte row windows (U = 8), an 8 KiB window a wave (Mixtral
// T=32 gate/up 0.117 -> 0.110 ms against 256-byte ones).  The MXFP4 down
// takes 256-byte windows (U = 16) with one token group a workgroup (the
// window's 16 token fragments beside it) and 128-byte ones with two.
template <bool GLU, int WF, int TG>
constexpr int unroll_of() {
  return WF == WF_BF16 ? (GLU ? 4 : 8) : (WF == WF_MX4 && !GLU && TG == 1 ? 16 : 8);
}

// S1, S2: fp32 row scales [N][wrows] (WF_FP8) or E8M0 block scales
// [N][wrows][K/32] (WF_MX4).
template <bool GLU, int TG, int WF>
__global__ __launch_bounds__(256) void decode_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ kept_offsets, int kslots,
    const void *__restrict__ W1, const void *__restrict__ W2, const void *__restrict__ S1,
    const void *__restrict__ S2, int64_t wrows, int K, int act, float bg, float bu,
    void *__restrict__ out, int64_t ldo) {
  constexpr bool FP8 = WF == WF_FP8;
  constexpr bool MX4 = WF == WF_MX4;
  constexpr int NM = GLU ? 2 : 1;
  constexpr int KSB = kstep_bytes<WF>();  // bytes per row per 32-k step
  constexpr int U = unroll_of<GLU, WF, TG>();
  constexpr int kPitch = U * KSB;         // bytes of one row's window in a slice
  constexpr int kLoads = kPitch / 32;     // 1 KiB load instructions per matrix
  constexpr int kSlice = NM * RB * kPitch;  // per-wave LDS slice: one iteration's weights
  static_assert(kPitch >= 128, "the chunk swizzle needs 8 chunks a row");
  // After the loop the same LDS holds the partial sums of waves 1 .. 3.
  constexpr int kRedBytes = NM * NRB * TG * 64 * 16;
  // MXFP4: each wave's window scales, [NM][RB rows][U bytes], after the slices.
  constexpr int kScale = MX4 ? NM * RB * U : 0;
  constexpr int kMain = kWaves * (kSlice + kScale);
  constexpr int kLds = kMain > (kWaves - 1) * kRedBytes ? kMain : (kWaves - 1) * kRedBytes;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  const int e = blockIdx.y;
  const int M = kept_offsets[e + 1] - kept_offsets[e];
  // Token groups of 16: this workgroup takes groups g0 .. g0 + TG - 1 of the
  // expert's (the grid's z splits an expert's groups between workgroups when
  // a single one would need more token registers than two waves per SIMD
  // allow; a workgroup with no group of its own exits at once).
  const int g0 = blockIdx.z * TG;
  if (M <= g0 * 16) return;
  const int row0 = blockIdx.x * RB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;           // weight row within block / token within group
  const int kq = (lane >> 4) * 8;     // k offset of this lane's 8 values
  const int Kw = K / kWaves;
  const int kb = wave * Kw;
  // Row r's 16-byte chunk c sits at chunk c ^ swz(r) of its slice row: the
  // low 4 row bits with 16 or more chunks a row, row bits 1-3 with 8 (two
  // 128-byte rows share the 256 bytes of banks).
  auto swz = [](int r) { return kPitch >= 256 ? (r & 15) : ((r >> 1) & 7); };

  // Byte offset of element k of a weight row (k a multiple of 8).
  auto kbytes = [](int64_t k) -> int64_t { return k * KSB / 32; };
  const int64_t rowK = kbytes(K);  // bytes of one weight row
  const char *w1 = static_cast<const char *>(W1) + ((int64_t)e * wrows + row0 + li) * rowK +
                   kbytes(kb + kq);
  const char *w2 = GLU ? static_cast<const char *>(W2) + ((int64_t)e * wrows + row0 + li) * rowK +
                             kbytes(kb + kq)
                       : nullptr;
  // MXFP4 block scales of this lane's row (row0 + li; + 16 for block 1).
  const int KB = K / 32;
  const uint8_t *sb1 = MX4 ? static_cast<const uint8_t *>(S1) +
                                 ((int64_t)e * wrows + row0 + li) * KB + kb / 32
                           : nullptr;
  const uint8_t *sb2 = (MX4 && GLU) ? static_cast<const uint8_t *>(S2) +
                                          ((int64_t)e * wrows + row0 + li) * KB + kb / 32
                                    : nullptr;
  const int64_t rbs = 16 * rowK;  // next 16-row block
  // Whole-line loads: instruction i takes rows 8*(i%4) + lane/8 and the
  // 128-byte piece i/4 of the iteration's window; lane%8 picks 16 bytes.
  const int lr = lane >> 3, lc = lane & 7;
  // The window loads go through buffer resources over the workgroup's 32
  // weight rows: one lane offset per matrix, the rest uniform.
  const uint32_t blk_bytes = (uint32_t)(RB * rowK);
  const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(
      static_cast<const char *>(W1) + ((int64_t)e * wrows + row0) * rowK, blk_bytes);
  const __amdgpu_buffer_rsrc_t rw2 =
      GLU ? make_rsrc(static_cast<const char *>(W2) + ((int64_t)e * wrows + row0) * rowK,
                      blk_bytes)
          : rw1;
  const uint32_t wlo = (uint32_t)(lr * rowK + kbytes(kb) + 16 * lc);
  char *slice = smem + wave * kSlice;
  char *sslot = smem + kWaves * kSlice + wave * kScale;  // MXFP4 window scales
  const uint16_t *xr[TG];
  bool xv[TG];
  // Token fragments of the windows are read through a buffer resource over
  // x: a lane with no token (past the expert's rows, or a group the expert
  // does not have) reads past the resource's end and gets zeros, so every
  // window issues the same loads with no branch around them, and the
  // compiler's waits for a window's weights count exactly the token loads
  // issued after them (with a branch per load it waited for those too, so
  // the next window's weights were requested only once the current window's
  // tokens had arrived).
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, kDecodeXBytes);
  uint32_t xo[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int j = (g0 + tg) * 16 + li;
    xv[tg] = j < M;
    int64_t row;
    if (GLU) row = xv[tg] ? perm[offsets[e] + j] / kslots : 0;
    else row = kept_offsets[e] + (xv[tg] ? j : 0);
    xr[tg] = x + row * ldx + kb + kq;
    xo[tg] = xv[tg] ? (uint32_t)((row * ldx + kb + kq) * 2) : kDecodeXBytes;
  }
  const int ngroups = (M + 15) / 16 - g0;  // this workgroup's groups (may exceed TG)

  f32x4 acc[NM][NRB][TG];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) acc[m][r][tg] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  // One MFMA operand (8 weights of row r, k-step u, this lane's k quarter)
  // from the slice: 16 bytes of bf16, 8 bytes of fp8 or 4 bytes of MXFP4
  // (with its block scale sc) widened to bf16.
  auto slice_frag = [&](int m, int r, int u, float sc) -> bf16x8 {
    const char *row = slice + m * RB * kPitch + r * kPitch;
    if constexpr (MX4) {
      const uint32_t raw =
          *reinterpret_cast<const uint32_t *>(row + ((u ^ swz(r)) << 4) + 4 * (lane >> 4));
      return e2m1x8_to_bf16x8(raw, sc);
    } else if constexpr (FP8) {
      const int q = lane >> 4;
      const int c = 2 * u + (q >> 1);
      const uint2 raw = *reinterpret_cast<const uint2 *>(row + ((c ^ swz(r)) << 4) + 8 * (q & 1));
      return e4m3x8_to_bf16x8(raw.x, raw.y);
    } else {
      const int c = 4 * u + (lane >> 4);
      return *reinterpret_cast<const bf16x8 *>(row + ((c ^ swz(r)) << 4));
    }
  };
  auto global_frag = [&](const char *w, int64_t byte_off, float sc) -> bf16x8 {
    if constexpr (MX4) {
      return e2m1x8_to_bf16x8(*reinterpret_cast<const uint32_t *>(w + byte_off), sc);
    } else if constexpr (FP8) {
      const uint2 raw = *reinterpret_cast<const uint2 *>(w + byte_off);
      return e4m3x8_to_bf16x8(raw.x, raw.y);
    } else {
      return *reinterpret_cast<const bf16x8 *>(w + byte_off);
    }
  };
  // The windows are software-pipelined.  An iteration requests its
  // window's token fragments (L2 hits), parks the window's weights (requested
  // one iteration earlier) in the slice, requests the next window's weights
  // and only then waits for its tokens, so a window of weights is in flight
  // while this one is multiplied and the token latency overlaps that request
  // instead of delaying it.  Every load of an iteration is unconditional, so
  // the waits count them exactly.
  // MXFP4 windows load their scales as dwords, which needs every wave's K
  // start 4-byte aligned in the scale rows (K / 128 a multiple of 4): K a
  // multiple of 512; other widths take the per-k-step loop below for the
  // whole K.
  const int nwin = (MX4 && K % 512 != 0) ? 0 : Kw / (32 * U);
  const int kfull = nwin * 32 * U;
  constexpr int kTokLoads = TG * U;  // token loads issued after a window's weights
  u32x4 v[NM][kLoads];
  // MXFP4: the window's U scale bytes of each of the 32 rows go straight to
  // the wave's scale slot (U = 8: one dword load per matrix, lane l: row
  // l / 2, dword l % 2; U = 16: two, lane l: row 16 q + l / 4, dword l % 4),
  // issued ahead of the window's own loads so that waiting for those covers
  // them.
  typedef __attribute__((address_space(3))) void *lds_ptr_t;
  __amdgpu_buffer_rsrc_t rs[NM];
  if constexpr (MX4) {
    const uint32_t sbytes = (uint32_t)(wrows * KB);
    rs[0] = make_rsrc(static_cast<const uint8_t *>(S1) + (int64_t)e * wrows * KB, sbytes);
    if constexpr (GLU)
      rs[NM - 1] = make_rsrc(static_cast<const uint8_t *>(S2) + (int64_t)e * wrows * KB, sbytes);
  }
  auto load_window = [&](int kw) {
    if constexpr (MX4) {
      static_assert(U == 8 || U == 16, "scale slot layouts for 8 or 16 bytes a row");
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if constexpr (U == 8) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs[m], (lds_ptr_t)(sslot + m * RB * U), 4,
              (uint32_t)((row0 + (lane >> 1)) * KB + (kb + kw) / 32 + 4 * (lane & 1)), 0, 0, 0);
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs[m], (lds_ptr_t)(sslot + m * RB * U + q * 256), 4,
                (uint32_t)((row0 + 16 * q + (lane >> 2)) * KB + (kb + kw) / 32 + 4 * (lane & 3)),
                0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const uint32_t so = (uint32_t)(8 * (i % 4) * rowK + kbytes(kw));
      v[0][i] = buf_load16(rw1, wlo + 128 * (i / 4), so);
      if (GLU) v[NM - 1][i] = buf_load16(rw2, wlo + 128 * (i / 4), so);
    }
  };
  // One window; LAST (the final window, peeled off the loop) requests no
  // next one, so every path through the loop body issues the same loads and
  // the compiler's waits for the token fragments stop short of the next
  // window's requests.
  auto window_step = [&](const int k, auto last_c) {
    constexpr bool LAST = decltype(last_c)::value;
    // The window's token fragments (zeros for lanes with no token).
    bf16x8 b[TG][U];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[tg][u] = __builtin_bit_cast(bf16x8, buf_load16(rx, xo[tg] + 2 * (k + 32 * u), 0));
    // (the scheduler would otherwise sink some token loads below the next
    // window's requests, and waiting for them would wait for that window)
    __builtin_amdgcn_sched_barrier(0);
    // Into the wave's own slice, swizzled.
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int r = 8 * (i % 4) + lr;
        const int c = 8 * (i / 4) + lc;
        *reinterpret_cast<u32x4 *>(slice + m * RB * kPitch + r * kPitch + ((c ^ swz(r)) << 4)) =
            v[m][i];
      }
    // MXFP4: the window's U block scales of each of the lane's rows, from
    // the scale slot (its loads were issued before this window's token
    // loads, so they are complete once at most those remain), read before
    // the next window's loads may overwrite the slot.
    uint32_t sw[NM][NRB][U / 4];
    if constexpr (MX4) {
      wait_vmcnt<kTokLoads>();
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const char *src = sslot + m * RB * U + (16 * rb + li) * U;
          if constexpr (U == 8) {
            const uint2 q2 = *reinterpret_cast<const uint2 *>(src);
            sw[m][rb][0] = q2.x;
            sw[m][rb][1] = q2.y;
          } else {
            const u32x4 q4 = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
            for (int j = 0; j < U / 4; ++j) sw[m][rb][j] = q4[j];
          }
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // The next window's weights; the MFMAs below then wait for this
    // window's tokens only.
    if constexpr (!LAST) load_window(k + 32 * U);
    __builtin_amdgcn_sched_barrier(0);
    // MFMA operands: lane l takes row 16 rb + l%16, k values 32u + 8(l/16) .. +7.
    // A group the expert does not have multiplies its zero token fragments:
    // a branch around it would let the compiler sink that group's token
    // loads into the branch, below the next window's requests.
    if constexpr (MX4) {
      // Widened operands of one k-step at a time, each with its block scale.
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bf16x8 a[NM][NRB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            a[m][rb] = slice_frag(m, 16 * rb + li, u,
                                  e8m0_to_f32((sw[m][rb][u >> 2] >> (8 * (u & 3))) & 0xFF));
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < NRB; ++r)
              acc[m][r][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][r], b[tg][u],
                                                                     acc[m][r][tg], 0, 0, 0);
      }
    } else if constexpr (FP8) {
      // Widened operands of one k-step at a time (all U would not fit
      // beside the loads in flight).
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bf16x8 a[NM][NRB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) a[m][rb] = slice_frag(m, 16 * rb + li, u, 1.f);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < NRB; ++r)
              acc[m][r][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][r], b[tg][u],
                                                                     acc[m][r][tg], 0, 0, 0);
      }
    } else {
      bf16x8 a[NM][NRB][U];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int u = 0; u < U; ++u) a[m][rb][u] = slice_frag(m, 16 * rb + li, u, 1.f);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < NRB; ++r)
              acc[m][r][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][r][u], b[tg][u],
                                                                     acc[m][r][tg], 0, 0, 0);
    }
  };
  if (nwin > 0) {
    load_window(0);
    for (int wi = 0; wi + 1 < nwin; ++wi) window_step(wi * 32 * U, std::false_type{});
    window_step((nwin - 1) * 32 * U, std::true_type{});
  }
  int k = kfull;
  for (; k < Kw; k += 32) {
    bf16x8 a[NM][NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      float s1 = 1.f, s2 = 1.f;
      if constexpr (MX4) {
        s1 = e8m0_to_f32(sb1[(int64_t)r * 16 * KB + k / 32]);
        if (GLU) s2 = e8m0_to_f32(sb2[(int64_t)r * 16 * KB + k / 32]);
      }
      a[0][r] = global_frag(w1, r * rbs + kbytes(k), s1);
      if (GLU) a[NM - 1][r] = global_frag(w2, r * rbs + kbytes(k), s2);
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
  // FP8: those rows' scales multiply the sums (fp32) before the epilogue.
  f32x4 sc[NM][NRB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      if constexpr (FP8) {
        const float *S = static_cast<const float *>((m == 0) ? S1 : S2);
        sc[m][r] = *reinterpret_cast<const f32x4 *>(S + (int64_t)e * wrows + row0 + 16 * r +
                                                    4 * (lane >> 4));
      } else {
        sc[m][r] = f32x4{1.f, 1.f, 1.f, 1.f};
      }
    }
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int j = (g0 + tg) * 16 + li;
    if (tg >= ngroups || j >= M) continue;
    const int64_t orow = kept_offsets[e] + j;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int col = row0 + 16 * r + 4 * (lane >> 4);
      if constexpr (GLU) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = FP8 ? acc[0][r][tg][q] * sc[0][r][q] : acc[0][r][tg][q];
          const float u = FP8 ? acc[1][r][tg][q] * sc[1][r][q] : acc[1][r][tg][q];
          v[q] = glu_act_fast(g, u, act, bg, bu);
        }
        uint2 pk;
        pk.x = pack_bf16x2_hw(v[0], v[1]);
        pk.y = pack_bf16x2_hw(v[2], v[3]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + orow * ldo + col) = pk;
      } else {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + orow * ldo + col) =
            FP8 ? acc[0][r][tg] * sc[0][r] : acc[0][r][tg];
      }
    }
  }
}

template <bool GLU, int WF>
hipError_t launch_decode(int tg, int64_t wrows, int N, hipStream_t st, const uint16_t *x,
                         int64_t ldx, const int32_t *perm, const int32_t *offsets,
                         const int32_t *kept_offsets, int kslots, const void *W1, const void *W2,
                         const void *S1, const void *S2, int K, int act, float bg, float bu,
                         void *out, int64_t ldo) {
  // tg token groups of 16 may be needed per expert (T up to 16 tg).  A
  // workgroup holds one of them up to T = 32 and two beyond (three or four
  // cost a wave per SIMD: Mixtral T=64 gate/up 0.324 -> 0.312 ms bf16,
  // 0.215 -> 0.140 ms MXFP4), and the grid's z covers the rest: with k of N
  // experts chosen per token an expert rarely gets more than half the
  // tokens, so the extra z workgroups exit at once, and an expert that does
  // use them reads its weights once per z.  One group a workgroup frees the
  // second group's token registers (Mixtral T=32, against two: MXFP4
  // forward 0.201 -> 0.190 ms, FP8 0.268 -> 0.265 ms, bf16 unchanged).
  const int cap = tg <= 2 ? 1 : 2;
  const int tgw = tg < cap ? tg : cap;
  const dim3 grid((unsigned)(wrows / RB), N, (unsigned)((tg + tgw - 1) / tgw));
#define MOE_DECODE_CASE(TGV)                                                                  \
  case TGV:                                                                                   \
    hipLaunchKernelGGL((decode_kernel<GLU, TGV, WF>), grid, dim3(256), 0, st, x, ldx, perm,   \
                       offsets, kept_offsets, kslots, W1, W2, S1, S2, wrows, K, act, bg, bu,  \
                       out, ldo);                                                             \
    break;
  switch (tgw) {
    MOE_DECODE_CASE(1)
    default:
    MOE_DECODE_CASE(2)
  }
#undef MOE_DECODE_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gu(const uint16_t *x, int64_t T, int w, const int32_t *perm,
                            const int32_t *offsets, const int32_t *kept_offsets, int kslots,
                            const void *Wg, const void *Wu, const void *sg, const void *su,
                            int wfmt, int h, int N, int act, float bg, float bu, uint16_t *hid,
                            hipStream_t st) {
  const int64_t maxrows = T < kDecodeMaxRows ? T : kDecodeMaxRows;
  const int tg = (int)((maxrows + 15) / 16);
  if (wfmt == WF_FP8)
    return launch_decode<true, WF_FP8>(tg, h, N, st, x, w, perm, offsets, kept_offsets, kslots,
                                       Wg, Wu, sg, su, w, act, bg, bu, hid, h);
  if (wfmt == WF_MX4)
    return launch_decode<true, WF_MX4>(tg, h, N, st, x, w, perm, offsets, kept_offsets, kslots,
                                       Wg, Wu, sg, su, w, act, bg, bu, hid, h);
  return launch_decode<true, WF_BF16>(tg, h, N, st, x, w, perm, offsets, kept_offsets, kslots,
                                      Wg, Wu, nullptr, nullptr, w, act, bg, bu, hid, h);
}

hipError_t launch_decode_down(const uint16_t *hid, int64_t T, const int32_t *kept_offsets,
                              const void *Wd, const void *sd, int wfmt, int h, int w, int N,
                              float *y_perm, hipStream_t st) {
  const int64_t maxrows = T < kDecodeMaxRows ? T : kDecodeMaxRows;
  const int tg = (int)((maxrows + 15) / 16);
  if (wfmt == WF_FP8)
    return launch_decode<false, WF_FP8>(tg, w, N, st, hid, h, nullptr, nullptr, kept_offsets, 1,
                                        Wd, nullptr, sd, nullptr, h, 0, 1.f, 1.f, y_perm, w);
  if (wfmt == WF_MX4)
    return launch_decode<false, WF_MX4>(tg, w, N, st, hid, h, nullptr, nullptr, kept_offsets, 1,
                                        Wd, nullptr, sd, nullptr, h, 0, 1.f, 1.f, y_perm, w);
  return launch_decode<false, WF_BF16>(tg, w, N, st, hid, h, nullptr, nullptr, kept_offsets, 1,
                                       Wd, nullptr, nullptr, nullptr, h, 0, 1.f, 1.f, y_perm, w);
}

}  // namespace moe
