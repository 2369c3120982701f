// Shared device helpers for the gfx950 MoE kernels: bf16 <-> fp32, MFMA
// vector types, buffer resources, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Raw buffer resource over [base, base + bytes); a read whose lane offset
// (plus the immediate) reaches past the end returns 0 (offsets that must be
// range-checked go in the lane offset, not the scalar one).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt field layout: vmcnt bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima, i.e. not waited for).  Issued as the
// builtin, the compiler's own wait insertion sees it and adds no stricter
// wait for the loads it covers; the empty asm keeps memory accesses from
// being moved across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier that leaves vector-memory loads in flight: LDS traffic
// is drained (lgkmcnt 0) but, unlike __syncthreads(), no vmcnt(0) is forced,
// so callers wait for exactly the loads they need with s_waitcnt vmcnt(N).
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---- lane exchanges without the LDS round trip of a shuffle ----------------
// Value of lane (lane ^ 1) / (lane ^ 2): DPP quad permutations, no LDS.
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ int lane_xor1(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ int lane_xor2(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
}
// Value of lane (lane ^ M) for M < 32 (ds_swizzle bit mode within each half
// of the wave: no LDS memory access).
template <int M>
__device__ __forceinline__ float lane_xor_swz(float v) {
  static_assert(M > 0 && M < 32, "within a 32-lane half");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}
template <int M>
__device__ __forceinline__ int lane_xor_swz(int v) {
  static_assert(M > 0 && M < 32, "within a 32-lane half");
  return __builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10));
}
// Mirror exchanges inside a row of 16 lanes (lane 7-i of each 8, 15-i of
// each 16): for reductions whose operation is commutative and associative.
__device__ __forceinline__ float lane_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}
__device__ __forceinline__ int lane_half_mirror(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
}
__device__ __forceinline__ int lane_mirror(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
}

// Arg-max over the wave of (v, i): the largest v, ties to the smaller i.
// Every lane returns the same pair.  Rows of 16 lanes reduce through DPP
// exchanges, then row_bcast:15 and row_bcast:31 fold rows 0-1 into row 1
// and rows 0-3 into row 3, and lane 63 holds the result.
__device__ __forceinline__ void argmax_step(float &v, int &i, float ov, int oi) {
  const bool t = (ov > v) | ((ov == v) & (oi < i));
  v = t ? ov : v;
  i = t ? oi : i;
}
__device__ __forceinline__ int dpp_bcast15(int v) {
  return __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false);
}
__device__ __forceinline__ int dpp_bcast31(int v) {
  return __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false);
}
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
  argmax_step(v, i, lane_xor1(v), lane_xor1(i));
  argmax_step(v, i, lane_xor2(v), lane_xor2(i));
  argmax_step(v, i, lane_half_mirror(v), lane_half_mirror(i));
  argmax_step(v, i, lane_mirror(v), lane_mirror(i));
  argmax_step(v, i, __int_as_float(dpp_bcast15(__float_as_int(v))), dpp_bcast15(i));
  argmax_step(v, i, __int_as_float(dpp_bcast31(__float_as_int(v))), dpp_bcast31(i));
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// Two fp32 values -> packed bf16 pair (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Eight OCP FP8 E4M3 codes (byte j = element j) -> the bf16x8 MFMA operand.
// Every E4M3 value is exact in bf16 (3 mantissa bits, exponents -9..8), and
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// OCP E8M0 scale byte -> its fp32 value 2^(s - 127) (0xFF: NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s == 0 ? 0x00400000u : (s == 0xFF ? 0x7FC00000u : s << 23));
}

// Eight E2M1 codes (4 bytes, element 2i in the low nibble of byte i) times
// 2^(s - 127) -> the bf16x8 MFMA operand (exact while in the bf16 range).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16x8(uint32_t raw, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ---- precise activations (fp32 path) -------------------------------------
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// act(g, v): SwiGLU (situ == 0) or SiTU-GLU with caps beta_g, beta_u.
__device__ __forceinline__ float glu_act(float g, float v, int situ, float bg, float bu) {
  if (situ) {
    g = bg * tanhf(g / bg);
    v = bu * tanhf(v / bu);
  }
  return silu(g) * v;
}

// ---- fast activations (bf16 epilogues) ------------------------------------
// exp(x) = 2^(x log2 e) on the hardware exp2 (about 1 ulp); SiLU(x) =
// x / (1 + e^-x) with the hardware reciprocal.  tanh(y) for |y| >= 1/16 is
// (1 - t) / (1 + t), t = e^(-2|y|) <= 0.89, so the subtraction amplifies the
// error of t by at most 8x (a few 1e-7 relative); below 1/16 the odd Taylor
// series y - y^3/3 + 2y^5/15 (truncation < 2e-10 relative).  The bf16
// outputs these feed are rounded to 2^-9 relative, far above these errors.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float fast_silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + fast_exp(-x));
}

__device__ __forceinline__ float fast_tanh(float y) {
  const float ay = fabsf(y);
  float r;
  if (ay < 0.0625f) {
    const float y2 = y * y;
    r = ay * (1.0f + y2 * (-0.3333333333f + y2 * 0.1333333333f));
  } else {
    const float t = fast_exp(-2.0f * ay);
    r = (1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t);
  }
  return copysignf(r, y);
}

__device__ __forceinline__ float glu_act_fast(float g, float v, int situ, float bg, float bu) {
  if (situ) {
    g = bg * fast_tanh(g * __builtin_amdgcn_rcpf(bg));
    v = bu * fast_tanh(v * __builtin_amdgcn_rcpf(bu));
  }
  return fast_silu(g) * v;
}

// Backward of h = act(g, v): (dg, dv) from dh, on the fast activations above
// (the GEMM epilogue that feeds bf16 dG and dU).  SwiGLU: silu'(g) =
// s(g) (1 + g (1 - s(g))); SiTU-GLU caps both factors with beta tanh(x / beta)
// first, which multiplies by 1 - tanh^2.
__device__ __forceinline__ void glu_act_backward_fast(float g, float v, float dh, int situ,
                                                      float bg, float bu, float &dg, float &dv) {
  float tg = 0.f, tv = 0.f;
  if (situ) {
    tg = fast_tanh(g * __builtin_amdgcn_rcpf(bg));
    tv = fast_tanh(v * __builtin_amdgcn_rcpf(bu));
    g = bg * tg;
    v = bu * tv;
  }
  const float s = __builtin_amdgcn_rcpf(1.0f + fast_exp(-g));
  dg = dh * v * s * (1.0f + g * (1.0f - s));
  dv = dh * g * s;
  if (situ) {
    dg *= 1.0f - tg * tg;
    dv *= 1.0f - tv * tv;
  }
}

}  // namespace moe
