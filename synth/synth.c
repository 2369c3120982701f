/*
 * Seeded, counter-based synthetic tensor generator.
 *
 * This file produces the random input values that both the fp64 oracle and the
 * GPU library consume. It holds none of the MoE layer's arithmetic: it only
 * draws numbers and rounds them to a storage format.
 *
 * Generator:
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): the n-th output for state K is
 *     mix(K + (n+1)*gamma), gamma = 0x9E3779B97F4A7C15, where mix is the
 *     two xorshift-multiply rounds of that paper's finaliser.
 *   - The stream key of a tensor is K = mix(mix(seed + gamma) ^ tensor_id + gamma),
 *     i.e. one SplitMix64 step from the seed, xored with the tensor id, and
 *     one step again.  Element e of that tensor belongs to Box-Muller pair
 *     j = e/2 and uses outputs n = 2j (u1) and n = 2j+1 (u2) of stream K.
 *   - Box-Muller (Box and Muller, 1958): u1 in (0,1], u2 in [0,1),
 *     r = sqrt(-2 ln u1), theta = 2 pi u2; element 2j = r cos theta,
 *     element 2j+1 = r sin theta.  Values are produced in fp64.
 *   Because every element is a pure function of (seed, tensor_id, index),
 *   any slice can be regenerated on its own, in any order, on any number of
 *   threads, with identical results.
 *
 * Storage rounding:
 *   - fp32: the C conversion double -> float (round to nearest, ties to even).
 *   - bf16: direct round-to-nearest-even from fp64 to the bf16 grid (1 sign,
 *     8 exponent, 7 mantissa bits), including subnormals, overflow to Inf and
 *     NaN propagation.  No intermediate fp32 rounding (no double rounding).
 *   - fp8 E4M3 rows: per-row fp32 scale max|row| / 448, codes rounded
 *     nearest-even from fp64 (synth_normal_e4m3_rows).
 *   - MXFP4 rows: E8M0 scale per 32 values, E2M1 elements rounded
 *     nearest-even (synth_normal_mxfp4_rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* n-th SplitMix64 output of a generator whose state starts at K. */
static inline uint64_t sm_output(uint64_t K, uint64_t n) {
  return sm_mix(K + (n + 1) * SM_GAMMA);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tensor_id) {
  return sm_output(sm_output(seed, 0) ^ tensor_id, 0);
}

uint64_t synth_splitmix64(uint64_t K, uint64_t n) { return sm_output(K, n); }

/* Both standard normal values of Box-Muller pair j of the stream keyed by K. */
static inline void normal_pair(uint64_t K, uint64_t j, double *c, double *s) {
  const uint64_t a = sm_output(K, 2 * j);
  const uint64_t b = sm_output(K, 2 * j + 1);
  const double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  *c = r * cos(th);
  *s = r * sin(th);
}

/* Calls EMIT(i, value) for every element start+i, i in [0, count), walking
   whole Box-Muller pairs so each pair is evaluated once. */
#define FOR_EACH_NORMAL(K, start, count, EMIT)                                 \
  do {                                                                         \
    const uint64_t s0_ = (start), n_ = (count), e1_ = s0_ + n_;                \
    if (n_ == 0) break;                                                        \
    const int64_t j0_ = (int64_t)(s0_ >> 1), j1_ = (int64_t)((e1_ + 1) >> 1);  \
    _Pragma("omp parallel for schedule(static)")                               \
    for (int64_t j_ = j0_; j_ < j1_; ++j_) {                                   \
      double c_, s_;                                                           \
      normal_pair((K), (uint64_t)j_, &c_, &s_);                                \
      const uint64_t e_ = 2 * (uint64_t)j_;                                    \
      if (e_ >= s0_ && e_ < e1_) { const uint64_t i = e_ - s0_; EMIT(i, c_); } \
      if (e_ + 1 >= s0_ && e_ + 1 < e1_) {                                     \
        const uint64_t i = e_ + 1 - s0_; EMIT(i, s_);                          \
      }                                                                        \
    }                                                                          \
  } while (0)

/* out[i] = mean + std * N(0,1)[start + i] in fp64. */
void synth_normal_f64(uint64_t seed, uint64_t tensor_id, uint64_t start,
                      uint64_t count, double mean, double std, double *out) {
  const uint64_t K = synth_stream_key(seed, tensor_id);
#define EMIT_F64(i, v) out[i] = mean + std * (v)
  FOR_EACH_NORMAL(K, start, count, EMIT_F64);
#undef EMIT_F64
}

/* Round one fp64 value to bf16 bits, nearest-even, directly. */
uint16_t synth_f64_to_bf16(double x) {
  uint64_t bits;
  memcpy(&bits, &x, 8);
  const uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  const int exp = (int)((bits >> 52) & 0x7FF);
  const uint64_t man = bits & 0xFFFFFFFFFFFFFULL;
  if (exp == 0x7FF) { /* Inf or NaN */
    if (man == 0) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | 0x7FC0u | (uint16_t)((man >> 45) & 0x3Fu));
  }
  const double ax = fabs(x);
  if (ax == 0.0) return sign;
  if (exp >= 1023 - 126 && exp < 1023 + 128) {
    /* Normal bf16 range: round the 52-bit mantissa to 7 bits (nearest, ties
       to even) on the integer pattern; a carry moves into the exponent. */
    const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFULL;
    const uint64_t r = (mag + 0xFFFFFFFFFFFULL + ((mag >> 45) & 1)) >> 45;
    const int rexp = (int)(r >> 7) - 1023 + 127;
    if (rexp >= 255) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)(rexp << 7) | (uint16_t)(r & 0x7F));
  }
  /* bf16 quantum: normal numbers with unbiased exponent E >= -126 have
     spacing 2^(E-7); below 2^-126 the spacing is fixed at 2^-133. */
  int E = exp - 1023;
  if (exp == 0) E = -1023; /* fp64 subnormal: far below the bf16 range */
  const int qexp = (E >= -126 ? E : -126) - 7;
  /* q = ax / 2^qexp is exact (power-of-two scaling within range). */
  const double q = ldexp(ax, -qexp);
  double n = floor(q);
  const double frac = q - n; /* exact */
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
  /* Rebuild the rounded magnitude and pack it. */
  const double r = ldexp(n, qexp);
  if (r >= 0x1.0p128) return (uint16_t)(sign | 0x7F80u); /* overflow */
  if (r < 0x1.0p-126) { /* bf16 subnormal (or rounded to zero) */
    return (uint16_t)(sign | (uint16_t)n);
  }
  int re;
  const double m = frexp(r, &re); /* r = m * 2^re, m in [0.5, 1) */
  const int bexp = re - 1 + 127;  /* biased bf16 exponent */
  const uint16_t bman = (uint16_t)((uint64_t)ldexp(m, 8) & 0x7Fu);
  return (uint16_t)(sign | (uint16_t)(bexp << 7) | bman);
}

void synth_round_bf16(const double *in, uint64_t count, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i) out[i] = synth_f64_to_bf16(in[i]);
}

void synth_round_f32(const double *in, uint64_t count, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i) out[i] = (float)in[i];
}

/* Fused draw + round, so large tensors never exist in fp64. */
void synth_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t start,
                       uint64_t count, double std, uint16_t *out) {
  const uint64_t K = synth_stream_key(seed, tensor_id);
#define EMIT_BF16(i, v) out[i] = synth_f64_to_bf16(std * (v))
  FOR_EACH_NORMAL(K, start, count, EMIT_BF16);
#undef EMIT_BF16
}

void synth_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t start,
                      uint64_t count, double std, float *out) {
  const uint64_t K = synth_stream_key(seed, tensor_id);
#define EMIT_F32(i, v) out[i] = (float)(std * (v))
  FOR_EACH_NORMAL(K, start, count, EMIT_F32);
#undef EMIT_F32
}

/* Round one fp64 value to an OCP FP8 E4M3 code, nearest-even, directly.
   E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
   field 0 holds the subnormals m * 2^-9; there are no infinities and
   S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448
   (code 0x7E).  Magnitudes at or above 448 saturate to it. */
uint8_t synth_f64_to_e4m3(double x) {
  const uint8_t sign = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  /* Unbiased exponent of a (clamped at the smallest normal exponent -6);
     the quantum of that binade is 2^(ue-3). */
  int fe = 0;
  if (a > 0.0) frexp(a, &fe); /* a = m 2^fe, m in [0.5, 1) */
  int ue = a > 0.0 ? fe - 1 : -6;
  if (ue < -6) ue = -6;
  const double n = nearbyint(ldexp(a, 3 - ue)); /* exact scaling, ties to even */
  const double r = ldexp(n, ue - 3);
  if (r < 0x1.0p-6) return (uint8_t)(sign | (uint8_t)n); /* subnormal or zero */
  int re = 0;
  frexp(r, &re);
  const int be = re - 1 + 7; /* 1..15 */
  const int man = (int)ldexp(r, 3 - (re - 1)) - 8;
  return (uint8_t)(sign | (uint8_t)(be << 3) | (uint8_t)man);
}

/* rows x cols values std * N(0,1)[start + r*cols + c], each row stored as
   E4M3 codes with one fp32 scale: scale_r = (float)(max_c |v_rc| / 448)
   (1 for an all-zero row), code_rc = E4M3(v_rc / scale_r). */
void synth_normal_e4m3_rows(uint64_t seed, uint64_t tensor_id, uint64_t start, uint64_t rows,
                            uint64_t cols, double std, uint8_t *codes, float *scale) {
  const uint64_t K = synth_stream_key(seed, tensor_id);
#pragma omp parallel
  {
    double *row = (double *)malloc(cols * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < (int64_t)rows; ++r) {
      uint64_t cached = UINT64_MAX;
      double c = 0.0, s = 0.0, amax = 0.0;
      for (uint64_t i = 0; i < cols; ++i) {
        const uint64_t e = start + (uint64_t)r * cols + i;
        if ((e >> 1) != cached) {
          cached = e >> 1;
          normal_pair(K, cached, &c, &s);
        }
        const double v = std * ((e & 1) ? s : c);
        row[i] = v;
        if (fabs(v) > amax) amax = fabs(v);
      }
      const float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
      scale[r] = sc;
      for (uint64_t i = 0; i < cols; ++i)
        codes[(uint64_t)r * cols + i] = synth_f64_to_e4m3(row[i] / (double)sc);
    }
    free(row);
  }
}

/* Round one fp64 value to an OCP E2M1 (FP4) code, nearest-even, saturating:
   1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
   0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7), no infinities or NaN. */
uint8_t synth_f64_to_e2m1(double x) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const uint8_t sign = signbit(x) ? 0x8u : 0u;
  const double a = fabs(x);
  if (isnan(x)) return sign; /* not produced by the generator */
  if (a >= 6.0) return (uint8_t)(sign | 7u);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    const double d = fabs(a - mag[c]), db = fabs(a - mag[best]);
    /* ties go to the code with an even mantissa bit (the even code) */
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)(sign | (uint8_t)best);
}

/* rows x cols values std * N(0,1)[start + r*cols + c] as OCP MXFP4: each run
   of 32 along a row shares the E8M0 scale 2^e with e = floor(log2(max |v|))
   - 2 (2 = the largest E2M1 exponent; e clamped to [-127, 127], 2^-127 for
   an all-zero block), and each element is E2M1(v / 2^e).  Element c of a row
   sits in byte c/2 of packed, the low nibble for even c.  cols % 32 == 0. */
void synth_normal_mxfp4_rows(uint64_t seed, uint64_t tensor_id, uint64_t start, uint64_t rows,
                             uint64_t cols, double std, uint8_t *packed, uint8_t *scale) {
  const uint64_t K = synth_stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)rows; ++r) {
    uint64_t cached = UINT64_MAX;
    double c0 = 0.0, s0 = 0.0;
    for (uint64_t b = 0; b < cols / 32; ++b) {
      double v[32], amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const uint64_t e = start + (uint64_t)r * cols + b * 32 + (uint64_t)i;
        if ((e >> 1) != cached) {
          cached = e >> 1;
          normal_pair(K, cached, &c0, &s0);
        }
        v[i] = std * ((e & 1) ? s0 : c0);
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
      }
      int ex = -127;
      if (amax > 0.0) {
        int fe = 0;
        frexp(amax, &fe); /* amax = m 2^fe, m in [0.5, 1): floor(log2) = fe - 1 */
        ex = fe - 1 - 2;
        if (ex < -127) ex = -127;
        if (ex > 127) ex = 127;
      }
      scale[(uint64_t)r * (cols / 32) + b] = (uint8_t)(ex + 127);
      for (int i = 0; i < 32; i += 2) {
        const uint8_t lo = synth_f64_to_e2m1(ldexp(v[i], -ex));
        const uint8_t hi = synth_f64_to_e2m1(ldexp(v[i + 1], -ex));
        packed[((uint64_t)r * cols + b * 32 + (uint64_t)i) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}
