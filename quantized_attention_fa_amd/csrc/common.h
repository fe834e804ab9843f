// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// access, bit-exact format encoders, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define FAQ_DEV static __device__ __forceinline__

// ---------------------------------------------------------------- bf16 / fp32

FAQ_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
FAQ_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round a finite float to bf16 (nearest, ties to even); returns the bits.
FAQ_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// Load 8 consecutive input elements (fp32, or bf16 held as uint16_t) as floats.
FAQ_DEV void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

FAQ_DEV void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
  v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
  v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

// ---------------------------------------------------------------- encoders
//
// Every encoder takes the already-divided float32 quotient u = fl32(x / s)
// and rounds it to the nearest code, ties to the even code.

// INT8: clamp(round_half_even(u), -128, 127).
FAQ_DEV int32_t enc_int8(float u) {
  float r = __builtin_rintf(u);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int32_t)r;
}

// FP8 E4M3FN (bias 7, 3 mantissa bits, no inf, S.1111.111 = NaN): nearest
// value, ties to even mantissa, |u| > 448 saturating to 0x7E, sign kept.
FAQ_DEV uint32_t enc_e4m3(float u) {
  const uint32_t b = __float_as_uint(u);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  // normal range (|u| >= 2^-6): drop 20 mantissa bits with round-half-even,
  // then rebias the exponent from 127 to 7.
  uint32_t rn = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  uint32_t cn = rn - (120u << 3);
  cn = cn > 0x7eu ? 0x7eu : cn;
  // subnormal range: k * 2^-9 with k = round_half_even(|u| * 2^9) in 0..8
  // (k = 8 is the smallest normal, code 0x08).
  uint32_t cs = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | (a >= 0x3c800000u ? cn : cs);
}

// FP8 E5M2 (bias 15, 2 mantissa bits) of a non-negative-or-signed value that
// is at most 6 in magnitude (no saturation needed): nearest, ties to even.
FAQ_DEV uint32_t enc_e5m2_small(float u) {
  const uint32_t b = __float_as_uint(u);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t rn = (a + 0xfffffu + ((a >> 21) & 1u)) >> 21;
  uint32_t cn = rn - (112u << 2);
  // subnormal: k * 2^-16, k = round_half_even(|u| * 2^16) in 0..4
  uint32_t cs = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
  return sign | (a >= 0x38800000u ? cn : cs);
}

// E2M1 magnitude code of |v| (0..7 for 0, .5, 1, 1.5, 2, 3, 4, 6): nearest,
// ties to even code, saturating at 6.
FAQ_DEV uint32_t enc_e2m1_mag(float a) {
  uint32_t c = 0;
  c += a > 0.25f;
  c += a >= 0.75f;
  c += a > 1.25f;
  c += a >= 1.75f;
  c += a > 2.5f;
  c += a >= 3.5f;
  c += a > 5.0f;
  return c;
}

FAQ_DEV uint32_t enc_e2m1(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  return sign | enc_e2m1_mag(fabsf(v));
}

// Shared MX exponent E = clamp(floor(log2 amax) - EMAX, -127, 127), exact
// from the float's exponent bits; zero or subnormal amax gives -127.  EMAX
// is the exponent of the element format's largest normal: 2 for E2M1
// (max 6), 8 for E4M3 (max 448).
template <int EMAX = 2>
FAQ_DEV int mx_exponent(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  int E = e - 127 - EMAX;
  E = E < -127 ? -127 : E;
  E = E > 127 ? 127 : E;
  return e == 0 ? -127 : E;
}

// ---------------------------------------------------------------- reductions

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the in-register row swaps of gfx950 (no LDS round trip).
FAQ_DEV float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// x of another lane by a DPP pattern (all lanes active, in-row sources)
template <int CTRL>
FAQ_DEV float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max over aligned groups of WIDTH lanes, all lanes active, in registers:
// quad swaps (lane ^ 1, lane ^ 2), the half-row and row mirrors (lane
// 7 - i within 8, 15 - i within 16), then the row swaps for a whole wave.
template <int WIDTH>
FAQ_DEV float group_max(float v) {
  static_assert(WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16 || WIDTH == 64, "group width");
  if constexpr (WIDTH >= 2) v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  if constexpr (WIDTH >= 4) v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  if constexpr (WIDTH >= 8) v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  if constexpr (WIDTH >= 16) v = fmaxf(v, dpp_f<0x140>(v)); // row_mirror
  if constexpr (WIDTH == 64) v = rows4_max(v);
  return v;
}

FAQ_DEV float wave_max(float v) { return group_max<64>(v); }

FAQ_DEV float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------- division
//
// The quantizers divide every element by its scale, correctly rounded.  A
// full IEEE division costs about ten instructions; with r = RN(1/s) taken
// once per scale, the quotient is q0 = x r (within an ulp), the residual
// x - q0 s is exact under fma, and one correction q0 + (x - q0 s) r rounds
// to the IEEE quotient (Markstein's theorem for round-to-nearest).  The
// theorem needs x, s, the quotient and the residual to be normal numbers:
// callers take this path only for s in [2^-80, 2^80] and rely on it only
// for quotients that can decide a code (|q| >= 2^-12, where all four are
// normal); smaller quotients stay smaller than any code boundary.

FAQ_DEV bool div_fast_ok(float s) { return s >= 0x1p-80f && s <= 0x1p80f; }

FAQ_DEV float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
}

// The sign of x on q (x / s has the sign of x for s > 0; the correction
// step alone turns x = -0 into +0).
FAQ_DEV float with_sign_of(float q, float x) {
  return __uint_as_float((__float_as_uint(q) & 0x7fffffffu) | (__float_as_uint(x) & 0x80000000u));
}

// INT8 code of x / s, clamp(rne(fl32(x / s)), -128, 127), in the low byte
// of the returned word: adding 1.5 * 2^23 to the clamped quotient rounds it
// to an integer (ties to even) held in the low mantissa bits.  On the fast
// path x r is first clamped to +-256, which keeps the correction finite for
// inputs far beyond the scale (their codes saturate either way).
template <bool FAST>
FAQ_DEV uint32_t int8_code_word(float x, float s, float r) {
  float q;
  if (FAST) {
    const float q0 = __builtin_amdgcn_fmed3f(x * r, -256.0f, 256.0f);
    q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
  } else {
    q = x / s;
  }
  return __float_as_uint(__builtin_amdgcn_fmed3f(q, -128.0f, 127.0f) + 0x1.8p23f);
}

// Low bytes of a, b, c, d as one word (a in byte 0).
FAQ_DEV uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// E4M3 codes of x0 / s .. x3 / s (nearest, ties to even) packed in a word,
// x0 in byte 0.  The hardware conversion rounds to nearest even and keeps
// the sign; every quotient here is at most 448 in magnitude.
template <bool FAST>
FAQ_DEV uint32_t e4m3_code_word(const float* x, float s, float r) {
  float q[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) q[k] = FAST ? with_sign_of(div_rn(x[k], s, r), x[k]) : x[k] / s;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  return (uint32_t)w;
}

// N / 4 code words of x[0..N) / s: the fast division, redone with IEEE
// divisions by the rare lanes whose scale is outside the fast path's range
// (a wave-uniform test first, so the common case skips that code).
template <int N>
FAQ_DEV void e4m3_code_words(const float* x, float s, uint32_t* w) {
  const float r = 1.0f / s;
#pragma unroll
  for (int j = 0; j < N / 4; ++j) w[j] = e4m3_code_word<true>(x + 4 * j, s, r);
  const bool slow = !div_fast_ok(s);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(slow) != 0, 0)) {
    if (slow) {
#pragma unroll
      for (int j = 0; j < N / 4; ++j) w[j] = e4m3_code_word<false>(x + 4 * j, s, r);
    }
  }
}

// E4M3 codes of x0 / s .. x3 / s for a static scale, where inputs beyond the
// calibrated range occur: quotients saturate at +-448 (the hardware
// conversion is only used within that range).  On the fast path x r is
// first clamped to +-512 (the correction then stays finite; quotients that
// large saturate either way).
template <bool FAST>
FAQ_DEV uint32_t e4m3_sat_code_word(const float* x, float s, float r) {
  float q[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float d;
    if (FAST) {
      const float q0 = __builtin_amdgcn_fmed3f(x[k] * r, -512.0f, 512.0f);
      d = __builtin_fmaf(__builtin_fmaf(-q0, s, x[k]), r, q0);
    } else {
      d = x[k] / s;
    }
    q[k] = with_sign_of(__builtin_amdgcn_fmed3f(d, -448.0f, 448.0f), x[k]);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  return (uint32_t)w;
}

// N / 4 words of INT8 codes of x[0..N) / s (x0 in byte 0 of word 0), with
// the same wave-uniform fallback to IEEE division as e4m3_code_words.
template <int N>
FAQ_DEV void int8_code_words(const float* x, float s, uint32_t* w) {
  const float r = 1.0f / s;
#pragma unroll
  for (int j = 0; j < N / 4; ++j)
    w[j] = pack_low_bytes(int8_code_word<true>(x[4 * j], s, r), int8_code_word<true>(x[4 * j + 1], s, r),
                          int8_code_word<true>(x[4 * j + 2], s, r), int8_code_word<true>(x[4 * j + 3], s, r));
  const bool slow = !div_fast_ok(s);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(slow) != 0, 0)) {
    if (slow) {
#pragma unroll
      for (int j = 0; j < N / 4; ++j)
        w[j] = pack_low_bytes(int8_code_word<false>(x[4 * j], s, r), int8_code_word<false>(x[4 * j + 1], s, r),
                              int8_code_word<false>(x[4 * j + 2], s, r), int8_code_word<false>(x[4 * j + 3], s, r));
    }
  }
}

// ---------------------------------------------------------------- misc

FAQ_DEV float scale_from_amax(float amax, float qmax) {
  return amax == 0.0f ? 1.0f : amax / qmax;  // IEEE division
}

// Workgroup barrier without a memory fence (a fence would wait for every
// global access in flight): this wave's LDS reads and writes complete first
// (lgkmcnt(0)); global loads - and copies into LDS - may stay in flight,
// their completion being waited for with vmcnt where their data is used.
// The signal fences keep the compiler from moving memory accesses across
// it.
FAQ_DEV void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
