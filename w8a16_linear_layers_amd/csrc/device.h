// Device helpers shared by the kernels: bf16 unpacking, the float -> OCP
// E4M3 conversion with saturation and round-to-nearest-even, the static
// quantization rule and the SwiGLU element rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-bit activation formats: kF16 = false is bf16, true is IEEE binary16.
// Unpacking is exact; packing rounds to nearest even (binary16 overflows to
// an infinity, as the conversion instruction does by default).
template <bool kF16>
__device__ __forceinline__ float h16_lo(uint32_t w) {
  if constexpr (kF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  else return bf16_lo(w);
}
template <bool kF16>
__device__ __forceinline__ float h16_hi(uint32_t w) {
  if constexpr (kF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else return bf16_hi(w);
}
template <bool kF16>
__device__ __forceinline__ uint32_t h16x2(float a, float b) {
  // one packed round-to-nearest-even convert of the pair
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
  } else {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
  }
}

// Saturate to the finite E4M3 range; +-Inf become +-448.
__device__ __forceinline__ float clamp448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// E4M3 code of a finite value already inside [-448, 448]: the gfx950
// converter rounds to nearest even and keeps the sign of zero.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
}

// Bracketing factors 1 -+ 2^-21 (both exact in float32).
constexpr float kBelow = 1.0f - 0x1p-21f;
constexpr float kAbove = 1.0f + 0x1p-21f;

// Fast static quantization of two bf16 values packed in `w`.
//
// The exact code is E4M3(RN32(x / s)). With r = RN32(1 / s) the product
// q = RN32(x * r) is within 1.5 float32 ulp of RN32(x / s) whenever q is a
// normal float, so RN32(x / s) lies between RN32(q * (1 - 2^-21)) and
// RN32(q * (1 + 2^-21)) (each at least 3 ulp away from q). E4M3 rounding is
// monotone, so when both bracket ends give the same code that code is exact.
// If q is subnormal or zero, every candidate is below 2^-11 and the code is
// a signed zero either way; if x * r overflows, the quotient saturates too.
// A disagreement (a value within a few ulp of an E4M3 rounding midpoint) or
// a NaN input sets `doubt`, and the caller redoes the vector exactly.
//
// Returns the two codes in bytes 0 and 2 (bytes 1 and 3 hold the upper
// bracket's codes).
__device__ __forceinline__ uint32_t quant_pair_fast(uint32_t w, float r, uint32_t& doubt) {
  const float q0 = bf16_lo(w) * r;
  const float q1 = bf16_hi(w) * r;
  uint32_t p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(q0 * kBelow), clamp448(q0 * kAbove), 0, false);
  p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(q1 * kBelow), clamp448(q1 * kAbove), (int)p, true);
  doubt |= (p ^ (p >> 8)) & 0x00ff00ffu;
  // bf16 NaN: magnitude bits above 0x7f80 (adding 0x7f carries into bit 15)
  doubt |= ((w & 0x7fff7fffu) + 0x007f007fu) & 0x80008000u;
  return p;
}

// Four codes from two quant_pair_fast results: bytes 0 and 2 of each.
__device__ __forceinline__ uint32_t pick_codes(uint32_t p0, uint32_t p1) {
  return (p0 & 0xffu) | ((p0 >> 8) & 0xff00u) | ((p1 & 0xffu) << 16) | ((p1 << 8) & 0xff000000u);
}

// Static quantization of two bf16 values for a power-of-two scale s = 2^k:
// r = 2^-k exactly, so q = x * r IS the exact quotient (or is below 2^-126,
// where every candidate code is a signed zero, or overflows, where the
// quotient saturates either way) and needs no bracket. Only a NaN input
// sets `doubt`.
// The four codes of two such words (bytes 0-3 from w0 lo, w0 hi, w1 lo,
// w1 hi): two packed converts, no byte shuffling.
__device__ __forceinline__ uint32_t quant_quad_pow2(uint32_t w0, uint32_t w1, float r, uint32_t& doubt) {
  uint32_t p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(bf16_lo(w0) * r), clamp448(bf16_hi(w0) * r), 0,
                                                         false);
  p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(bf16_lo(w1) * r), clamp448(bf16_hi(w1) * r), (int)p, true);
  doubt |= (((w0 & 0x7fff7fffu) + 0x007f007fu) | ((w1 & 0x7fff7fffu) + 0x007f007fu)) & 0x80008000u;
  return p;
}

// Exact static quantization of one bf16 value (bits in the low 16 bits).
// If q = x * (1/s) satisfies q * s == x exactly (FMA residual zero), q is
// the exact quotient and its code is final. That test is sound when the
// residual cannot underflow to zero, i.e. for s >= 2^-92 (`exact_ok`): a
// nonzero residual of a code-relevant quotient (|q| >= 2^-11) is then at
// least 2^-149. Otherwise the IEEE correctly rounded float32 division.
__device__ __forceinline__ uint32_t quant_one_exact(uint32_t bits, float s, float r, bool exact_ok) {
  const float x = __uint_as_float(bits << 16);
  if (__builtin_isnan(x)) return 0x7fu | ((bits >> 8) & 0x80u);
  const float q0 = x * r;
  if (exact_ok && __builtin_fmaf(-q0, s, x) == 0.0f) return e4m3_code(clamp448(q0));
  const float q = x / s;  // correctly rounded division (hipcc default)
  return e4m3_code(clamp448(q));
}

__device__ __forceinline__ uint32_t quant_word_exact(uint32_t w, float s, float r, bool exact_ok) {
  return quant_one_exact(w & 0xffffu, s, r, exact_ok) | (quant_one_exact(w >> 16, s, r, exact_ok) << 8);
}

// e^x on the exp2 instruction (v_exp_f32): x log2(e) = hi + lo, with hi =
// fl32(x L) and lo its rounding error recovered by an FMA plus x times the
// tail of log2(e), and e^x = 2^hi (1 + lo ln 2) to first order in lo (|lo|
// <= 2^-17). About 2 float32 ulp in all (the instruction's 1 ulp, two
// roundings); overflow gives inf and underflow 0, with no NaN in between.
__device__ __forceinline__ float exp_via_exp2(float x) {
  constexpr float kL = 0x1.715476p+0f;       // log2(e) rounded to float32
  constexpr float kLtail = 0x1.4ae0cp-26f;   // log2(e) - kL
  constexpr float kLn2 = 0x1.62e43p-1f;
  const float hi = x * kL;
  const float lo = fmaf(x, kLtail, fmaf(x, kL, -hi));
  return __builtin_amdgcn_exp2f(hi) * fmaf(lo, kLn2, 1.0f);
}

// SwiGLU element rule ([TRT-17476] "What changed": silu(g) * u in float32
// from the two 16-bit inputs, emitted as E4M3 with the down projection's
// static input scale). silu(g) * u = g * u / (1 + exp(-g)), so h stays
// within a few float32 ulp of the exact value for every finite input; a
// very negative gate gives exp(-g) = inf and h = -0 or 0, a large gate gives
// g * u. Shared by the two-input SwiGLU kernel and the fused gate/up
// epilogue, so both produce the same codes from the same inputs.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = exp_via_exp2(-g);
  return (g * u) * __builtin_amdgcn_rcpf(1.0f + e);
}

// E4M3 code of h * rs (rs = 1 / s_h); NaN keeps its sign as S.1111.111.
__device__ __forceinline__ uint32_t swiglu_code(float h, float rs) {
  const float t = h * rs;
  if (__builtin_isnan(t)) return 0x7fu | ((__float_as_uint(t) >> 24) & 0x80u);
  return e4m3_code(clamp448(t));
}

// The codes of h[0..3] * rs in one word (byte k from h[k]), by the rule of
// swiglu_code: two packed converts of the clamped values; a word holding a
// NaN (rare; their sum is then NaN, as it is for +inf + -inf) is redone
// element by element.
__device__ __forceinline__ uint32_t swiglu_codes4(float h0, float h1, float h2, float h3, float rs) {
  const float t0 = h0 * rs, t1 = h1 * rs, t2 = h2 * rs, t3 = h3 * rs;
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(t0), clamp448(t1), 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(t2), clamp448(t3), (int)w, true);
  const float probe = (t0 + t1) + (t2 + t3);
  if (__builtin_isnan(probe))
    w = swiglu_code(h0, rs) | (swiglu_code(h1, rs) << 8) | (swiglu_code(h2, rs) << 16) | (swiglu_code(h3, rs) << 24);
  return w;
}

}  // namespace fp8lin
