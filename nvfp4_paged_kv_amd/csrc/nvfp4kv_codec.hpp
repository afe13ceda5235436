// nvfp4kv_codec.hpp -- NVFP4 (E2M1 elements + E4M3 block scales) codec used by
// the gfx950 append and attention kernels.
//
// Format (FlashInfer PR #4769 page, introduction: NVFP4 KV tiles are E2M1
// values with E4M3 scale factors; the decode of an element is
// e2m1(code) * E4M3(sf) * g with g the per-tensor global decode scale of the
// PR #6204 page's append docstring section):
//   * a block is 16 consecutive head_dim elements of one (token, head);
//   * E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa,
//     magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6};
//   * E4M3 scale byte: OCP E4M3FN, unsigned use, largest finite 448 (0x7E).
//
// The block quantizer follows one fixed fp32 operation order so that results
// are reproducible bit for bit:
//   a = max|x_i| (NaN ignored); s = a / (6 g); sf = E4M3_rne_satfinite(s);
//   r = sf ? 1 / (S g) : 0;  code_i = sign(x_i) | E2M1_rne_sat(x_i * r).
//
// Everything here is plain integer / fp32 code usable from device and host,
// so the host build can check the device logic on the CPU.
#pragma once
#include <stdint.h>

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
#define NVFP4KV_HD __host__ __device__ __forceinline__
#else
#define NVFP4KV_HD static inline
#endif

namespace nvfp4kv {

// Device error-flag bits (also declared in include/nvfp4kv.h).
constexpr uint32_t kErrBadKScale = 1u;
constexpr uint32_t kErrBadVScale = 2u;
constexpr uint32_t kErrSlotOob = 4u;
constexpr uint32_t kErrPageOob = 8u;

NVFP4KV_HD float u2f(uint32_t u) {
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}
NVFP4KV_HD uint32_t f2u(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  return u;
}

// Global decode scale validity: positive and finite.
NVFP4KV_HD bool scale_ok(float g) { return (f2u(g) - 1u) < 0x7F7FFFFFu; }

// E4M3FN encode of a block scale s >= 0 (never negative here): round to
// nearest, ties to even; s >= 448 (and +inf) saturate to 0x7E; zero and NaN
// give 0.
NVFP4KV_HD uint32_t e4m3_encode(float s) {
  uint32_t u = f2u(s);
  if (!(s > 0.0f)) return 0u;
  if (s >= 448.0f) return 0x7Eu;
  if (u < 0x3C800000u) {  // s < 2^-6: subnormal codes are multiples of 2^-9
    // s * 2^9 is exact; adding 2^23 rounds it to an integer with ties to even
    float t = s * 512.0f + 8388608.0f;
    return f2u(t) - 0x4B000000u;  // 0..8 (8 is the smallest normal, 2^-6)
  }
  // normal: keep 3 mantissa bits with round-half-even, rebias 127 -> 7
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

// Exact fp32 value of a non-NaN, non-negative E4M3 code.
NVFP4KV_HD float e4m3_decode(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  return e ? u2f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// E2M1 magnitude (0..7) of a non-NaN fp32 given as |bits| (sign cleared):
// round to nearest, ties to the even code, saturating at 6 (code 7).
NVFP4KV_HD uint32_t e2m1_mag_from_abs_bits(uint32_t u) {
  // |y| < 2: the grid step is 0.5 = ulp(2^22), so adding 2^22 rounds to it.
  uint32_t lo = f2u(u2f(u) + 4194304.0f) - 0x4A800000u;
  // |y| >= 2: keep one mantissa bit (round half even); (E<<1|m) - 252 is the code
  uint32_t r = (u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22;
  uint32_t hi = r - 252u;
  hi = hi < 7u ? hi : 7u;
  return u < 0x40000000u ? lo : hi;
}

// Unsigned division by a fixed divisor d (1 <= d < 2^31) through a
// multiply-high (the round-up method of Granlund & Montgomery, 1994), valid
// for every 32-bit dividend.
struct FastDiv {
  uint32_t mul, shift, d;
};
static inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.shift = l;
  f.mul = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  return f;
}
NVFP4KV_HD uint32_t fastdiv(uint32_t n, FastDiv f) {
  // branch-free (a select for d = 1, where shift is 0), so that it does not
  // split the straight-line code it is used in
  uint32_t t = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  uint32_t q = (t + ((n - t) >> 1)) >> ((f.shift - 1) & 31u);
  return f.shift ? q : n;
}

}  // namespace nvfp4kv

#if defined(__HIPCC__)
namespace nvfp4kv {
// gfx950 hardware FP4 conversion of two fp32 values (scale operand 1.0, so
// the values are converted as they are): returns `old` with byte `SEL`
// replaced by the packed pair (first value in the low nibble).  Only finite
// values and +-inf reach this in the append kernel; its rounding, saturation
// and sign handling are checked against the oracle over every fp32 pattern
// by the GPU probe tests.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk_e2m1(uint32_t old, float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, SEL);
#else
  return old;  // host pass: never called
#endif
}
}  // namespace nvfp4kv
#endif
