// Device-side helpers shared by the library's kernels (gfx950 only).
//
// Element formats (Prime Inference write-up, "Making room for low-latency
// decode"): the latent is stored as four-bit E2M1 values with one E4M3
// scale per 16 values, the rope as E4M3.  Every E2M1 x E4M3 product has at
// most 6 significant bits and lies in [2^-10, 2688], so it is an exact FP16
// value; E4M3 values are FP16 values too.  Decoding to FP16 is therefore
// exact, and the helpers below do it with integer bit moves plus one FP16
// multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kQK = 576;
constexpr int kRowBytes = 352;
constexpr int kFp8RowBytes = 576;
constexpr int kScaleOff = 256;
constexpr int kRopeOff = 288;
constexpr int kMaxTopk = 2048;

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // byte k of the result = byte sel_k of the 8-byte value (hi:lo); 0x0C = 0x00
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// ---------------------------------------------------------------- decode

// Eight E2M1 codes packed in a dword (code 2i in the low nibble of byte i,
// code 2i+1 in the high nibble) -> eight FP16 values, in element order.
// The FP16 encodings of the E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 all
// have a zero low byte; their high bytes 00 38 3C 3E 40 42 44 46 form an
// 8-entry table that one byte permute indexes four values at a time.
__device__ __forceinline__ half8_t e2m1x8_to_half8(uint32_t w) {
  const uint32_t kLutLo = 0x3E3C3800u;  // magnitudes 0..3
  const uint32_t kLutHi = 0x46444240u;  // magnitudes 4..7
  uint32_t me = w & 0x07070707u;               // even elements' magnitudes
  uint32_t mo = (w >> 4) & 0x07070707u;        // odd elements' magnitudes
  uint32_t he = perm(kLutHi, kLutLo, me) | ((w << 4) & 0x80808080u);
  uint32_t ho = perm(kLutHi, kLutLo, mo) | (w & 0x80808080u);
  // interleave high bytes into FP16 pairs (low bytes zero): (e0,e1) (e2,e3) ...
  u32x4 r;
  r.x = perm(ho, he, 0x040C000Cu);
  r.y = perm(ho, he, 0x050C010Cu);
  r.z = perm(ho, he, 0x060C020Cu);
  r.w = perm(ho, he, 0x070C030Cu);
  return __builtin_bit_cast(half8_t, r);
}

// Two E4M3 bytes (b0 in bits 7:0 and b1 in bits 23:16 of `t`, other bits
// zero) -> two FP16 values.  Moving the 7 magnitude bits to bits 13:7 of an
// FP16 word gives the value times 2^-8 (normal and subnormal alike); the
// multiply by 256 restores it exactly.
__device__ __forceinline__ half2_t e4m3_pair_to_half2(uint32_t t) {
  uint32_t h = ((t & 0x007F007Fu) << 7) | ((t & 0x00800080u) << 8);
  return as_half2(h) * (half2_t){(half_t)256.0f, (half_t)256.0f};
}

// Four E4M3 bytes of a dword -> four FP16 values in byte order.
__device__ __forceinline__ half4_t e4m3x4_to_half4(uint32_t w) {
  half2_t a = e4m3_pair_to_half2(perm(0u, w, 0x0C010C00u));  // bytes 0,1
  half2_t b = e4m3_pair_to_half2(perm(0u, w, 0x0C030C02u));  // bytes 2,3
  return (half4_t){a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ half8_t e4m3x8_to_half8(uint32_t lo, uint32_t hi) {
  half4_t a = e4m3x4_to_half4(lo), b = e4m3x4_to_half4(hi);
  return (half8_t){a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// One E4M3 scale byte -> FP16 (s, s) pair.
__device__ __forceinline__ half2_t e4m3_to_half2_splat(uint32_t b) {
  return e4m3_pair_to_half2((b & 0xFFu) * 0x00010001u);
}

// Hardware conversions (gfx950 v_cvt_scalef32_pk_f16_{fp4,fp8}).  These
// instructions apply only the exponent of their float scale operand, so
// they are used with scale 1.0 (an exact E2M1 / E4M3 -> FP16 conversion);
// the E4M3 group scale is applied afterwards with one FP16 multiply, which
// is exact because every code x scale product is an FP16 value.
__device__ __forceinline__ half8_t e2m1x8_to_half8_hw(uint32_t w) {
  const half2_t a = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
  const half2_t b = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
  const half2_t c = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
  const half2_t d = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
  return (half8_t){a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ half8_t e4m3x8_to_half8_hw(uint32_t lo, uint32_t hi) {
  const half2_t a = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
  const half2_t b = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
  const half2_t c = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
  const half2_t d = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
  return (half8_t){a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Low byte of `b` (an E4M3 scale) as FP16, repeated eight times.
__device__ __forceinline__ half8_t e4m3_splat8_hw(uint32_t b) {
  const half2_t v = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b & 0xFFu, 1.0f, false));
  const half_t s = v.x;
  return (half8_t){s, s, s, s, s, s, s, s};
}

// ---------------------------------------------------------------- encode

// E4M3 magnitude code (7 bits) of a >= 0, round to nearest even,
// saturating to 448 (code 0x7E).  Works on the float32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_mag_rne(float a) {
  if (!(a < 448.0f)) return 0x7Eu;  // also catches +inf
  uint32_t b = __float_as_uint(a);
  int e = (int)(b >> 23) - 127;
  if (e >= -6) {
    uint32_t m = b & 0x7FFFFFu;
    uint32_t q = ((uint32_t)(e + 7) << 3) | (m >> 20);
    uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1u;  // carry may bump the exponent
    return q;
  }
  // below the smallest normal 2^-6 the grid is k * 2^-9, k = 0..8 (8 is 0x08 = 2^-6)
  return (uint32_t)__builtin_rintf(a * 512.0f);
}

// E4M3 byte of a finite float, sign bit copied from the input.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  return e4m3_mag_rne(__builtin_fabsf(x)) | ((__float_as_uint(x) >> 24) & 0x80u);
}

// E2M1 magnitude code (3 bits) of ax = |x| against scale s: round to
// nearest even on the grid {0,.5,1,1.5,2,3,4,6}*s, saturating at 6*s; 0 if
// s == 0.  Each threshold t*s has at most 7 significant bits, so it is
// exact in float32 and every decision matches the exact real comparison.
__device__ __forceinline__ uint32_t e2m1_mag(float ax, float s) {
  uint32_t m = (uint32_t)(ax > 0.25f * s) + (uint32_t)(ax >= 0.75f * s) +
               (uint32_t)(ax > 1.25f * s) + (uint32_t)(ax >= 1.75f * s) +
               (uint32_t)(ax > 2.5f * s) + (uint32_t)(ax >= 3.5f * s) +
               (uint32_t)(ax > 5.0f * s);
  return s > 0.0f ? m : 0u;
}

// The same against the two-level scale s * g: thresholds fl32((t * s) * g),
// t * s exact; with g = 1 identical to e2m1_mag.
__device__ __forceinline__ uint32_t e2m1_mag_scaled(float ax, float s, float g) {
  uint32_t m = (uint32_t)(ax > (0.25f * s) * g) + (uint32_t)(ax >= (0.75f * s) * g) +
               (uint32_t)(ax > (1.25f * s) * g) + (uint32_t)(ax >= (1.75f * s) * g) +
               (uint32_t)(ax > (2.5f * s) * g) + (uint32_t)(ax >= (3.5f * s) * g) +
               (uint32_t)(ax > (5.0f * s) * g);
  return s > 0.0f ? m : 0u;
}

// Decoded value of an E4M3 magnitude code (for encoders that need the
// rounded scale as a float).
__device__ __forceinline__ float e4m3_mag_value(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 0u) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------- fp16/bf16 I/O

__device__ __forceinline__ float bf16_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace mla
