// Device-side helpers shared by the q4rac HIP kernels (gfx950).
//
// NVFP4 format: QUADS (arXiv 2607.15810) section 2.2 paragraph "FP4" -- E2M1
// codes {0,0.5,1,1.5,2,3,4,6}, an E4M3 scale per sixteen elements (maximum 448,
// paragraph "FP8") and an FP32 tensor scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef int i32x8v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kScoreTileRows = 32;   // rows summed in order into one tile sum
constexpr int kScoreGroupTiles = 8;  // tile sums added in order into one group sum

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------ E4M3
// Value of a non-negative E4M3 code 0..126: 2^(e-7) (1 + m/8), subnormal m 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  float sub = (float)m * 0x1p-9f;
  float nor = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e ? nor : sub;
}

// Nearest E4M3 code of a non-negative fp32 value (ties to even), saturating at
// 448.  Used on an approximate quotient; the caller corrects it exactly.
__device__ __forceinline__ uint32_t e4m3_code_near(float u) {
  if (u >= 448.0f) return 126u;
  if (u < 0x1p-6f) return (uint32_t)__builtin_rintf(u * 512.0f);
  uint32_t b = __float_as_uint(u);
  uint32_t r = (b + 0x7ffffu + ((b >> 20) & 1u)) & 0xfff00000u;
  return (r >> 20) - (120u << 3);
}

// Exact E4M3 block-scale code: the E4M3 value nearest to a / (6 s_t) on the
// exact real quotient, ties to the even code, saturating at 448.
//   a      block amax (a bf16 value, exact in fp32)
//   inv6st approximate 1 / (6 s_t) (any rounding)
//   st6    6 s_t in fp64 (exact: 26 significant bits)
// The approximate quotient lands on the right code or a neighbour; one exact
// comparison of a with st6 * midpoint (<= 31 significant bits, exact in fp64)
// settles it.
__device__ __forceinline__ uint32_t e4m3_scale_code(float a, float inv6st, double st6) {
  float u = a * inv6st;
  uint32_t c = e4m3_code_near(u);
  float vc = e4m3_to_f32(c);
  double ad = (double)a;
  if (u >= vc) {
    if (c < 126u) {
      double t = st6 * (0.5 * ((double)vc + (double)e4m3_to_f32(c + 1u)));
      if (ad > t || (ad == t && ((c + 1u) & 1u) == 0u)) c += 1u;
    }
  } else if (c > 0u) {
    double t = st6 * (0.5 * ((double)e4m3_to_f32(c - 1u) + (double)vc));
    if (ad < t || (ad == t && (c & 1u) != 0u)) c -= 1u;
  }
  return c;
}

// ------------------------------------------------------------------ E2M1
__device__ __forceinline__ float e2m1_mag(uint32_t m) {
  // 0, 0.5, 1, 1.5, 2 | 3, 4, 6
  return m <= 4u ? (float)m * 0.5f : (m == 5u ? 3.0f : (m == 6u ? 4.0f : 6.0f));
}

__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  float v = e2m1_mag(nib & 7u);
  return (nib & 8u) ? -v : v;
}

// Exact E2M1 nibble of x against the scale S = s * st (both fp32, s with at
// most 4 significant bits, or a power of two): the magnitude nearest to
// |x| / S on exact reals, ties to the even code, saturating at 6; sign bit of x.
// Thresholds (midpoint * s) * st are exact in fp64.
__device__ __forceinline__ uint32_t e2m1_nibble_exact(float x, float s, float st) {
  uint32_t sign = (__float_as_uint(x) >> 31) << 3;
  if (s == 0.0f) return sign;
  double ax = (double)fabsf(x);
  double S = (double)s * (double)st;
  // midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5; ties go up where the upper code is even
  uint32_t m = 0;
  m += (ax > 0.25 * S) ? 1u : 0u;
  m += (ax >= 0.75 * S) ? 1u : 0u;
  m += (ax > 1.25 * S) ? 1u : 0u;
  m += (ax >= 1.75 * S) ? 1u : 0u;
  m += (ax > 2.5 * S) ? 1u : 0u;
  m += (ax >= 3.5 * S) ? 1u : 0u;
  m += (ax > 5.0 * S) ? 1u : 0u;
  return sign | m;
}

// ------------------------------------------------------------------ tensor scales
// Y = s_A s_W * sum, without letting the product of the two tensor scales
// underflow: when s_A s_W is a normal fp32 number one multiply by it (one
// rounding of the exact product s_A s_W sum), otherwise the mantissas and the
// exponents apart, fA fW (one rounding) and an exact power-of-two scaling, so
// that only a result that is itself subnormal loses bits.
struct OutScale {
  float mul;   // s_A s_W, or fA fW when split
  int e;       // eA + eW when split
  bool split;
};

__device__ __forceinline__ OutScale out_scale(float sa, float sw) {
  OutScale o;
  o.mul = sa * sw;
  o.e = 0;
  o.split = !(o.mul >= 0x1p-126f);
  if (o.split) {
    int ea, ew;
    const float fa = frexpf(sa, &ea), fw = frexpf(sw, &ew);
    o.mul = fa * fw;
    o.e = ea + ew;
  }
  return o;
}

__device__ __forceinline__ float apply_scale(const OutScale& o, float v) {
  return o.split ? ldexpf(v * o.mul, o.e) : v * o.mul;
}

// ------------------------------------------------------------------ wave ops
__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace q4
