// NVFP4 / MXFP4 encoding of one lane's elements of a row (gfx950 device code),
// shared by the stand-alone quantizer and the quantizing GEMM epilogue.
//
// QUADS (arXiv 2607.15810) section 2.2 "FP4": E2M1 codes with one E4M3 scale
// per 16 elements and an FP32 tensor scale (NVFP4), or one E8M0 scale per 32
// elements (MXFP4); codes round to nearest, ties to the even code.
#pragma once

#include "q4_device.h"

namespace q4 {

// How the codes of elements whose x / (s s_t) lies within 2^-20 of an E2M1
// rounding midpoint are decided (uniform per launch).
//
// With s_t = RN32(a / 2688) taken from the tensor's bf16 amax a, every such
// element is an exact tie of rationals, x * 2688 = mid * a * s: x (8
// significant bits) * 21 and mid * a * s (3 + 8 + 4 bits) differ by at least
// one part in 2^15 otherwise, far outside the 2^-20 window.  For an exact tie
// |x| - mid * s * s_t has the sign of a / 2688 - s_t, the same for every
// element of the launch: the tie rounds up in magnitude when s_t was rounded
// down, down when it was rounded up, and to the even code when the quotient
// was exact.  MXFP4 (s a power of two, no s_t) only has exact ties: even.
// A supplied s_t of the same form, RN32(a / 2688) for some bf16 a (a scale
// kept from an earlier amax), has the same structure; any other supplied s_t
// has none, and each element near a midpoint is then settled exactly.
enum TieMode : int { kTieUp = 0, kTieDown = 1, kTieEven = 2, kTieExact = 3 };

// tie mode of s_t against the bf16 amax a it is the rounded quotient of
__device__ __forceinline__ int tie_mode_of(float st, float a) {
  const double back = (double)st * 2688.0;   // exact: 24 + 5 significant bits
  return back < (double)a ? kTieUp : (back > (double)a ? kTieDown : kTieEven);
}

// tie mode of a supplied s_t: that of the bf16 amax it is the rounded
// quotient of, when there is one; otherwise every near tie is settled exactly
__device__ __forceinline__ int supplied_tie_mode(float st) {
  int mode = kTieExact;
  if (st > 0.0f && st <= 0x1p100f && st >= 0x1p-100f) {
    // the bf16 nearest to s_t * 2688 is the only amax s_t can come from
    const uint32_t pb = __float_as_uint((float)((double)st * 2688.0));
    const float ac = __uint_as_float((pb + 0x7fffu + ((pb >> 16) & 1u)) & 0xffff0000u);
    if ((float)((double)ac / 2688.0) == st) mode = tie_mode_of(st, ac);
  }
  return mode;
}

// lane l <- lane l^1 / l^2 inside a quad (DPP quad permutes)
__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// E4M3 rounding of u = a / D for a block amax a = (1 + ma/128) 2^ea (a normal
// bf16) and D = 6 s_t = Dp 2^eDp, Dp in [1, 2): the mantissa decision depends
// on ma alone, so one exact table per launch covers every normal case.
// Entry = E4M3 mantissa m (3 bits) | (exponent adjust + 1) << 3.
// The comparisons num vs Dp * (17 + 2j) / 16 are exact in fp64 (<= 31 bits).
__device__ uint32_t e4m3_mantissa_entry(int ma, double Dp) {
  const double A = 1.0 + ma / 128.0;
  int adj = 0;
  double num = A;
  if (A < Dp) {
    adj = -1;
    num = 2.0 * A;
  }
  int m = 0;
  for (int j = 0; j < 8; ++j) {
    const double t = Dp * (1.0 + (2 * j + 1) / 16.0);
    if (num > t || (num == t && ((j + 1) & 1) == 0)) m = j + 1;   // ties to even mantissa
  }
  if (m == 8) {
    m = 0;
    adj += 1;
  }
  return (uint32_t)(m | ((adj + 1) << 3));
}
// element pos of a lane's row, from its raw words v0 (channels 0-7) and v1
// (channels 8-15; ignored when CPL = 8), by selects only
template <int CPL>
__device__ __forceinline__ float lane_x(uint4 v0, uint4 v1, int pos) {
  const int d = pos >> 1;
  const bool hi4 = CPL == 16 && (d & 4);
  const uint32_t x = hi4 ? v1.x : v0.x, y = hi4 ? v1.y : v0.y;
  const uint32_t z = hi4 ? v1.z : v0.z, w = hi4 ? v1.w : v0.w;
  const uint32_t lo2 = (d & 2) ? z : x, hi2 = (d & 2) ? w : y;
  const uint32_t wd = (d & 1) ? hi2 : lo2;
  return (pos & 1) ? bf16_hi(wd) : bf16_lo(wd);
}

// 4 * (E2M1 midpoint above magnitude m), m = 0..6: 1 3 5 7 10 14 20
__device__ __forceinline__ float e2m1_mid_above(uint32_t m) {
  const uint32_t q = __builtin_amdgcn_perm(0x00140e0au, 0x07050301u, m);
  return (float)(q & 255u) * 0.25f;
}

// The exact path of nvfp4_lane_encode: the block scale (NVFP4: from the block
// amax m; MXFP4: *sc and *s as given) and the codes of the lane's CPL elements
// (raw words v0, v1) one element at a time.  Returns the code words.
template <bool MX, int CPL>
__device__ __forceinline__ uint2 nvfp4_lane_exact(uint4 v0, uint4 v1, float m, float st,
                                                  float inv6st, double st6, uint32_t* sc,
                                                  float* s) {
  if constexpr (!MX) {
    *sc = m == 0.0f ? 0u : e4m3_scale_code(m, inv6st, st6);
    *s = e4m3_to_f32(*sc);
  }
  uint32_t c[2] = {0u, 0u};
#pragma unroll 1
  for (int i = 0; i < CPL; ++i) {
    const uint32_t nib = e2m1_nibble_exact(lane_x<CPL>(v0, v1, i), *s, st);
    const uint32_t sh = 4u * (uint32_t)(i & 7);
    if (i < 8) c[0] |= nib << sh;
    else c[1] |= nib << sh;
  }
  return make_uint2(c[0], c[1]);
}

// the same as a called function (for a caller whose registers are scarce,
// where inlining the rare path costs more than the call)
template <bool MX, int CPL>
__device__ __attribute__((noinline)) uint2 nvfp4_lane_exact_call(uint4 v0, uint4 v1, float m,
                                                                 float st, float inv6st,
                                                                 double st6, uint32_t* sc,
                                                                 float* s) {
  return nvfp4_lane_exact<MX, CPL>(v0, v1, m, st, inv6st, st6, sc, s);
}

// Codes and block scale of one lane's CPL elements of a row (xf, decoded from
// the raw bf16 words w, which the rare exact paths re-read) given the block
// amax m (already reduced over the lanes that share the block), the tensor
// scale st (NVFP4; 1 for MXFP4), its table `tab` (e4m3_mantissa_entry for
// 6 st = Dp 2^eDp, Dp in [1, 2)), inv6st = 1 / (6 st), st6 = 6 st in fp64 and
// the launch's tie mode.  Out: code[CPL / 8] (eight nibbles each, element 0
// in the low nibble), the scale code *sc and its value *s.
//
// Codes: the FP4 conversion instruction on v * (1 - 2^-20) and v * (1 + 2^-20),
// v = x / (s s_t) (approximate reciprocal, relative error < 2^-22).  Where the
// two brackets agree the code is exact.  Where they differ, x lies within
// 2^-20 of a rounding midpoint; the tie mode settles it, or (kTieExact) each
// such element is settled by comparing |x| with midpoint * s * s_t, exact in
// fp32, one element per lane per round, all lanes of the wave at once.
template <bool MX, int CPL, bool CALL_EXACT = false>
__device__ __forceinline__ void nvfp4_lane_encode(const uint4* w, const float* xf, float m,
                                                  float st, int eDp, const uint8_t* tab,
                                                  float inv6st, double st6, int tie_mode,
                                                  uint32_t* code, uint32_t* sc_out,
                                                  float* s_out) {
  constexpr int NW = CPL / 8;
  uint32_t sc;
  float s;
  bool ok;
  if constexpr (MX) {
    // floor(log2 m) - 2 clamped to [-127, 127]: exponent field - 129
    const int ef = (int)(__float_as_uint(m) >> 23);
    const int e = max(ef - 129, -127);
    sc = (uint32_t)(e + 127);
    s = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : 0x1p-127f;
    ok = true;
  } else {
    const uint32_t ab = __float_as_uint(m);
    const int ea = (int)(ab >> 23);
    const uint32_t ent = tab[(ab >> 16) & 127u];
    const int e = ea - 127 - eDp + (int)(ent >> 3) - 1;
    const int ci = ((e + 7) << 3) | (int)(ent & 7u);
    sc = (uint32_t)min(ci, 126);
    ok = (ea != 0 && e >= -6) || ab == 0;
    sc = ab == 0 ? 0u : sc;
    s = sc >= 8u ? __uint_as_float((((sc >> 3) + 120u) << 23) | ((sc & 7u) << 20)) : 0.0f;
  }
  const float S = s * st;
  // (an all-zero block, m = 0, encodes exactly here whatever its scale: its
  // codes are the signed zeros x * 0)
  ok = ok && (S >= 0x1p-60f || S == 0.0f || m == 0.0f);
  const float rinv = (S > 0.0f && m != 0.0f) ? __builtin_amdgcn_rcpf(S) : 0.0f;
  const float rlo = rinv * (1.0f - 0x1p-20f), rhi = rinv * (1.0f + 0x1p-20f);
  // codes of x * rhi; where the tie mode needs them, also of x * rlo (the
  // two differ only at elements within 2^-20 of a midpoint)
  const float r1 = tie_mode == kTieDown ? rlo : rhi;
  uint32_t diff[NW];
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    uint32_t c = 0;
    const float* xq = xf + 8 * q;
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, xq[0] * r1, xq[1] * r1, 1.0f, 0);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, xq[2] * r1, xq[3] * r1, 1.0f, 1);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, xq[4] * r1, xq[5] * r1, 1.0f, 2);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, xq[6] * r1, xq[7] * r1, 1.0f, 3);
    code[q] = c;
    diff[q] = 0;
  }
  if (tie_mode >= kTieEven) {
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      uint32_t lo = 0;
      const float* xq = xf + 8 * q;
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xq[0] * rlo, xq[1] * rlo, 1.0f, 0);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xq[2] * rlo, xq[3] * rlo, 1.0f, 1);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xq[4] * rlo, xq[5] * rlo, 1.0f, 2);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xq[6] * rlo, xq[7] * rlo, 1.0f, 3);
      if (tie_mode == kTieEven) {
        // the two candidates of a tie are neighbouring magnitudes: keep the
        // nibble whose magnitude is even (lo where lo's low bit is clear)
        const uint32_t keep_lo = ((~lo) & 0x11111111u) * 15u;
        code[q] = (lo & keep_lo) | (code[q] & ~keep_lo);
      } else {
        diff[q] = lo ^ code[q];
        code[q] = lo;
      }
    }
  }
  if (__builtin_expect(!ok, 0)) {
    // a block scale outside the table's range or an extreme scale:
    // decide the scale and every code exactly (rare; CALL_EXACT keeps its
    // code and registers out of the caller)
    const uint2 c = CALL_EXACT
                        ? nvfp4_lane_exact_call<MX, CPL>(w[0], w[NW - 1], m, st, inv6st, st6, &sc, &s)
                        : nvfp4_lane_exact<MX, CPL>(w[0], w[NW - 1], m, st, inv6st, st6, &sc, &s);
    code[0] = c.x;
    diff[0] = 0;
    if constexpr (NW == 2) {
      code[NW - 1] = c.y;
      diff[NW - 1] = 0;
    }
  }
  // near-ties under a supplied s_t: one element per lane per round
  if (tie_mode == kTieExact) {
    uint32_t dany = diff[0];
#pragma unroll
    for (int q = 1; q < NW; ++q) dany |= diff[q];
    while (__builtin_expect(__any(dany != 0u), 0)) {
      if (dany != 0u) {
        int q = 0;
        if constexpr (NW == 2) q = diff[0] != 0u ? 0 : 1;
        const uint32_t dq = NW == 2 ? (q ? diff[1] : diff[0]) : diff[0];
        const uint32_t wq = NW == 2 ? (q ? code[1] : code[0]) : code[0];
        const int nib = (int)(__builtin_ctz(dq) >> 2);
        const uint32_t sh = 4u * (uint32_t)nib;
        const uint32_t ml = (wq >> sh) & 7u, mh = ((wq ^ dq) >> sh) & 7u;
        const uint32_t mlow = ml < mh ? ml : mh;
        // |x| against the midpoint t = (mid s) s_t, exactly in fp32: t = p + e
        // with p = RN(ms s_t) and e = its rounding error (exact: ms has at
        // most 9 significant bits and no product here is subnormal), and
        // |x| - p is exact (|x| lies within a factor 1 +- 2^-19 of t)
        const float ax = fabsf(lane_x<CPL>(w[0], w[NW - 1], 8 * q + nib));
        const float ms = e2m1_mid_above(mlow) * s;
        const float pt = ms * st, et = fmaf(ms, st, -pt);
        const float dt = ax - pt;
        const bool up = dt > et || (dt == et && ((mlow + 1u) & 1u) == 0u);
        const uint32_t nw = (wq & ~(7u << sh)) | ((up ? mlow + 1u : mlow) << sh);
        const uint32_t nd = dq & ~(15u << sh);
        if constexpr (NW == 2) {
          if (q) { code[1] = nw; diff[1] = nd; } else { code[0] = nw; diff[0] = nd; }
        } else {
          code[0] = nw;
          diff[0] = nd;
        }
        dany = diff[0];
#pragma unroll
        for (int q2 = 1; q2 < NW; ++q2) dany |= diff[q2];
      }
    }
  }
  *sc_out = sc;
  *s_out = s;
}

}  // namespace q4
