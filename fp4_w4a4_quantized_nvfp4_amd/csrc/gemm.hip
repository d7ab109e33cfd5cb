// W4A4 NVFP4 GEMM with fused Residual Activation Compensation (gfx950).
//
// QUADS (arXiv 2607.15810) section 3.3: the main product stays a W4A4 GEMM on
// the FP4 operands (remark after Eq. 22) and the compensation adds the
// residual of the selected channels (Eq. 21) on top.
//
// gfx950 has no matrix instruction that consumes an E4M3 scale per sixteen
// elements, but c * sb (an E2M1 value times an E4M3 scale) has at most six
// significant bits and lies in [2^-10, 2688], so it is exact in fp16.  FP4
// codes and scales are staged through LDS as bytes; each wave decodes its own
// MFMA fragments to fp16 with the gfx950 FP4 conversion, multiplies by the
// block scale (exact) and feeds v_mfma_f32_32x32x16_f16 (fp32 accumulate).
// After the K loop the accumulator is scaled by s_A * s_W and the residual
// operands (bf16 R [rows][kp], bf16 W_S [N][kp]) run as kp/16 extra
// v_mfma_f32_32x32x16_bf16 steps into the same accumulator tile.
//
// Tiles: 256 x 128 per workgroup of four waves (2 x 2), 128 x 64 per wave
// (4 x 2 MFMA 32x32 tiles), K chunks of 128 double-buffered in LDS.
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 128;
constexpr int CB = BK / 2;                            // code bytes per row per chunk
constexpr int NBLK = BK / 16;                         // scale blocks per row per chunk
constexpr int B_CODE_OFF = BM * CB;                   // 16384
constexpr int A_SC_OFF = B_CODE_OFF + BN * CB;        // 24576
constexpr int B_SC_OFF = A_SC_OFF + BM * NBLK * 2;    // 28672 (fp16 scales)
constexpr int STAGE = B_SC_OFF + BN * NBLK * 2;       // 30720

// 16-byte piece p of row r, xor-swizzled so that 16 consecutive rows reading
// the same piece hit distinct bank groups
__device__ __forceinline__ int swz(int row, int piece) {
  return row * CB + ((piece ^ ((row >> 2) & 3)) << 4);
}

// E4M3 code -> fp16 bits (exact: 4 significant bits, 2^-9 .. 448)
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t c) {
  const uint32_t m = c & 7u;
  const uint32_t sub =
      m ? ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)m) - 0x2400u) : 0u;
  return c >= 8u ? (c << 7) + 0x2000u : sub;
}

__device__ __forceinline__ uint32_t dup_lo(uint32_t d) { return (d & 0xffffu) | (d << 16); }
__device__ __forceinline__ uint32_t dup_hi(uint32_t d) { return (d >> 16) | (d & 0xffff0000u); }

// eight FP4 codes (one dword) -> eight fp16 values c * sb
__device__ __forceinline__ half8v decode8(uint32_t w, uint32_t pair) {
  const half2v s = __builtin_bit_cast(half2v, pair);
  const half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  half8v r;
  r[0] = h0.x; r[1] = h0.y; r[2] = h1.x; r[3] = h1.y;
  r[4] = h2.x; r[5] = h2.y; r[6] = h3.x; r[7] = h3.y;
  return r;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <bool FULLK, bool GROUPED, int EPI, bool MX>
__global__ __launch_bounds__(256, 2) void gemm_nvfp4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int K = g.K;
  const int64_t N = g.N;

  // ------------------------------------------------------------ tile
  int64_t m0, m_end, n0;
  int e = 0;
  if constexpr (GROUPED) {
    const int nbn = (int)((N + BN - 1) / BN);
    const int mt = blockIdx.x / nbn, nt = blockIdx.x % nbn;
    if (mt >= g.ntiles_dev[0]) return;
    const int4 t = ((const int4*)g.tiles)[mt];
    e = t.x;
    m0 = t.y;
    m_end = t.z;
    n0 = (int64_t)nt * BN;
  } else {
    const int nbm = (int)((g.M + BM - 1) / BM), nbn = (int)((N + BN - 1) / BN);
    const int nb = nbm * nbn;
    int b = blockIdx.x;
    // consecutive workgroups land on different XCDs; give each XCD a
    // contiguous range of tiles so that neighbouring tiles share its L2
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    // groups of 8 M tiles, M fastest inside a group
    const int GM = 8;
    const int group = b / (GM * nbn);
    const int first = group * GM;
    const int gsz = min(nbm - first, GM);
    const int in = b - group * GM * nbn;
    const int bm = first + in % gsz, bn = in / gsz;
    m0 = (int64_t)bm * BM;
    m_end = g.M;
    n0 = (int64_t)bn * BN;
  }

  const int64_t cstride = K / 2, sstride = MX ? K / 32 : K / 16;
  const uint8_t* wc = g.w_codes + (int64_t)e * N * cstride;
  const uint8_t* ws = g.w_scales + (int64_t)e * N * sstride;

  // ------------------------------------------------------------ staging rows
  const uint8_t* a_ptr[4];
  bool a_ok[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (it * 256 + tid) >> 2;
    const int64_t rr = m0 + r;
    a_ok[it] = rr < m_end;
    const int64_t ar = a_ok[it] ? (g.a_rows ? (int64_t)g.a_rows[rr] : rr) : 0;
    a_ptr[it] = g.a_codes + ar * cstride + ((it * 256 + tid) & 3) * 16;
  }
  const uint8_t* b_ptr[2];
  bool b_ok[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = (it * 256 + tid) >> 2;
    b_ok[it] = n0 + r < N;
    b_ptr[it] = wc + (b_ok[it] ? (n0 + r) : 0) * cstride + ((it * 256 + tid) & 3) * 16;
  }
  const uint8_t* as_ptr;
  bool as_ok;
  {
    const int64_t rr = m0 + tid;
    as_ok = rr < m_end;
    const int64_t ar = as_ok ? (g.a_rows ? (int64_t)g.a_rows[rr] : rr) : 0;
    as_ptr = g.a_scales + ar * sstride;
  }
  const bool bs_ok = tid < BN && n0 + tid < N;
  const uint8_t* bs_ptr = ws + (bs_ok ? n0 + tid : 0) * sstride;

  uint4 pa[4], pb[2];
  uint2 psa, psb;

  auto load = [&](int kc) {
    const int k0 = kc * BK;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int kel = k0 + 32 * ((it * 256 + tid) & 3);
      pa[it] = (a_ok[it] && (FULLK || kel < K)) ? *(const uint4*)(a_ptr[it] + k0 / 2)
                                                : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int kel = k0 + 32 * ((it * 256 + tid) & 3);
      pb[it] = (b_ok[it] && (FULLK || kel < K)) ? *(const uint4*)(b_ptr[it] + k0 / 2)
                                                : make_uint4(0, 0, 0, 0);
    }
    if constexpr (MX) {
      // E8M0 scales: one byte per 32 elements, four per row per chunk
      if constexpr (FULLK) {
        psa.x = as_ok ? *(const uint32_t*)(as_ptr + k0 / 32) : 0u;
        psb.x = bs_ok ? *(const uint32_t*)(bs_ptr + k0 / 32) : 0u;
      } else {
        uint32_t s = 0, t = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (k0 + 32 * q < K) {
            if (as_ok) s |= (uint32_t)as_ptr[k0 / 32 + q] << (8 * q);
            if (bs_ok) t |= (uint32_t)bs_ptr[k0 / 32 + q] << (8 * q);
          }
        }
        psa.x = s;
        psb.x = t;
      }
      psa.y = psb.y = 0u;
    } else if constexpr (FULLK) {
      psa = as_ok ? *(const uint2*)(as_ptr + k0 / 16) : make_uint2(0, 0);
      psb = bs_ok ? *(const uint2*)(bs_ptr + k0 / 16) : make_uint2(0, 0);
    } else {
      // scale rows are only 2-byte aligned when K % 128 != 0
      uint32_t s[4] = {0, 0, 0, 0}, t[4] = {0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (k0 + 32 * q < K) {
          if (as_ok) s[q] = *(const uint16_t*)(as_ptr + k0 / 16 + 2 * q);
          if (bs_ok) t[q] = *(const uint16_t*)(bs_ptr + k0 / 16 + 2 * q);
        }
      }
      psa = make_uint2(s[0] | (s[1] << 16), s[2] | (s[3] << 16));
      psb = make_uint2(t[0] | (t[1] << 16), t[2] | (t[3] << 16));
    }
  };

  auto store = [&](int stg) {
    uint8_t* base = smem + stg * STAGE;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = it * 256 + tid;
      *(uint4*)(base + swz(q >> 2, q & 3)) = pa[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = it * 256 + tid;
      *(uint4*)(base + B_CODE_OFF + swz(q >> 2, q & 3)) = pb[it];
    }
    if constexpr (MX) {
      *(uint32_t*)(base + A_SC_OFF + tid * 4) = psa.x;
      if (tid < BN) *(uint32_t*)(base + B_SC_OFF + tid * 4) = psb.x;
    } else {
      {
        const uint32_t w0 = psa.x, w1 = psa.y;
        uint4 f;
        f.x = e4m3_to_f16_bits(w0 & 255u) | (e4m3_to_f16_bits((w0 >> 8) & 255u) << 16);
        f.y = e4m3_to_f16_bits((w0 >> 16) & 255u) | (e4m3_to_f16_bits(w0 >> 24) << 16);
        f.z = e4m3_to_f16_bits(w1 & 255u) | (e4m3_to_f16_bits((w1 >> 8) & 255u) << 16);
        f.w = e4m3_to_f16_bits((w1 >> 16) & 255u) | (e4m3_to_f16_bits(w1 >> 24) << 16);
        *(uint4*)(base + A_SC_OFF + tid * 16) = f;
      }
      if (tid < BN) {
        const uint32_t w0 = psb.x, w1 = psb.y;
        uint4 f;
        f.x = e4m3_to_f16_bits(w0 & 255u) | (e4m3_to_f16_bits((w0 >> 8) & 255u) << 16);
        f.y = e4m3_to_f16_bits((w0 >> 16) & 255u) | (e4m3_to_f16_bits(w0 >> 24) << 16);
        f.z = e4m3_to_f16_bits(w1 & 255u) | (e4m3_to_f16_bits((w1 >> 8) & 255u) << 16);
        f.w = e4m3_to_f16_bits((w1 >> 16) & 255u) | (e4m3_to_f16_bits(w1 >> 24) << 16);
        *(uint4*)(base + B_SC_OFF + tid * 16) = f;
      }
    }
  };

  f32x16v acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  auto compute = [&](int stg) {
    const uint8_t* base = smem + stg * STAGE;
    if constexpr (MX) {
      // the scaled FP4 instruction consumes codes and E8M0 scales directly:
      // lane half h supplies the 32-element block 2j + h of the chunk
      uint32_t sa[4], sb[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        sa[mi] = *(const uint32_t*)(base + A_SC_OFF + (wm * 128 + mi * 32 + l32) * 4);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        sb[ni] = *(const uint32_t*)(base + B_SC_OFF + (wn * 64 + ni * 32 + l32) * 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = 2 * j + h;
        i32x8v af[4], bf[2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const uint4 v = *(const uint4*)(base + swz(wm * 128 + mi * 32 + l32, p));
          af[mi] = (i32x8v){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const uint4 v = *(const uint4*)(base + B_CODE_OFF + swz(wn * 64 + ni * 32 + l32, p));
          bf[ni] = (i32x8v){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[mi], bf[ni], acc[mi][ni], 4, 4, 0, (int)(sa[mi] >> (8 * p)), 0,
                (int)(sb[ni] >> (8 * p)));
      }
      return;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int p = 2 * h + s2;
      uint4 ra[4], rb[2];
      uint32_t sa[4], sb[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 128 + mi * 32 + l32;
        ra[mi] = *(const uint4*)(base + swz(row, p));
        sa[mi] = *(const uint32_t*)(base + A_SC_OFF + row * 16 + h * 8 + s2 * 4);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + l32;
        rb[ni] = *(const uint4*)(base + B_CODE_OFF + swz(row, p));
        sb[ni] = *(const uint32_t*)(base + B_SC_OFF + row * 16 + h * 8 + s2 * 4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8v af[4], bf[2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = decode8(word(ra[mi], j), j < 2 ? dup_lo(sa[mi]) : dup_hi(sa[mi]));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bf[ni] = decode8(word(rb[ni], j), j < 2 ? dup_lo(sb[ni]) : dup_hi(sb[ni]));
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
      }
    }
  };

  const int nk = (K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    if (kc + 1 < nk) load(kc + 1);
    compute(kc & 1);
    if (kc + 1 < nk) store((kc + 1) & 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ tensor scales
  const float alpha = g.a_ts ? g.a_ts[0] * g.w_ts[e] : 1.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= alpha;

  // ------------------------------------------------------------ residual tail
  if (g.kp > 0 && g.r_res) {
    const uint16_t* wsel = g.w_sel + (int64_t)e * N * g.kp;
    const uint16_t* rrow[4];
    bool rok[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int64_t rr = m0 + wm * 128 + mi * 32 + l32;
      rok[mi] = rr < m_end;
      const int64_t ar = rok[mi] ? (g.a_rows ? (int64_t)g.a_rows[rr] : rr) : 0;
      rrow[mi] = g.r_res + ar * g.ld_r + 8 * h;
    }
    const uint16_t* wrow[2];
    bool wok[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int64_t cc = n0 + wn * 64 + ni * 32 + l32;
      wok[ni] = cc < N;
      wrow[ni] = wsel + (wok[ni] ? cc : 0) * g.kp + 8 * h;
    }
    for (int kt = 0; kt < g.kp; kt += 16) {
      bf16x8v af[4], bf[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const uint4 v = rok[mi] ? *(const uint4*)(rrow[mi] + kt) : make_uint4(0, 0, 0, 0);
        af[mi] = __builtin_bit_cast(bf16x8v, v);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const uint4 v = wok[ni] ? *(const uint4*)(wrow[ni] + kt) : make_uint4(0, 0, 0, 0);
        bf[ni] = __builtin_bit_cast(bf16x8v, v);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // ------------------------------------------------------------ epilogue
  // accumulator element r of lane l: row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= m_end) continue;
      if constexpr (EPI == kEpiSwiGLU) {
        const int64_t f = (n0 + wn * 64) / 2 + l32;
        if (n0 + wn * 64 + 32 + l32 < N) {
          const float gv = acc[mi][0][r], uv = acc[mi][1][r];
          ((uint16_t*)g.Y)[row * g.ldy + f] = (uint16_t)f32_to_bf16_rne(silu(gv) * uv);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int64_t col = n0 + wn * 64 + ni * 32 + l32;
          if (col >= N) continue;
          const float v = acc[mi][ni][r];
          if (g.y_bf16)
            ((uint16_t*)g.Y)[row * g.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            ((float*)g.Y)[row * g.ldy + col] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dense kernel with 256 x 256 tiles: four waves of 128 x 128 (4 x 4 MFMA
// tiles, accumulators in AGPRs, one wave per SIMD).  Every decoded fragment
// feeds four MFMAs, so decode costs four VALU instructions per MFMA.
namespace big {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int CB = BK / 2;
constexpr int B_CODE_OFF = BM * CB;                 // 16384
constexpr int A_SC_OFF = B_CODE_OFF + BN * CB;      // 32768
constexpr int B_SC_OFF = A_SC_OFF + BM * 16;        // 36864 (fp16 scales, 8 per row)
constexpr int STAGE = B_SC_OFF + BN * 16;           // 40960

__device__ __forceinline__ int swzb(int row, int piece) {
  return row * CB + ((piece ^ ((row >> 2) & 3)) << 4);
}

// four E4M3 bytes -> two dwords of fp16 pairs (exact)
__device__ __forceinline__ uint2 e4m3x4_to_f16(uint32_t w) {
  const uint32_t t = w & 0x78787878u;
  const bool any_sub = ((t - 0x01010101u) & ~t & 0x80808080u) != 0u;   // some exponent field 0
  uint2 r;
  if (!any_sub) {
    const uint32_t lo2 = __builtin_amdgcn_perm(0u, w, 0x0c010c00u);     // b0 | b1 << 16
    const uint32_t hi2 = __builtin_amdgcn_perm(0u, w, 0x0c030c02u);     // b2 | b3 << 16
    r.x = (lo2 << 7) + 0x20002000u;
    r.y = (hi2 << 7) + 0x20002000u;
  } else {
    r.x = e4m3_to_f16_bits(w & 255u) | (e4m3_to_f16_bits((w >> 8) & 255u) << 16);
    r.y = e4m3_to_f16_bits((w >> 16) & 255u) | (e4m3_to_f16_bits(w >> 24) << 16);
  }
  return r;
}

template <bool FULLK>
__global__ __launch_bounds__(256, 1) void gemm_nvfp4_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int K = g.K;
  const int64_t N = g.N;

  const int nbm = (int)((g.M + BM - 1) / BM), nbn = (int)((N + BN - 1) / BN);
  const int nb = nbm * nbn;
  int b = blockIdx.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);   // contiguous tile range per XCD
  const int GM = 4;
  const int group = b / (GM * nbn);
  const int first = group * GM;
  const int gsz = min(nbm - first, GM);
  const int in = b - group * GM * nbn;
  const int64_t m0 = (int64_t)(first + in % gsz) * BM;
  const int64_t n0 = (int64_t)(in / gsz) * BN;
  const int64_t m_end = g.M;

  const uint32_t cstride = (uint32_t)(K / 2), sstride = (uint32_t)(K / 16);
  // 32-bit offsets from the (uniform) operand bases keep the staging state small
  const uint8_t* const a_base = g.a_codes + (size_t)m0 * cstride;
  const uint8_t* const b_base = g.w_codes + (size_t)n0 * cstride;
  uint32_t a_off[4], b_off[4];
  uint32_t ab_ok = 0;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int q = it * 256 + tid;
    const int r = q >> 2;
    const bool aok = m0 + r < m_end, bok = n0 + r < N;
    ab_ok |= (aok ? 1u : 0u) << it;
    ab_ok |= (bok ? 1u : 0u) << (4 + it);
    a_off[it] = (aok ? (uint32_t)r : 0u) * cstride + (uint32_t)(q & 3) * 16u;
    b_off[it] = (bok ? (uint32_t)r : 0u) * cstride + (uint32_t)(q & 3) * 16u;
  }
  const bool as_ok = m0 + tid < m_end, bs_ok = n0 + tid < N;
  const uint8_t* const as_base = g.a_scales + (size_t)m0 * sstride;
  const uint8_t* const bs_base = g.w_scales + (size_t)n0 * sstride;
  const uint32_t as_off = (as_ok ? (uint32_t)tid : 0u) * sstride;
  const uint32_t bs_off = (bs_ok ? (uint32_t)tid : 0u) * sstride;

  uint4 pa[4], pb[4];
  uint2 psa, psb;
  auto load = [&](int kc) {
    const int k0 = kc * BK;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int kel = k0 + 32 * ((it * 256 + tid) & 3);
      pa[it] = (((ab_ok >> it) & 1u) && (FULLK || kel < K))
                   ? *(const uint4*)(a_base + a_off[it] + k0 / 2) : make_uint4(0, 0, 0, 0);
      pb[it] = (((ab_ok >> (4 + it)) & 1u) && (FULLK || kel < K))
                   ? *(const uint4*)(b_base + b_off[it] + k0 / 2) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (FULLK) {
      psa = as_ok ? *(const uint2*)(as_base + as_off + k0 / 16) : make_uint2(0, 0);
      psb = bs_ok ? *(const uint2*)(bs_base + bs_off + k0 / 16) : make_uint2(0, 0);
    } else {
      uint32_t sa4[4] = {0, 0, 0, 0}, sb4[4] = {0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (k0 + 32 * q < K) {
          if (as_ok) sa4[q] = *(const uint16_t*)(as_base + as_off + k0 / 16 + 2 * q);
          if (bs_ok) sb4[q] = *(const uint16_t*)(bs_base + bs_off + k0 / 16 + 2 * q);
        }
      }
      psa = make_uint2(sa4[0] | (sa4[1] << 16), sa4[2] | (sa4[3] << 16));
      psb = make_uint2(sb4[0] | (sb4[1] << 16), sb4[2] | (sb4[3] << 16));
    }
  };
  auto store = [&](int stg) {
    uint8_t* base = smem + stg * STAGE;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = it * 256 + tid;
      *(uint4*)(base + swzb(q >> 2, q & 3)) = pa[it];
      *(uint4*)(base + B_CODE_OFF + swzb(q >> 2, q & 3)) = pb[it];
    }
    const uint2 a0 = e4m3x4_to_f16(psa.x), a1 = e4m3x4_to_f16(psa.y);
    const uint2 b0 = e4m3x4_to_f16(psb.x), b1 = e4m3x4_to_f16(psb.y);
    *(uint4*)(base + A_SC_OFF + tid * 16) = make_uint4(a0.x, a0.y, a1.x, a1.y);
    *(uint4*)(base + B_SC_OFF + tid * 16) = make_uint4(b0.x, b0.y, b1.x, b1.y);
  };

  f32x16v acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  auto compute = [&](int stg) {
    const uint8_t* base = smem + stg * STAGE;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int p = 2 * h + s2;
      uint4 ra[4], rb[4];
      uint32_t sa[4], sb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 128 + mi * 32 + l32;
        ra[mi] = *(const uint4*)(base + swzb(row, p));
        sa[mi] = *(const uint32_t*)(base + A_SC_OFF + row * 16 + h * 8 + s2 * 4);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = wn * 128 + ni * 32 + l32;
        rb[ni] = *(const uint4*)(base + B_CODE_OFF + swzb(row, p));
        sb[ni] = *(const uint32_t*)(base + B_SC_OFF + row * 16 + h * 8 + s2 * 4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8v af[4], bf[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = decode8(word(ra[mi], j), j < 2 ? dup_lo(sa[mi]) : dup_hi(sa[mi]));
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          bf[ni] = decode8(word(rb[ni], j), j < 2 ? dup_lo(sb[ni]) : dup_hi(sb[ni]));
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
      }
    }
  };

  const int nk = (K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    if (kc + 1 < nk) load(kc + 1);
    compute(kc & 1);
    if (kc + 1 < nk) store((kc + 1) & 1);
    __syncthreads();
  }

  const float alpha = g.a_ts ? g.a_ts[0] * g.w_ts[0] : 1.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= alpha;

  if (g.kp > 0 && g.r_res) {
    const uint16_t* rrow[4];
    const uint16_t* wrow[4];
    bool rok[4], wok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t rr = m0 + wm * 128 + q * 32 + l32;
      rok[q] = rr < m_end;
      rrow[q] = g.r_res + (rok[q] ? rr : 0) * g.ld_r + 8 * h;
      const int64_t cc = n0 + wn * 128 + q * 32 + l32;
      wok[q] = cc < N;
      wrow[q] = g.w_sel + (wok[q] ? cc : 0) * g.kp + 8 * h;
    }
    for (int kt = 0; kt < g.kp; kt += 16) {
      bf16x8v af[4], bf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        af[q] = __builtin_bit_cast(bf16x8v, rok[q] ? *(const uint4*)(rrow[q] + kt) : make_uint4(0, 0, 0, 0));
        bf[q] = __builtin_bit_cast(bf16x8v, wok[q] ? *(const uint4*)(wrow[q] + kt) : make_uint4(0, 0, 0, 0));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= m_end) continue;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t col = n0 + wn * 128 + ni * 32 + l32;
        if (col >= N) continue;
        const float v = acc[mi][ni][r];
        if (g.y_bf16)
          ((uint16_t*)g.Y)[row * g.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
        else
          ((float*)g.Y)[row * g.ldy + col] = v;
      }
    }
  }
}
}  // namespace big

template <bool FULLK, bool GROUPED, bool MX>
hipError_t launch_t(const GemmArgs& g, int64_t max_mtiles, hipStream_t stream) {
  const int64_t nbn = (g.N + BN - 1) / BN;
  const int64_t nbm = GROUPED ? max_mtiles : (g.M + BM - 1) / BM;
  const int64_t nb = nbm * nbn;
  if (nb == 0) return hipSuccess;
  if (g.epilogue == kEpiSwiGLU)
    hipLaunchKernelGGL((gemm_nvfp4_kernel<FULLK, GROUPED, kEpiSwiGLU, MX>), dim3((unsigned)nb),
                       dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_nvfp4_kernel<FULLK, GROUPED, kEpiStore, MX>), dim3((unsigned)nb),
                       dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a4_gemm(const GemmArgs& g, int64_t max_mtiles, hipStream_t stream) {
  const bool fullk = (g.K % BK) == 0;
  const bool grouped = g.tiles != nullptr;
  if (g.mx) {
    if (fullk)
      return grouped ? launch_t<true, true, true>(g, max_mtiles, stream)
                     : launch_t<true, false, true>(g, max_mtiles, stream);
    return grouped ? launch_t<false, true, true>(g, max_mtiles, stream)
                   : launch_t<false, false, true>(g, max_mtiles, stream);
  }
  if (!grouped && g.epilogue == kEpiStore && g.M >= 512 && g.N >= 512) {
    const int64_t nb = ((g.M + big::BM - 1) / big::BM) * ((g.N + big::BN - 1) / big::BN);
    if (fullk)
      hipLaunchKernelGGL(big::gemm_nvfp4_big_kernel<true>, dim3((unsigned)nb), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL(big::gemm_nvfp4_big_kernel<false>, dim3((unsigned)nb), dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (fullk)
    return grouped ? launch_t<true, true, false>(g, max_mtiles, stream)
                   : launch_t<true, false, false>(g, max_mtiles, stream);
  return grouped ? launch_t<false, true, false>(g, max_mtiles, stream)
                 : launch_t<false, false, false>(g, max_mtiles, stream);
}

}  // namespace q4
