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
#include <algorithm>
#include <type_traits>

#include "q4_internal.h"
#include "q4_nvfp4_enc.h"
#include "q4_prep.h"

namespace q4 {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 128;
constexpr int CB = BK / 2;                            // code bytes per row per chunk
constexpr int NBLK = BK / 16;                         // scale blocks per row per chunk
constexpr int B_CODE_OFF = BM * CB;                   // 16384
constexpr int A_SC_OFF = B_CODE_OFF + BN * CB;        // 24576
constexpr int B_SC_OFF = A_SC_OFF + BM * NBLK * 2;    // 28672 (fp16 scales)
constexpr int STAGE = B_SC_OFF + BN * NBLK * 2;       // 30720

// 16-byte piece p of row r (rows of 64 bytes), xor-swizzled so that 8 (or 16)
// consecutive rows reading the same piece hit distinct 16-byte bank groups
// whether the LDS serves 128 or 256 bytes per cycle
__device__ __forceinline__ int swz(int row, int piece) {
  return row * CB + ((piece ^ ((row >> 1) ^ (row >> 2)) & 3) << 4);
}

// dword d of a 16-byte per-row scale record, xor-swizzled so that 32
// consecutive rows reading the same dword hit distinct banks
__device__ __forceinline__ int swz_sc(int row, int d) {
  return row * 16 + ((d ^ ((row >> 3) & 3)) << 2);
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
        *(uint4*)(base + A_SC_OFF + tid * 16) = swz_sc_rec(f, tid);
      }
      if (tid < BN) {
        const uint32_t w0 = psb.x, w1 = psb.y;
        uint4 f;
        f.x = e4m3_to_f16_bits(w0 & 255u) | (e4m3_to_f16_bits((w0 >> 8) & 255u) << 16);
        f.y = e4m3_to_f16_bits((w0 >> 16) & 255u) | (e4m3_to_f16_bits(w0 >> 24) << 16);
        f.z = e4m3_to_f16_bits(w1 & 255u) | (e4m3_to_f16_bits((w1 >> 8) & 255u) << 16);
        f.w = e4m3_to_f16_bits((w1 >> 16) & 255u) | (e4m3_to_f16_bits(w1 >> 24) << 16);
        *(uint4*)(base + B_SC_OFF + tid * 16) = swz_sc_rec(f, tid);
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
        sa[mi] = *(const uint32_t*)(base + A_SC_OFF + swz_sc(row, 2 * h + s2));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + l32;
        rb[ni] = *(const uint4*)(base + B_CODE_OFF + swz(row, p));
        sb[ni] = *(const uint32_t*)(base + B_SC_OFF + swz_sc(row, 2 * h + s2));
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
  // With a scaled compensation term (beta = -s_R s_W) the W4A4 sum is taken
  // to alpha / beta = -s_A / s_R, the term added, and the sum scaled by beta.
  // (s_A s_W is applied without underflow: out_scale).  NVFP4 compensation
  // operands are fp16; without their own scale they come in the sum's units
  // and add to the unscaled sum before that multiply.  MXFP4 (no tensor
  // scale): bf16 operands.
  const bool rac = g.kp > 0 && g.r_res;
  const bool rscaled = rac && g.r_ts && g.a_ts;
  const bool units = rac && !rscaled && !MX;
  OutScale pre{1.0f, 0, false}, post{1.0f, 0, false};
  if (rscaled) {
    pre.mul = -(g.a_ts[0] / g.r_ts[0]);
    post = out_scale(g.r_ts[0], g.w_ts[e]);
    post.mul = -post.mul;
  } else if (g.a_ts) {
    (units ? post : pre) = out_scale(g.a_ts[0], g.w_ts[e]);
  }
  if (!units) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = apply_scale(pre, acc[mi][ni][r]);
  }

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
      uint4 av[4], bv[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        av[mi] = rok[mi] ? *(const uint4*)(rrow[mi] + kt) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bv[ni] = wok[ni] ? *(const uint4*)(wrow[ni] + kt) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          if constexpr (MX)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8v, av[mi]), __builtin_bit_cast(bf16x8v, bv[ni]),
                acc[mi][ni], 0, 0, 0);
          else
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(half8v, av[mi]), __builtin_bit_cast(half8v, bv[ni]),
                acc[mi][ni], 0, 0, 0);
        }
    }
  }
  if (rscaled || units) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = apply_scale(post, acc[mi][ni][r]);
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
// Dense kernel with 256 x 256 tiles for K % 128 == 0: four waves of 128 x 128
// (4 x 4 MFMA tiles, accumulators in AGPRs, one wave per SIMD).  Every decoded
// fragment feeds four MFMAs, so decode costs about four VALU instructions per
// MFMA.
//
// Pipeline: three LDS stages filled straight from global memory
// (global_load_lds, no registers), three chunks ahead: FP4 codes as 16-byte
// pieces, raw E4M3 scales as dwords.  Each wave widens its own scales to fp16
// when it reads a fragment.  Each chunk is consumed in two halves (s2): while
// the MFMAs of one half run, the fragments of the next half are read from
// LDS, and the decode of step j + 1 overlaps the MFMAs of step j.  One
// workgroup barrier per chunk sits between the two halves.
namespace big {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int CB = BK / 2;
constexpr int NST = 3;
constexpr int B_CODE_OFF = BM * CB;                 // 16384
constexpr int A_SC_OFF = B_CODE_OFF + BN * CB;      // 32768
// scale bytes per row per chunk: 8 raw E4M3, or 16 as tiled fp16 records
template <bool TILED> constexpr int SC_ROW = TILED ? 16 : 8;
template <bool TILED> constexpr int B_SC_OFF = A_SC_OFF + BM * SC_ROW<TILED>;
template <bool TILED> constexpr int STAGE = B_SC_OFF<TILED> + BN * SC_ROW<TILED>;
// global -> LDS loads per wave per chunk: 8 code pieces + 4 raw scale dwords,
// or + one 16-byte tiled scale record per operand
template <bool TILED> constexpr int DMA_PER_CHUNK = TILED ? 10 : 12;

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and leaves the other counters alone
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// byte `which` of an E4M3 pair -> that scale as fp16 in both halves (exact,
// subnormal scales included): the byte shifted left by 7 is an fp16 whose
// value is the E4M3 value times 2^-8, normal and subnormal alike, and the
// multiply by 256 is exact
__device__ __forceinline__ uint32_t e4m3_dup_f16(uint32_t pair, int which) {
  const half2v k256 = {(_Float16)256.0f, (_Float16)256.0f};
  const uint32_t d = __builtin_amdgcn_perm(0u, pair, which ? 0x0c010c01u : 0x0c000c00u) << 7;
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d) * k256);
}

struct Frag {
  uint4 a[4], b[4];
  uint32_t sa[4], sb[4];   // two raw E4M3 scales (blocks 2p, 2p + 1) per row
};

// RSC: the compensation term carries its own scale (g.r_ts); a separate
// instantiation so the plain kernels keep their register allocation
// MX: MXFP4 operands (E8M0 scale per 32 elements, no tensor scale) fed
// straight from LDS to the scaled FP4 instruction, no decode (dense only)
// WIDE: grouped 128 x 512 tiles (NVFP4, tiled records, store or SwiGLU
// epilogue) for experts whose row counts leave mostly empty 256-row tiles:
// every wave still owns a 128 x 128 block (all 128 rows, its own quarter of
// the columns), so the per-wave work and LDS reads are those of 256 x 256
template <bool TILED, bool GROUPED, int EPI, bool RSC = false, bool MX = false, bool WIDE = false>
__global__ __launch_bounds__(256, 1) void gemm_nvfp4_big_kernel(GemmArgs g) {
  static_assert(GROUPED || EPI == kEpiStore, "SwiGLU is a grouped epilogue");
  static_assert(EPI != kEpiSwiGLUQuant || !MX, "the quantizing epilogue writes NVFP4");
  static_assert(!MX || (!TILED && !RSC), "MXFP4: raw scales, no scaled compensation");
  static_assert(!WIDE || (TILED && GROUPED && !RSC && !MX && EPI != kEpiSwiGLUQuant),
                "128 x 512 tiles: grouped NVFP4 with scale records, store or SwiGLU epilogue");
  constexpr int TBM = WIDE ? 128 : BM, TBN = WIDE ? 512 : BN;
  // stage layout: A codes, B codes, A scales, B scales (MX: 4 E8M0 bytes per
  // row per chunk)
  constexpr int B_CODE_OFF = TBM * CB;
  constexpr int A_SC_OFF = (TBM + TBN) * CB;
  constexpr int B_SC_OFF = MX ? A_SC_OFF + BM * 4 : A_SC_OFF + TBM * SC_ROW<TILED>;
  constexpr int STAGE = WIDE ? B_SC_OFF + TBN * 16 : big::STAGE<TILED>;
  // WIDE: 2 + 8 code loads, one A record load (waves 2 and 3 repeat the
  // records of waves 0 and 1, byte for byte) and two B record loads
  constexpr int DMA_PER_CHUNK = MX ? 10 : (WIDE ? 13 : big::DMA_PER_CHUNK<TILED>);
  static_assert(3 * STAGE <= 160 * 1024, "three stages fit the LDS");
  // one LDS object per stage, addressed with compile-time stage indices, so
  // the compiler can tell that reads of one stage do not wait for the
  // global -> LDS loads still filling another
  __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t stage2[STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // the wave's 128 x 128 block: tile rows arow .. + 127, columns bcol .. + 127
  const int arow = WIDE ? 0 : wm * 128, bcol = WIDE ? wave * 128 : wn * 128;
  const int l32 = lane & 31, h = lane >> 5;
  const int K = g.K;
  const int64_t N = g.N;
  const int nk = K / BK;

  int64_t m0, n0, m_end;
  int ex = 0;   // expert (grouped)
  int mt = 0;   // M tile of the table (grouped)
  if constexpr (GROUPED) {
    // tiles of the table ({expert, first row, end row} per M tile), M tile
    // major; each XCD (workgroup index mod 8; the grid is a multiple of 8)
    // takes a contiguous range of the tiles that exist, so it works through
    // whole experts and their weights stay in its L2
    const int nbn = (int)((N + TBN - 1) / TBN);
    const int total = g.ntiles_dev[0] * nbn;
    const int per = (total + 7) >> 3;
    const int l = (int)(blockIdx.x >> 3), t = (int)(blockIdx.x & 7) * per + l;
    if (l >= per || t >= total) return;
    mt = t / nbn;
    const int4 tt = ((const int4*)g.tiles)[mt];
    ex = tt.x;
    m0 = tt.y;
    m_end = tt.z;
    n0 = (int64_t)(t - mt * nbn) * TBN;
  } else {
    const int nbm = (int)((g.M + BM - 1) / BM), nbn = (int)((N + BN - 1) / BN);
    const int nb = nbm * nbn;
    int b = blockIdx.x;
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);   // contiguous tile range per XCD
    const int GM = 4;
    const int group = b / (GM * nbn);
    const int first = group * GM;
    const int gsz = min(nbm - first, GM);
    const int in = b - group * GM * nbn;
    m0 = (int64_t)(first + in % gsz) * BM;
    n0 = (int64_t)(in / gsz) * BN;
    m_end = g.M;
  }
  const int64_t wrow0 = (int64_t)ex * N + n0;   // first W row of the tile

  // Global -> LDS loads go through buffer resources based at the tile's
  // first row, with the operand's extent from there as the range: rows past
  // the end of A or W read as zeros (their products land only in output rows
  // and columns that are never stored).  Every per-lane offset is the same
  // for all chunks and all load instructions of one operand; the chunk and
  // the instruction's row block go into the scalar offset.
  const uint32_t cstride = (uint32_t)(K / 2), sstride = (uint32_t)(MX ? K / 32 : K / 16);
  auto rsrc = [](const void* base, int64_t bytes) {
    // every input is uniform; readfirstlane says so, so that the resource
    // stays in scalar registers
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)n), 0x00020000);
  };
  // Grouped: A rows are addressed absolutely (gathered through a_rows when
  // given; rows past the tile's end repeat its last row, whose products
  // land only in rows that are never stored), from the whole A operand.
  const int64_t a_src_rows = g.a_src_rows > 0 ? g.a_src_rows : g.M;
  const __amdgpu_buffer_rsrc_t a_rs =
      GROUPED ? rsrc(g.a_codes, a_src_rows * cstride)
              : rsrc(g.a_codes + (size_t)m0 * cstride, (g.M - m0) * cstride);
  const __amdgpu_buffer_rsrc_t b_rs = rsrc(g.w_codes + (size_t)wrow0 * cstride, (N - n0) * cstride);
  auto a_src = [&](int r) {   // A row of tile row r
    const int64_t row = m0 + r < m_end ? m0 + r : m_end - 1;
    return g.a_rows ? (int64_t)g.a_rows[row] : row;
  };
  // code loads: instruction `it` of this wave fills the 1 KiB of LDS that
  // holds tile rows 16 * (4 * it + wave) .. + 15; lane l writes 16 bytes at
  // l * 16, i.e. row 16 * c + l / 4, swizzled slot l % 4, which holds the
  // logical 16-byte piece slot ^ f(row) (f sees row bits 1..3 only, which
  // `it` does not change)
  const int c_row = 16 * wave + (lane >> 2);
  const uint32_t c_piece = (uint32_t)(((lane & 3) ^ (((c_row >> 1) ^ (c_row >> 2)) & 3)) * 16);
  const uint32_t c_voff = (uint32_t)c_row * cstride + c_piece;
  uint32_t ga_voff[4] = {0, 0, 0, 0};   // grouped: A code offset of load `it` (< TBM / 64)
  if constexpr (GROUPED) {
#pragma unroll
    for (int it = 0; it < TBM / 64; ++it)
      ga_voff[it] = (uint32_t)a_src(16 * (4 * it + wave) + (lane >> 2)) * cstride + c_piece;
  }
  // raw scale loads: instruction `it` of this wave fills 256 bytes of LDS
  // (rows 32 * (4 * it + wave) .. + 31, 8 bytes each); lane l loads dword
  // l % 2 of row 32 * c + l / 2
  const __amdgpu_buffer_rsrc_t as_rs =
      GROUPED ? rsrc(g.a_scales, a_src_rows * sstride)
              : rsrc(g.a_scales + (size_t)m0 * sstride, (g.M - m0) * sstride);
  const __amdgpu_buffer_rsrc_t bs_rs = rsrc(g.w_scales + (size_t)wrow0 * sstride, (N - n0) * sstride);
  const uint32_t s_voff = (uint32_t)(32 * wave + (lane >> 1)) * sstride + (uint32_t)(lane & 1) * 4u;
  uint32_t gs_voff[2] = {0, 0};   // grouped: A scale offset of load `it`
  if constexpr (GROUPED) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
      gs_voff[it] = (uint32_t)a_src(32 * (4 * it + wave) + (lane >> 1)) * sstride + (uint32_t)(lane & 1) * 4u;
  }
  // tiled scale records [chunk][padded row][16 B]: lane l of the wave loads
  // the record of tile row 64 * wave + l.  Grouped: the A records follow the
  // sorted rows (each swizzled by its row's offset within its expert, which
  // is its LDS row, tiles starting at multiples of 256 rows into an expert),
  // and each expert's W records are a block of their own.
  const __amdgpu_buffer_rsrc_t ast_rs =
      rsrc(g.a_scales_t + ((size_t)m0 << 4), ((int64_t)nk * g.a_rows_pad - m0) << 4);
  const __amdgpu_buffer_rsrc_t bst_rs =
      rsrc(g.w_scales_t + (((size_t)ex * nk * g.w_rows_pad + n0) << 4),
           ((int64_t)nk * g.w_rows_pad - n0) << 4);
  const uint32_t t_voff = (uint32_t)(64 * wave + lane) << 4;
  const int ta_row = WIDE ? 64 * (wave & 1) : 64 * wave;   // first A record row of the wave
  const uint32_t ta_voff = (uint32_t)(ta_row + lane) << 4;

  // LDS read offsets within a stage of fragment q = 0 for half s2 (piece
  // p = 2 h + s2 holds scale blocks 2p and 2p + 1).  Both swizzles depend on
  // row bits 1..4 only, so fragment q sits at a fixed distance (q * 32 rows)
  // from fragment 0: one address register per operand and half, the rest
  // goes into the instruction's immediate offset.
  uint32_t ca_off[2], cb_off[2], sa_off[2], sb_off[2];
  {
    const int ra = arow + l32, rb = bcol + l32;
    ca_off[0] = (uint32_t)swz(ra, 2 * h);
    cb_off[0] = (uint32_t)(B_CODE_OFF + swz(rb, 2 * h));
    ca_off[1] = ca_off[0] ^ 16u;
    cb_off[1] = cb_off[0] ^ 16u;
    if constexpr (TILED) {
      sa_off[0] = (uint32_t)(A_SC_OFF + swz_sc(ra, 2 * h));
      sb_off[0] = (uint32_t)(B_SC_OFF + swz_sc(rb, 2 * h));
      sa_off[1] = sa_off[0] ^ 4u;
      sb_off[1] = sb_off[0] ^ 4u;
    } else {
      sa_off[0] = (uint32_t)(A_SC_OFF + ra * 8 + 4 * h);
      sb_off[0] = (uint32_t)(B_SC_OFF + rb * 8 + 4 * h);
      sa_off[1] = sa_off[0] + 2u;
      sb_off[1] = sb_off[0] + 2u;
    }
  }
  constexpr uint32_t Q_CODE = 32 * CB, Q_SC = 32 * SC_ROW<TILED>;

  // global -> LDS traffic of FP4 chunk kc (kc < nk): codes, then scales
  auto issue_codes = [&](int kc, uint8_t* const sbase) {
    const uint32_t kb = (uint32_t)kc * (BK / 2);
    uint8_t* const dst = sbase + wave * 1024;
#pragma unroll
    for (int it = 0; it < TBN / 64; ++it) {
      const uint32_t so = kb + (uint32_t)(64 * it) * cstride;
      if (it < TBM / 64) {
        if constexpr (GROUPED)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lptr_t)(dst + it * 4096), 16,
                                                   ga_voff[it < TBM / 64 ? it : 0], kb, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lptr_t)(dst + it * 4096), 16, c_voff, so, 0,
                                                   0);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rs, (lptr_t)(dst + B_CODE_OFF + it * 4096), 16,
                                               c_voff, so, 0, 0);
    }
  };
  // MX: lane l of the wave loads the chunk's four E8M0 bytes of tile row
  // 64 * wave + l (one dword per operand); grouped A rows through a_src
  const uint32_t mxs_voff = (uint32_t)(64 * wave + lane) * sstride;
  uint32_t mxa_voff = mxs_voff;
  if constexpr (MX && GROUPED) mxa_voff = (uint32_t)a_src(64 * wave + lane) * sstride;
  auto issue_scales = [&](int kc, uint8_t* const sbase) {
    if constexpr (MX) {
      const uint32_t ks = (uint32_t)kc * (BK / 32);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rs, (lptr_t)(sbase + A_SC_OFF + wave * 256), 4,
                                               mxa_voff, ks, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rs, (lptr_t)(sbase + B_SC_OFF + wave * 256), 4,
                                               mxs_voff, ks, 0, 0);
    } else if constexpr (TILED) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ast_rs, (lptr_t)(sbase + A_SC_OFF + ta_row * 16), 16,
                                               ta_voff, (uint32_t)(kc * g.a_rows_pad) << 4, 0, 0);
#pragma unroll
      for (int it = 0; it < TBN / 256; ++it)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            bst_rs, (lptr_t)(sbase + B_SC_OFF + wave * 1024 + it * 4096), 16, t_voff,
            ((uint32_t)(kc * g.w_rows_pad) << 4) + (uint32_t)it * 4096u, 0, 0);
    } else {
      const uint32_t ks = (uint32_t)kc * (BK / 16);
      uint8_t* const sdst = sbase + wave * 256;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const uint32_t so = ks + (uint32_t)(128 * it) * sstride;
        if constexpr (GROUPED)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rs, (lptr_t)(sdst + A_SC_OFF + it * 1024), 4,
                                                   gs_voff[it], ks, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rs, (lptr_t)(sdst + A_SC_OFF + it * 1024), 4,
                                                   s_voff, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rs, (lptr_t)(sdst + B_SC_OFF + it * 1024), 4,
                                                 s_voff, so, 0, 0);
      }
    }
  };
  // every chunk issue is DMA_PER_CHUNK loads per wave, whatever it carries
  auto issue_chunk = [&](int kc, uint8_t* const sbase) {   // FP4 chunk kc < nk
    issue_codes(kc, sbase);
    issue_scales(kc, sbase);
  };

  // Residual compensation chunks: R [M][ld_r] and W_S [N][kp] (bf16,
  // kp % 32 == 0) go through the same stages ahead of the FP4 chunks, 32
  // channels per chunk (64 bytes per row, the code chunks' layout), straight
  // into bf16 MFMAs.  Chunk j < nrac is RAC chunk j, chunk nrac + kc is FP4
  // chunk kc.
  const int nrac = (g.kp > 0 && g.r_res) ? g.kp / 32 : 0;
  const uint32_t r_stride = (uint32_t)g.ld_r * 2u, w_stride = (uint32_t)g.kp * 2u;
  // (grouped: R rows of the A source rows, W_S rows of the expert's)
  const __amdgpu_buffer_rsrc_t r_rs =
      GROUPED ? rsrc(g.r_res, nrac ? a_src_rows * (int64_t)r_stride : 0)
              : rsrc(g.r_res + (size_t)m0 * g.ld_r, nrac ? (g.M - m0) * (int64_t)r_stride : 0);
  const __amdgpu_buffer_rsrc_t w_rs =
      rsrc(g.w_sel + (size_t)wrow0 * g.kp, nrac ? (N - n0) * (int64_t)w_stride : 0);
  // same row / piece layout as the code loads, with the operands' own strides
  const uint32_t r_voff = (uint32_t)c_row * r_stride + c_piece;
  const uint32_t w_voff = (uint32_t)c_row * w_stride + c_piece;
  uint32_t gr_voff[4] = {0, 0, 0, 0};   // grouped: R offset of load `it` (< TBM / 64)
  if constexpr (GROUPED) {
    if (nrac > 0) {
#pragma unroll
      for (int it = 0; it < TBM / 64; ++it)
        gr_voff[it] = (uint32_t)a_src(16 * (4 * it + wave) + (lane >> 2)) * r_stride + c_piece;
    }
  }
  auto issue_rac = [&](int j, uint8_t* const sbase) {
#pragma unroll
    for (int it = 0; it < TBN / 64; ++it) {
      if (it < TBM / 64) {
        if constexpr (GROUPED)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_rs, (lptr_t)(sbase + wave * 1024 + it * 4096), 16,
                                                   gr_voff[it < TBM / 64 ? it : 0], 64u * (uint32_t)j,
                                                   0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              r_rs, (lptr_t)(sbase + wave * 1024 + it * 4096), 16, r_voff,
              64u * (uint32_t)j + (uint32_t)(64 * it) * r_stride, 0, 0);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rs, (lptr_t)(sbase + B_CODE_OFF + wave * 1024 + it * 4096), 16, w_voff,
          64u * (uint32_t)j + (uint32_t)(64 * it) * w_stride, 0, 0);
    }
  };
  // chunk c of the whole schedule: RAC, FP4, or (past the end) a repeat of
  // the last FP4 chunk into a stage nobody reads again
  auto issue_any = [&](int c, uint8_t* const sbase) {
    if (c < nrac) {
      issue_rac(c, sbase);
      issue_scales(0, sbase);   // keeps the count; the scale area is unused
    } else {
      issue_chunk(min(c - nrac, nk - 1), sbase);
    }
  };
  auto read_frag = [&](Frag& f, const uint8_t* const base, int s2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f.a[q] = *(const uint4*)(base + ca_off[s2] + q * Q_CODE);
      if constexpr (TILED)
        f.sa[q] = *(const uint32_t*)(base + sa_off[s2] + q * Q_SC);
      else
        f.sa[q] = *(const uint16_t*)(base + sa_off[s2] + q * Q_SC);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f.b[q] = *(const uint4*)(base + cb_off[s2] + q * Q_CODE);
      if constexpr (TILED)
        f.sb[q] = *(const uint32_t*)(base + sb_off[s2] + q * Q_SC);
      else
        f.sb[q] = *(const uint16_t*)(base + sb_off[s2] + q * Q_SC);
    }
  };
  auto decode = [&](const Frag& f, int j, half8v* da, half8v* db) {
    // the scale of each block in both fp16 halves
    auto dup = [&](uint32_t v) {
      if constexpr (TILED)   // fp16 pair (block 2p, block 2p + 1)
        return __builtin_amdgcn_perm(v, v, j >= 2 ? 0x03020302u : 0x01000100u);
      else                   // raw E4M3 pair
        return e4m3_dup_f16(v, j >= 2);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) da[q] = decode8(word(f.a[q], j), dup(f.sa[q]));
#pragma unroll
    for (int q = 0; q < 4; ++q) db[q] = decode8(word(f.b[q], j), dup(f.sb[q]));
  };

  f32x16v acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  auto mfma16 = [&](const half8v* da, const half8v* db) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[mi], db[ni], acc[mi][ni], 0, 0, 0);
  };

  // one half-chunk: MFMAs of steps j = 0..3 on `cur`, decoding step j + 1
  // (or step 0 of `next` after the last) into the other register set
  // The instruction order is pinned step by step: each MFMA is followed by
  // about five independent VALU instructions (the matrix core runs them in
  // its shadow); in the first step of a half the sixteen LDS reads of the
  // next half, and the `vmem` global -> LDS loads, go out behind the MFMAs.
  half8v da[2][4], db[2][4];
  auto half_chunk = [&](const Frag& cur, const Frag& next, int vmem) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3)
        decode(cur, j + 1, da[(j + 1) & 1], db[(j + 1) & 1]);
      else
        decode(next, 0, da[0], db[0]);
      mfma16(da[j & 1], db[j & 1]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
        if (j == 0) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
          if (i < vmem) __builtin_amdgcn_sched_group_barrier(0x060, 1, 0);   // VMEM
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);      // VALU
        } else {
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);      // VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Schedule chunk c lives in stage (c + roff) % 3, with roff chosen so that
  // FP4 chunk 0 (schedule chunk nrac) lands in stage 0: the FP4 loop then
  // needs no head, and only the cheap RAC part has one.  Prologue: chunks
  // 0..2 in flight.
  const int roff = (3 - nrac % 3) % 3;
  if (roff == 0) {
    issue_any(0, stage0); issue_any(1, stage1); issue_any(2, stage2);
  } else if (roff == 1) {
    issue_any(0, stage1); issue_any(1, stage2); issue_any(2, stage0);
  } else {
    issue_any(0, stage2); issue_any(1, stage0); issue_any(2, stage1);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_PER_CHUNK));   // chunk 0 has landed
  lds_barrier();

  // RAC first, into the zeroed accumulators: RAC chunk jr in stage
  // (jr + roff) % 3.  Each chunk is consumed in two halves of 16 bf16 MFMAs;
  // a half's fragments are read from LDS under the previous half's MFMAs, and
  // the wait for the next chunk (two more are in flight behind it) sits
  // between the halves, so no LDS read is exposed after the first.
  // Piece 2 s2 + h of a row: half s2 = 1 is half 0 with offset bit 5 flipped.
  if (nrac > 0) {
    uint32_t ra_off[2], rb_off[2];
    ra_off[0] = (uint32_t)swz(arow + l32, h);
    rb_off[0] = (uint32_t)(B_CODE_OFF + swz(bcol + l32, h));
    ra_off[1] = ra_off[0] ^ 32u;
    rb_off[1] = rb_off[0] ^ 32u;
    uint4 A0[4], B0[4], A1[4], B1[4];
    auto rd = [&](uint4* A, uint4* B, const uint8_t* const sb, int s2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        A[q] = *(const uint4*)(sb + ra_off[s2] + q * Q_CODE);
        B[q] = *(const uint4*)(sb + rb_off[s2] + q * Q_CODE);
      }
    };
    // NVFP4: fp16 operands (in the units of the W4A4 sum, or the exact
    // Eq. 21 values); MXFP4: bf16
    auto mm = [&](const uint4* A, const uint4* B) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          if constexpr (MX)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8v, A[mi]), __builtin_bit_cast(bf16x8v, B[ni]),
                acc[mi][ni], 0, 0, 0);
          else
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(half8v, A[mi]), __builtin_bit_cast(half8v, B[ni]),
                acc[mi][ni], 0, 0, 0);
        }
    };
    // RAC chunk jr in `cur`, the next chunk (RAC jr + 1, or FP4 chunk 0) in `nxt`
    auto rstep = [&](int jr, uint8_t* const cur, uint8_t* const nxt) {
      rd(A1, B1, cur, 1);
      mm(A0, B0);
      // chunk jr + 1 has landed; after the barrier every wave is done with `cur`
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_PER_CHUNK));
      lds_barrier();
      issue_any(jr + 3, cur);
      if (jr + 1 < nrac) rd(A0, B0, nxt, 0);
      mm(A1, B1);
    };
    auto rrun = [&](uint8_t* const s0, uint8_t* const s1, uint8_t* const s2) {
      rd(A0, B0, s0, 0);
      int jr = 0;
      for (; jr + 3 <= nrac; jr += 3) {
        rstep(jr, s0, s1);
        rstep(jr + 1, s1, s2);
        rstep(jr + 2, s2, s0);
      }
      if (jr < nrac) rstep(jr, s0, s1);
      if (jr + 1 < nrac) rstep(jr + 1, s1, s2);
    };
    // RAC chunk 0 sits in stage roff
    if (roff == 0)
      rrun(stage0, stage1, stage2);
    else if (roff == 1)
      rrun(stage1, stage2, stage0);
    else
      rrun(stage2, stage0, stage1);
  }

  // Y = s_A s_W (W4A4 sum + RAC'), the NVFP4 compensation operands coming
  // in fp16 in the sum's units (R 2^-e_A, W_S / (s_W f_A), s_A = f_A 2^e_A):
  // no scaling between the compensation and the FP4 chunks, and the product
  // of the tensor scales applied once in the epilogue without underflow
  // (out_scale).  The Eq. 21 form (RSC) adds its exact fp16 compensation with
  // the factor beta = -s_R s_W: the accumulators are taken to
  // beta / (s_A s_W) = -s_R / s_A (one fp32 division) before the FP4 chunks.
  // MXFP4: no tensor scale.
  const OutScale os =
      (!MX && g.a_ts) ? out_scale(g.a_ts[0], g.w_ts[ex]) : OutScale{1.0f, 0, false};
  if constexpr (RSC) {
    if (nrac > 0) {
      const float to_alpha = -(g.r_ts[0] / g.a_ts[0]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= to_alpha;
    }
  }

  if constexpr (MX) {
    // A fourth stage (the MXFP4 stage is smaller, and a chunk's 32 MFMAs are
    // a quarter of an NVFP4 chunk's work, so more of the load latency needs
    // cover): chunks 0..2 are in stages 0..2 (the RAC part or the prologue
    // put them there), chunk 3 goes to stage 3 now, and FP4 chunk kc lives
    // in stage kc % 4.  Per chunk: the chunk has landed, every wave reads
    // its fragments (two 64-element steps: lane half h supplies 32-element
    // block 2 j + h of its row), a barrier frees the stage for chunk kc + 4,
    // then 32 scaled FP4 MFMAs.
    __shared__ __attribute__((aligned(16))) uint8_t stage3[STAGE];
    issue_chunk(min(3, nk - 1), stage3);
    const int ra = arow + l32, rb = bcol + l32;
    uint32_t xa[2], xb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      xa[j] = (uint32_t)swz(ra, 2 * j + h);
      xb[j] = (uint32_t)(B_CODE_OFF + swz(rb, 2 * j + h));
    }
    const uint32_t xsa = (uint32_t)(A_SC_OFF + ra * 4), xsb = (uint32_t)(B_SC_OFF + rb * 4);
    auto mx_chunk = [&](int kc, uint8_t* const cur) {
      // chunks kc .. kc + 3 in flight: wait until chunk kc has landed
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * DMA_PER_CHUNK));
      lds_barrier();
      uint4 fa[2][4], fb[2][4];
      uint32_t sa[4], sb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sa[q] = *(const uint32_t*)(cur + xsa + q * 128);
        sb[q] = *(const uint32_t*)(cur + xsb + q * 128);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          fa[j][q] = *(const uint4*)(cur + xa[j] + q * Q_CODE);
          fb[j][q] = *(const uint4*)(cur + xb[j] + q * Q_CODE);
        }
      lds_barrier();   // every wave is done with this stage
      issue_chunk(min(kc + 4, nk - 1), cur);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = 2 * j + h;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const uint4 va = fa[j][mi], vb = fb[j][ni];
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                (i32x8v){(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0},
                (i32x8v){(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0}, acc[mi][ni], 4,
                4, 0, (int)(sa[mi] >> (8 * p)), 0, (int)(sb[ni] >> (8 * p)));
          }
      }
    };
    int kc = 0;
    for (; kc + 4 <= nk; kc += 4) {
      mx_chunk(kc, stage0);
      mx_chunk(kc + 1, stage1);
      mx_chunk(kc + 2, stage2);
      mx_chunk(kc + 3, stage3);
    }
    if (kc < nk) mx_chunk(kc, stage0);
    if (kc + 1 < nk) mx_chunk(kc + 1, stage1);
    if (kc + 2 < nk) mx_chunk(kc + 2, stage2);
  } else {
    // FP4 chunk kc is schedule chunk nrac + kc, in stage kc % 3; FP4 chunk 0
    // has landed behind a barrier (the prologue, or the last RAC step)
    Frag f0, f1;
    read_frag(f0, stage0, 0);
    decode(f0, 0, da[0], db[0]);

    // one FP4 chunk; the chunk issued three ahead is FP4 chunk kc + 3, or a
    // repeat of the last one past the end.  In the main loop its loads are
    // interleaved with the MFMAs (LOOP); the tail copies issue them in one
    // block, which also keeps the compiler from merging those copies with
    // the loop body (that would make the stage addresses dynamic).
    auto chunk = [&](int kc, uint8_t* const cur, uint8_t* const nxt, auto loop) {
      read_frag(f1, cur, 1);
      half_chunk(f0, f1, 0);
      // chunk kc + 1 has landed (chunk kc + 2 may still be in flight); after
      // the barrier every wave is done with stage `cur`
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_PER_CHUNK));
      lds_barrier();
      read_frag(f0, nxt, 0);
      issue_chunk(min(kc + 3, nk - 1), cur);
      half_chunk(f1, f0, decltype(loop)::value ? DMA_PER_CHUNK : 0);
    };
    using in_loop = std::true_type;
    using edge = std::false_type;
    int kc = 0;
    for (; kc + 3 <= nk; kc += 3) {
      chunk(kc, stage0, stage1, in_loop{});
      chunk(kc + 1, stage1, stage2, in_loop{});
      chunk(kc + 2, stage2, stage0, in_loop{});
    }
    if (kc < nk) chunk(kc, stage0, stage1, edge{});
    if (kc + 1 < nk) chunk(kc + 1, stage1, stage2, edge{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  // The epilogue, once with the single multiply by s_A s_W and once (a
  // product below fp32's normal range) with mantissa and exponent apart.
  auto epilogue = [&](auto split) {
    auto sc = [&](float v) {
      if constexpr (decltype(split)::value)
        return ldexpf(v * os.mul, os.e);
      else
        return v * os.mul;
    };
    // Accumulator element r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32 of its 32 x 32 tile.
    if constexpr (EPI == kEpiSwiGLU || EPI == kEpiSwiGLUQuant) {
      // W13 with gate and up rows interleaved in blocks of 32: MFMA column
      // tile ni = 2p is the gate and 2p + 1 the up of h columns
      // (n0 + 128 wn) / 2 + 32 p + l % 32; h = silu(gate) * up as bf16 into
      // Y [rows][ldy], ldy >= N / 2.  Staged through LDS per pass (a wave's 16
      // rows x 64 h columns) so that every store writes 16 contiguous bytes.
      constexpr bool QH = EPI == kEpiSwiGLUQuant;
      const int64_t fcols = N / 2, f0 = (n0 + bcol) / 2;
      const bool staged =
          QH || ((fcols % 8) == 0 && (g.ldy % 8) == 0 && (((uintptr_t)g.Y) & 15u) == 0);
      auto hval = [&](int mi, int p, int r) {
        return silu(sc(acc[mi][2 * p][r])) * (sc(acc[mi][2 * p + 1][r]));
      };
      if (staged) {
        __syncthreads();   // every wave is done with the stages
        constexpr int PS = 144;   // row pitch (bytes): 64 bf16 and 16 bytes of pad
        uint8_t* const ep = stage0 + wave * (16 * PS);
        // QH: h quantized as it is stored (NVFP4 under the supplied tensor
        // scale q_ts, the stand-alone quantizer's encoding): the lane that
        // stores 8 h values of a row encodes them, its neighbour (lane ^ 1)
        // holding the other half of their 16-block; each lane keeps the fp64
        // sums of squared residuals of its 8 columns.
        float qst = 1.0f, inv6st = 1.0f;
        double st6 = 6.0;
        int eDp = 0, tie_mode = kTieEven;
        uint8_t* const tab = stage2;
        if constexpr (QH) {
          qst = g.q_ts[0];
          tie_mode = supplied_tie_mode(qst);
          int eD;
          const double Dm = frexp(6.0 * (double)qst, &eD);   // 6 s_t = Dm 2^eD, Dm in [0.5, 1)
          eDp = eD - 1;
          inv6st = 1.0f / (6.0f * qst);
          st6 = 6.0 * (double)qst;
          if (tid < 128) tab[tid] = (uint8_t)e4m3_mantissa_entry(tid, 2.0 * Dm);
          __syncthreads();
        }
        if constexpr (!QH) {
  #pragma unroll
          for (int mi = 0; mi < 4; ++mi) {
  #pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int64_t rbase = m0 + arow + mi * 32 + 16 * half;
  #pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
  #pragma unroll
                for (int rr = 0; rr < 8; rr += 2) {
                  const int r = 8 * half + rr;
                  const int lr = 8 * (rr >> 2) + 4 * h + (rr & 3);
                  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                  const bf16x2 pr = {(__bf16)hval(mi, pp, r), (__bf16)hval(mi, pp, r + 1)};
                  const uint32_t w = __builtin_bit_cast(uint32_t, pr);
                  uint8_t* const q = ep + lr * PS + (pp * 32 + l32) * 2;
                  *(uint16_t*)q = (uint16_t)w;
                  *(uint16_t*)(q + PS) = (uint16_t)(w >> 16);
                }
              }
  #pragma unroll
              for (int it = 0; it < 2; ++it) {
                const int cid = it * 64 + lane, lr = cid >> 3, cc = (cid & 7) * 8;
                const uint4 v = *(const uint4*)(ep + lr * PS + cc * 2);
                const int64_t row = rbase + lr, col = f0 + cc;
                if (row < m_end && col < fcols) *(uint4*)((uint16_t*)g.Y + row * g.ldy + col) = v;
              }
            }
          }
        } else {
          // The wave's whole 128 x 64 h block goes to LDS first (its own
          // region, two waves per stage), then comes back in 16 groups of 8
          // values per lane, encoded four groups at a time: independent
          // chains, so that one wave per SIMD still hides the latencies.
          uint8_t* const epq = (wave < 2 ? stage0 : stage1) + (wave & 1) * (128 * PS);
  #pragma unroll
          for (int mi = 0; mi < 4; ++mi) {
  #pragma unroll
            for (int half = 0; half < 2; ++half) {
  #pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
  #pragma unroll
                for (int rr = 0; rr < 8; rr += 2) {
                  const int r = 8 * half + rr;
                  const int lr = mi * 32 + 16 * half + 8 * (rr >> 2) + 4 * h + (rr & 3);
                  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                  const bf16x2 pr = {(__bf16)hval(mi, pp, r), (__bf16)hval(mi, pp, r + 1)};
                  const uint32_t w = __builtin_bit_cast(uint32_t, pr);
                  uint8_t* const q = epq + lr * PS + (pp * 32 + l32) * 2;
                  *(uint16_t*)q = (uint16_t)w;
                  *(uint16_t*)(q + PS) = (uint16_t)(w >> 16);
                }
              }
            }
          }
          // QH: h quantized as it is stored (NVFP4 under the supplied tensor
          // scale q_ts, the stand-alone quantizer's encoding): the lane that
          // stores 8 h values of a row encodes them, its neighbour (lane ^ 1)
          // holding the other half of their 16-block; each lane keeps the
          // fp64 sums of squared residuals of its 8 columns (lane % 8 fixes
          // them).  Every lane encodes (the block amax and the near-tie
          // rounds span lanes); only live ones store and count.
          double qacc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) qacc[i] = 0.0;
          const int cc = (lane & 7) * 8;
          const int64_t col = f0 + cc;
#pragma unroll
          for (int g4 = 0; g4 < 16; g4 += 4) {
            uint4 v[4];
            float xf[4][8], bm[4];
            int lrow[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              lrow[u] = 16 * ((g4 + u) >> 1) + 8 * ((g4 + u) & 1) + (lane >> 3);
              v[u] = *(const uint4*)(epq + lrow[u] * PS + cc * 2);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              xf[u][0] = bf16_lo(v[u].x); xf[u][1] = bf16_hi(v[u].x);
              xf[u][2] = bf16_lo(v[u].y); xf[u][3] = bf16_hi(v[u].y);
              xf[u][4] = bf16_lo(v[u].z); xf[u][5] = bf16_hi(v[u].z);
              xf[u][6] = bf16_lo(v[u].w); xf[u][7] = bf16_hi(v[u].w);
              float m = 0.0f;
#pragma unroll
              for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(xf[u][i]));
              bm[u] = fmaxf(m, dpp_quad_xor1(m));   // 16-block = lane pair
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int64_t row = m0 + arow + lrow[u];
              const bool live = row < m_end && col < fcols;
              uint32_t code, scode;
              float s;
              nvfp4_lane_encode<false, 8, true>(&v[u], xf[u], bm[u], qst, eDp, tab, inv6st, st6,
                                                tie_mode, &code, &scode, &s);
              if (live) {
                *(uint4*)((uint16_t*)g.Y + row * g.ldy + col) = v[u];
                *(uint32_t*)(g.q_codes + row * (fcols / 2) + col / 2) = code;
                if ((lane & 1) == 0) g.q_scales[row * (fcols / 16) + col / 16] = (uint8_t)scode;
                const f32x2v c2[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0),
                                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 1),
                                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 2),
                                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 3)};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                  // r = RN32(x - c s s_t): c s is exact, one fused rounding
                  const double r0 = (double)fmaf(-(c2[b].x * s), qst, xf[u][2 * b]);
                  const double r1 = (double)fmaf(-(c2[b].y * s), qst, xf[u][2 * b + 1]);
                  qacc[2 * b] = fma(r0, r0, qacc[2 * b]);
                  qacc[2 * b + 1] = fma(r1, r1, qacc[2 * b + 1]);
                }
              }
            }
          }
          // lanes with the same lane % 8 hold the same 8 columns over
          // different rows: add them (fixed order), then lanes 0..7 write the
          // wave's 128-row half-tile sums
#pragma unroll
          for (int o = 8; o < 64; o <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i) qacc[i] += __shfl_xor(qacc[i], o, 64);
          if (lane < 8) {
            double* const dst = g.q_partial + (int64_t)(2 * mt + wm) * fcols + f0 + lane * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (f0 + lane * 8 + i < fcols) dst[i] = qacc[i];
          }
        }
      } else {
  #pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + arow + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (row >= m_end) continue;
  #pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int64_t col = f0 + pp * 32 + l32;
              if (col < fcols)
                ((uint16_t*)g.Y)[row * g.ldy + col] = (uint16_t)f32_to_bf16_rne(hval(mi, pp, r));
            }
          }
        }
      }
      return;
    }

    // Epilogue through LDS so that every global store writes 16 contiguous
    // bytes: per pass, a wave's 16 rows x 128 columns (rows 16 * half .. + 15 of
    // MFMA tile row mi) go to its own LDS region and come back as row chunks.
    const int vec = g.y_bf16 ? 8 : 4;
    const bool staged = (N % vec) == 0 && (g.ldy % vec) == 0 && (((uintptr_t)g.Y) & 15u) == 0;
    if (staged) {
      __syncthreads();   // every wave is done with the stages
      constexpr int PB = 272, PF = 544;   // row pitches (bytes) of the bf16 / fp32 staging tiles
      uint8_t* const ep = stage0 + wave * (16 * PF);
  #pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
  #pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int64_t rbase = m0 + arow + mi * 32 + 16 * half;
          if (g.y_bf16) {
  #pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
  #pragma unroll
              for (int rr = 0; rr < 8; rr += 2) {
                const int r = 8 * half + rr;
                const int lr = 8 * ((r >> 2) - 2 * half) + 4 * h + (r & 3);
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 pr = {(__bf16)sc(acc[mi][ni][r]),
                                   (__bf16)sc(acc[mi][ni][r + 1])};
                const uint32_t w = __builtin_bit_cast(uint32_t, pr);
                uint8_t* const p = ep + lr * PB + (ni * 32 + l32) * 2;
                *(uint16_t*)p = (uint16_t)w;
                *(uint16_t*)(p + PB) = (uint16_t)(w >> 16);
              }
            }
  #pragma unroll
            for (int it = 0; it < 4; ++it) {
              const int cid = it * 64 + lane, lr = cid >> 4, cc = (cid & 15) * 8;
              const uint4 v = *(const uint4*)(ep + lr * PB + cc * 2);
              const int64_t row = rbase + lr, col = n0 + bcol + cc;
              if (row < m_end && col < N)   // nontemporal, as the fp32 rows below
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, v),
                                            (u32x4v*)((uint16_t*)g.Y + row * g.ldy + col));
            }
          } else {
  #pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
  #pragma unroll
              for (int rr = 0; rr < 8; ++rr) {
                const int r = 8 * half + rr;
                const int lr = 8 * ((r >> 2) - 2 * half) + 4 * h + (r & 3);
                *(float*)(ep + lr * PF + (ni * 32 + l32) * 4) = sc(acc[mi][ni][r]);
              }
            }
  #pragma unroll
            for (int it = 0; it < 8; ++it) {
              const int cid = it * 64 + lane, lr = cid >> 5, cc = (cid & 31) * 4;
              const uint4 v = *(const uint4*)(ep + lr * PF + cc * 4);
              const int64_t row = rbase + lr, col = n0 + bcol + cc;
              // nontemporal: an output of this size is read back by another
              // kernel, once, long after; keeping it out of the caches frees
              // the write path for the next tiles' loads
              if (row < m_end && col < N)
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, v),
                                            (u32x4v*)((float*)g.Y + row * g.ldy + col));
            }
          }
        }
      }
      return;
    }
  #pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
  #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + arow + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row >= m_end) continue;
  #pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int64_t col = n0 + bcol + ni * 32 + l32;
          if (col >= N) continue;
          const float v = sc(acc[mi][ni][r]);
          if (g.y_bf16)
            ((uint16_t*)g.Y)[row * g.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            ((float*)g.Y)[row * g.ldy + col] = v;
        }
      }
    }
  };
  if (os.split)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
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

// Grouped 256 x 256 tiles address A (codes, scales) and R rows absolutely,
// from the start of the operand, with 32-bit offsets: at most 4 GiB of them
static bool grouped_offsets_fit(const GemmArgs& g) {
  const int64_t rows = g.a_src_rows > 0 ? g.a_src_rows : g.M;
  const int64_t row_bytes = std::max<int64_t>(g.K / 2, g.r_res ? 2 * (int64_t)g.ld_r : 0);
  return rows * row_bytes <= (int64_t)0xffffffffLL;
}

bool grouped_wide_ok(int64_t K, int64_t N) { return K % BK == 0 && K >= 512 && N % 512 == 0; }

bool grouped_big_path(const GemmArgs& g) {
  if (g.mx || g.tiles == nullptr || (g.K % BK) != 0 || g.N % big::BN != 0) return false;
  if (!grouped_offsets_fit(g)) return false;
  return (g.a_scales_t && g.w_scales_t) ? g.K >= 512 : g.K >= 1024;
}

hipError_t launch_w4a4_gemm(const GemmArgs& g, int64_t max_mtiles, hipStream_t stream) {
  const bool fullk = (g.K % BK) == 0;
  const bool grouped = g.tiles != nullptr;
  // 128 x 512 tiles: the caller's table lists kWideBM-row M tiles
  if (g.wide) {
    if (!grouped || !g.a_scales_t || !g.w_scales_t || !grouped_wide_ok(g.K, g.N) ||
        g.epilogue == kEpiSwiGLUQuant || g.mx || !grouped_offsets_fit(g))
      return hipErrorInvalidValue;
    const int64_t nb = (max_mtiles * (g.N / 512) + 7) / 8 * 8;
    if (nb == 0) return hipSuccess;
    if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, true, kEpiSwiGLU, false, false, true>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, true, kEpiStore, false, false, true>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  // MXFP4 grouped: the 256 x 256 tiles win from K = 512 on (no decode, so a
  // tile's fixed cost is smaller than on the NVFP4 path, which keeps its
  // 256 x 128 tiles below K = 1024)
  if (g.mx && grouped && fullk && g.N % big::BN == 0 && g.K >= 512 && grouped_offsets_fit(g)) {
    const int64_t nb = (max_mtiles * (g.N / big::BN) + 7) / 8 * 8;
    if (nb == 0) return hipSuccess;
    if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, true, kEpiSwiGLU, false, true>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, true, kEpiStore, false, true>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (g.mx && !grouped && fullk && g.epilogue == kEpiStore && g.M >= 512 && g.N >= 512) {
    const int64_t nb = ((g.M + big::BM - 1) / big::BM) * ((g.N + big::BN - 1) / big::BN);
    hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, false, kEpiStore, false, true>),
                       dim3((unsigned)nb), dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (g.mx) {
    if (fullk)
      return grouped ? launch_t<true, true, true>(g, max_mtiles, stream)
                     : launch_t<true, false, true>(g, max_mtiles, stream);
    return grouped ? launch_t<false, true, true>(g, max_mtiles, stream)
                   : launch_t<false, false, true>(g, max_mtiles, stream);
  }
  if (!grouped && fullk && g.epilogue == kEpiStore && g.M >= 512 && g.N >= 512) {
    const int64_t nb = ((g.M + big::BM - 1) / big::BM) * ((g.N + big::BN - 1) / big::BN);
    if (g.r_ts && g.a_ts && g.a_scales_t && g.w_scales_t)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, false, kEpiStore, true>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    else if (g.r_ts && g.a_ts)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, false, kEpiStore, true>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    else if (g.a_scales_t && g.w_scales_t)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, false, kEpiStore>), dim3((unsigned)nb),
                         dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, false, kEpiStore>), dim3((unsigned)nb),
                         dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  // Grouped 256 x 256 tiles: with the tiled scale records from K = 512 on,
  // with raw scales from K = 1024 (below that the fixed cost of a 256 x 256
  // tile outweighs its better decode reuse; the 256 x 128 kernel does those).
  // The grid covers every possible tile, rounded up to whole XCD rounds;
  // workgroups past the tiles that exist return at once.
  if (g.epilogue == kEpiSwiGLUQuant && !grouped_big_path(g)) return hipErrorInvalidValue;
  if (grouped && fullk && g.N % big::BN == 0 && g.a_scales_t && g.w_scales_t && g.K >= 512 &&
      grouped_offsets_fit(g)) {
    const int64_t nb = (max_mtiles * (g.N / big::BN) + 7) / 8 * 8;
    if (nb == 0) return hipSuccess;
    if (g.epilogue == kEpiSwiGLUQuant)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, true, kEpiSwiGLUQuant>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    else if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, true, kEpiSwiGLU>), dim3((unsigned)nb),
                         dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<true, true, kEpiStore>), dim3((unsigned)nb),
                         dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (grouped && fullk && g.N % big::BN == 0 && g.K >= 1024 && grouped_offsets_fit(g)) {
    const int64_t nb = (max_mtiles * (g.N / big::BN) + 7) / 8 * 8;
    if (nb == 0) return hipSuccess;
    if (g.epilogue == kEpiSwiGLUQuant)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, true, kEpiSwiGLUQuant>),
                         dim3((unsigned)nb), dim3(256), 0, stream, g);
    else if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, true, kEpiSwiGLU>), dim3((unsigned)nb),
                         dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((big::gemm_nvfp4_big_kernel<false, true, kEpiStore>), dim3((unsigned)nb),
                         dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (fullk)
    return grouped ? launch_t<true, true, false>(g, max_mtiles, stream)
                   : launch_t<true, false, false>(g, max_mtiles, stream);
  return grouped ? launch_t<false, true, false>(g, max_mtiles, stream)
                 : launch_t<false, false, false>(g, max_mtiles, stream);
}

// tiled fp16 scale records for the 256 x 256 kernel (body in q4_prep.h)
__global__ __launch_bounds__(256) void scale_tile_kernel(const uint8_t* __restrict__ sc,
                                                         int64_t rows, int32_t K,
                                                         int64_t rows_pad,
                                                         uint4* __restrict__ out) {
  scale_tile_part(sc, rows, K, rows_pad, out, blockIdx.x, gridDim.x);
}

hipError_t launch_scale_tile(const uint8_t* scales, int64_t rows, int32_t K, int64_t rows_pad,
                             uint8_t* out, hipStream_t stream) {
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  grid = grid > 8192 ? 8192 : grid;
  hipLaunchKernelGGL(scale_tile_kernel, dim3((unsigned)grid), dim3(256), 0, stream, scales, rows,
                     K, rows_pad, (uint4*)out);
  return hipGetLastError();
}

// records of `batch` operands of [rows][K / 16] scales each, one block of
// [K / 128][rows_pad][16 B] per operand (the expert weights of a grouped GEMM)
__global__ __launch_bounds__(256) void scale_tile_batched_kernel(const uint8_t* __restrict__ sc,
                                                                 int64_t rows, int32_t K,
                                                                 int64_t rows_pad,
                                                                 uint4* __restrict__ out) {
  const int64_t b = blockIdx.y;
  scale_tile_part(sc + b * rows * (K / 16), rows, K, rows_pad, out + b * (K / 128) * rows_pad,
                  blockIdx.x, gridDim.x);
}

hipError_t launch_scale_tile_batched(const uint8_t* scales, int64_t batch, int64_t rows, int32_t K,
                                     int64_t rows_pad, uint8_t* out, hipStream_t stream) {
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  if (total == 0 || batch == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  grid = grid > 1024 ? 1024 : grid;
  hipLaunchKernelGGL(scale_tile_batched_kernel, dim3((unsigned)grid, (unsigned)batch), dim3(256), 0,
                     stream, scales, rows, K, rows_pad, (uint4*)out);
  return hipGetLastError();
}

// MXFP4 scale records: the four E8M0 bytes of one row and 128-column chunk,
// chunk-major, so that a tile's rows of one chunk are contiguous
__global__ __launch_bounds__(256) void mx_scale_records_kernel(const uint8_t* __restrict__ sc,
                                                               int64_t rows, int32_t K,
                                                               int64_t rows_pad,
                                                               uint32_t* __restrict__ out) {
  const int64_t b = blockIdx.y;
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  const uint8_t* src = sc + b * rows * (K / 32);
  uint32_t* dst = out + b * total;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t c = i / rows_pad, r = i - c * rows_pad;
    dst[i] = r < rows ? *(const uint32_t*)(src + r * (K / 32) + 4 * c) : 0u;
  }
}

hipError_t launch_mx_scale_records(const uint8_t* scales, int64_t batch, int64_t rows, int32_t K,
                                   int64_t rows_pad, uint8_t* out, hipStream_t stream) {
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  if (total == 0 || batch == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  grid = grid > 1024 ? 1024 : grid;
  hipLaunchKernelGGL(mx_scale_records_kernel, dim3((unsigned)grid, (unsigned)batch), dim3(256), 0,
                     stream, scales, rows, K, rows_pad, (uint32_t*)out);
  return hipGetLastError();
}

// Records of the R token-sorted rows of a grouped GEMM's A operand: record
// (c, r) holds the scales of source row a_rows[r] (r itself without a_rows),
// swizzled for the row's offset within its expert (the expert being the last
// e with offsets[e] <= r), which is the row's place in its 256-row tile;
// rows R .. rows_pad - 1 are zero.
__global__ __launch_bounds__(256) void scale_tile_sorted_kernel(
    const uint8_t* __restrict__ sc, const int32_t* __restrict__ a_rows, int64_t R, int32_t K,
    const int32_t* __restrict__ offsets, int32_t E, int64_t rows_pad, uint4* __restrict__ out) {
  // the experts' first rows, searched in LDS (E <= 1024)
  __shared__ int32_t s_off[1025];
  for (int e = threadIdx.x; e <= E; e += 256) s_off[e] = offsets[e];
  __syncthreads();
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  const half2v k256 = {(_Float16)256.0f, (_Float16)256.0f};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t c = i / rows_pad, r = i - c * rows_pad;
    uint2 raw = make_uint2(0, 0);
    int in_tile = 0;
    if (r < R) {
      const int64_t src = a_rows ? (int64_t)a_rows[r] : r;
      raw = *(const uint2*)(sc + src * (K / 16) + 8 * c);
      int lo = 0, hi = E;   // offsets[0] <= r < offsets[E]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)s_off[mid] <= r) lo = mid;
        else hi = mid;
      }
      in_tile = (int)((r - s_off[lo]) & 255);
    }
    // each E4M3 byte shifted left by 7 is an fp16 of 2^-8 times its value;
    // the multiply by 256 is exact
    const uint32_t d0 = __builtin_amdgcn_perm(0u, raw.x, 0x0c010c00u) << 7;
    const uint32_t d1 = __builtin_amdgcn_perm(0u, raw.x, 0x0c030c02u) << 7;
    const uint32_t d2 = __builtin_amdgcn_perm(0u, raw.y, 0x0c010c00u) << 7;
    const uint32_t d3 = __builtin_amdgcn_perm(0u, raw.y, 0x0c030c02u) << 7;
    const uint4 rec = make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d0) * k256),
                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d1) * k256),
                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d2) * k256),
                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d3) * k256));
    out[i] = swz_sc_rec(rec, in_tile);
  }
}

hipError_t launch_scale_tile_sorted(const uint8_t* scales, const int32_t* a_rows, int64_t R,
                                    int32_t K, const int32_t* offsets, int32_t E, int64_t rows_pad,
                                    uint8_t* out, hipStream_t stream) {
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  grid = grid > 4096 ? 4096 : grid;
  hipLaunchKernelGGL(scale_tile_sorted_kernel, dim3((unsigned)grid), dim3(256), 0, stream, scales,
                     a_rows, R, K, offsets, E, rows_pad, (uint4*)out);
  return hipGetLastError();
}

}  // namespace q4
