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

// the four dwords of a 16-byte scale record in swizzled order for row `row`
__device__ __forceinline__ uint4 swz_sc_rec(uint4 v, int row) {
  const int q = (row >> 3) & 3;
  uint4 r;
  r.x = q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
  r.y = q == 0 ? v.y : (q == 1 ? v.x : (q == 2 ? v.w : v.z));
  r.z = q == 0 ? v.z : (q == 1 ? v.w : (q == 2 ? v.x : v.y));
  r.w = q == 0 ? v.w : (q == 1 ? v.z : (q == 2 ? v.y : v.x));
  return r;
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
constexpr int A_SC_OFF = B_CODE_OFF + BN * CB;      // 32768 (E4M3, 8 bytes per row)
constexpr int B_SC_OFF = A_SC_OFF + BM * 8;         // 34816
constexpr int STAGE = B_SC_OFF + BN * 8;            // 36864
constexpr int DMA_PER_CHUNK = 12;                   // per wave: 8 code + 4 scale loads

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

__global__ __launch_bounds__(256, 1) void gemm_nvfp4_big_kernel(GemmArgs g) {
  // one LDS object per stage, addressed with compile-time stage indices, so
  // the compiler can tell that reads of one stage do not wait for the
  // global -> LDS loads still filling another
  __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t stage2[STAGE];
  uint8_t* const stages[NST] = {stage0, stage1, stage2};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int K = g.K;
  const int64_t N = g.N;
  const int nk = K / BK;

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
  // rows past the end of A or W read the last row again: their products land
  // only in output rows / columns that are never stored
  const int a_last = (int)min<int64_t>(BM - 1, g.M - 1 - m0);
  const int b_last = (int)min<int64_t>(BN - 1, N - 1 - n0);

  const uint32_t cstride = (uint32_t)(K / 2), sstride = (uint32_t)(K / 16);
  const uint8_t* const a_base = g.a_codes + (size_t)m0 * cstride;
  const uint8_t* const b_base = g.w_codes + (size_t)n0 * cstride;
  // direct loads: instruction `it` of this wave fills the 1 KiB of LDS that
  // holds tile rows 16 * (4 * it + wave) .. + 15; lane l writes 16 bytes at
  // l * 16, i.e. row 16 * c + l / 4, swizzled slot l % 4, which holds the
  // logical 16-byte piece slot ^ f(row)
  uint32_t a_goff[4], b_goff[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 16 * (4 * it + wave) + (lane >> 2);
    const int piece = (lane & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
    a_goff[it] = (uint32_t)min(row, a_last) * cstride + (uint32_t)piece * 16u;
    b_goff[it] = (uint32_t)min(row, b_last) * cstride + (uint32_t)piece * 16u;
  }
  // scale loads: instruction `it` of this wave fills 256 bytes of LDS (rows
  // 32 * (4 * it + wave) .. + 31, 8 bytes each); lane l loads dword l % 2 of
  // row 32 * c + l / 2
  const uint8_t* const as_base = g.a_scales + (size_t)m0 * sstride;
  const uint8_t* const bs_base = g.w_scales + (size_t)n0 * sstride;
  uint32_t as_goff[2], bs_goff[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int row = 32 * (4 * it + wave) + (lane >> 1);
    as_goff[it] = (uint32_t)min(row, a_last) * sstride + (uint32_t)(lane & 1) * 4u;
    bs_goff[it] = (uint32_t)min(row, b_last) * sstride + (uint32_t)(lane & 1) * 4u;
  }

  // LDS read offsets within a stage for half s2 = 0 (s2 = 1: code ^ 16,
  // scale + 2); piece p = 2 h + s2 holds scale blocks 2p and 2p + 1
  uint32_t ca_off[4], cb_off[4], sa_off[4], sb_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ra = wm * 128 + q * 32 + l32, rb = wn * 128 + q * 32 + l32;
    ca_off[q] = (uint32_t)swz(ra, 2 * h);
    cb_off[q] = (uint32_t)(B_CODE_OFF + swz(rb, 2 * h));
    sa_off[q] = (uint32_t)(A_SC_OFF + ra * 8 + 4 * h);
    sb_off[q] = (uint32_t)(B_SC_OFF + rb * 8 + 4 * h);
  }

  // all global -> LDS traffic of chunk kc (clamped: chunks past the end
  // reload the last one into a stage nobody reads again)
  auto issue_chunk = [&](int kc, uint8_t* const sbase) {
    const uint32_t kb = (uint32_t)min(kc, nk - 1) * (BK / 2);
    const uint32_t ks = (uint32_t)min(kc, nk - 1) * (BK / 16);
    uint8_t* const dst = sbase + wave * 1024;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      __builtin_amdgcn_global_load_lds((gptr_t)(a_base + kb + a_goff[it]),
                                       (lptr_t)(dst + it * 4096), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(b_base + kb + b_goff[it]),
                                       (lptr_t)(dst + B_CODE_OFF + it * 4096), 16, 0, 0);
    }
    uint8_t* const sdst = sbase + wave * 256;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      __builtin_amdgcn_global_load_lds((gptr_t)(as_base + ks + as_goff[it]),
                                       (lptr_t)(sdst + A_SC_OFF + it * 1024), 4, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(bs_base + ks + bs_goff[it]),
                                       (lptr_t)(sdst + B_SC_OFF + it * 1024), 4, 0, 0);
    }
  };
  auto read_frag = [&](Frag& f, const uint8_t* const base, int s2) {
    const uint32_t cx = s2 ? 16u : 0u, sx = s2 ? 2u : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f.a[q] = *(const uint4*)(base + (ca_off[q] ^ cx));
      f.sa[q] = *(const uint16_t*)(base + sa_off[q] + sx);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f.b[q] = *(const uint4*)(base + (cb_off[q] ^ cx));
      f.sb[q] = *(const uint16_t*)(base + sb_off[q] + sx);
    }
  };
  auto decode = [&](const Frag& f, int j, half8v* da, half8v* db) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      da[q] = decode8(word(f.a[q], j), e4m3_dup_f16(f.sa[q], j >= 2));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      db[q] = decode8(word(f.b[q], j), e4m3_dup_f16(f.sb[q], j >= 2));
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

  // prologue: chunks 0..2 in flight
  issue_chunk(0, stages[0]);
  issue_chunk(1, stages[1]);
  issue_chunk(2, stages[2]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_PER_CHUNK));   // chunk 0 has landed
  lds_barrier();
  Frag f0, f1;
  read_frag(f0, stages[0], 0);
  decode(f0, 0, da[0], db[0]);

  // chunk kc lives in stage kc % 3
  auto chunk = [&](int kc, uint8_t* const cur, uint8_t* const nxt) {
    read_frag(f1, cur, 1);
    half_chunk(f0, f1, 0);
    // chunk kc + 1 has landed (chunk kc + 2 may still be in flight); after
    // the barrier every wave is done with stage `cur`
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_PER_CHUNK));
    lds_barrier();
    read_frag(f0, nxt, 0);
    issue_chunk(kc + 3, cur);
    half_chunk(f1, f0, DMA_PER_CHUNK);
  };
  int kc = 0;
  for (; kc + 3 <= nk; kc += 3) {
    chunk(kc, stages[0], stages[1]);
    chunk(kc + 1, stages[1], stages[2]);
    chunk(kc + 2, stages[2], stages[0]);
  }
  if (kc < nk) chunk(kc, stages[0], stages[1]);
  if (kc + 1 < nk) chunk(kc + 1, stages[1], stages[2]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

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
  if (!grouped && fullk && g.epilogue == kEpiStore && g.M >= 512 && g.N >= 512) {
    const int64_t nb = ((g.M + big::BM - 1) / big::BM) * ((g.N + big::BN - 1) / big::BN);
    hipLaunchKernelGGL(big::gemm_nvfp4_big_kernel, dim3((unsigned)nb), dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (fullk)
    return grouped ? launch_t<true, true, false>(g, max_mtiles, stream)
                   : launch_t<true, false, false>(g, max_mtiles, stream);
  return grouped ? launch_t<false, true, false>(g, max_mtiles, stream)
                 : launch_t<false, false, false>(g, max_mtiles, stream);
}

}  // namespace q4
