// Grouped W4A4 (+ residual compensation) GEMM for expert groups of few rows:
// the decode-shaped MoE layer, where each expert sees a handful of tokens and
// the layer is bound by streaming the expert weights from HBM.
//
// QUADS (arXiv 2607.15810) section 3.3: the W4A4 product on FP4 operands with
// the residual of the selected channels (Eq. 21) accumulated on top; the
// expert layer is the top-k MoE block the page profiles (W13 site, Figure 4b).
//
// A tile is at most 32 rows of one expert (the 32-row tile table) by 256
// output columns; each wave owns 64 of the columns (two 32 x 32 MFMA tiles)
// and streams its own weight rows straight from global memory into registers,
// one K-chunk ahead, with no LDS and no barriers.  The few activation rows are
// read by every wave (they stay in the caches).  NVFP4 fragments are decoded
// exactly to fp16 (c * sb has at most six significant bits) for
// v_mfma_f32_32x32x16_f16; MXFP4 fragments go to the scaled FP4 instruction
// with their E8M0 block scales.  Lane (row l % 32, half h) supplies, for
// K-step (s2, j), word j of the 16-byte piece 2 h + s2 of its row's 64-byte
// chunk, the same K order for both operands.
#include <algorithm>

#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int SM = 32;    // rows per tile
constexpr int SN = 256;   // output columns per workgroup
constexpr int CK = 128;   // K per chunk

__device__ __forceinline__ uint32_t e4m3_dup_f16_s(uint32_t pair, int which) {
  const half2v k256 = {(_Float16)256.0f, (_Float16)256.0f};
  const uint32_t d = __builtin_amdgcn_perm(0u, pair, which ? 0x0c010c01u : 0x0c000c00u) << 7;
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d) * k256);
}

__device__ __forceinline__ half8v decode8_s(uint32_t w, uint32_t pair) {
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

__device__ __forceinline__ uint32_t word_s(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// one K-chunk of one lane: codes of the lane's A row and of its two W rows
// (pieces 2h and 2h + 1), and the E4M3 bytes of blocks 4h .. 4h + 3 (NVFP4)
// or the E8M0 bytes of blocks 2 s + h (MXFP4, two 64-element steps)
struct SkinnyChunk {
  uint4 a[2], b[2][2];
  uint32_t sa, sb[2];
};

// The tail of a skinny tile: Y = s_A s_W * (sum + compensation), the NVFP4
// compensation operands in fp16 in the sum's units, MXFP4's in bf16 added
// after the (unit) scaling; the product of the tensor scales applied without
// underflow.  The compensation's R rows are the lane's activation row ar
// (rok: inside the tile), its weight columns the gathered W_S.
template <bool MX>
__device__ __forceinline__ void skinny_tail(const GemmArgs& g, f32x16v (&acc)[2], int e,
                                            int64_t ar, bool rok, const bool (&cok)[2], int64_t c0,
                                            int l32, int h) {
  const int64_t N = g.N;
  const OutScale os = g.a_ts ? out_scale(g.a_ts[0], g.w_ts[e]) : OutScale{1.0f, 0, false};
  const bool units = g.kp > 0 && g.r_res && !MX;
  if (!units) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[ni][q] = apply_scale(os, acc[ni][q]);
  }
  if (g.kp > 0 && g.r_res) {
    const uint16_t* rrow = g.r_res + ar * g.ld_r + 8 * h;
    const uint16_t* wrw[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int64_t col = c0 + ni * 32 + l32;
      wrw[ni] = g.w_sel + ((int64_t)e * N + (cok[ni] ? col : 0)) * g.kp + 8 * h;
    }
    for (int kt = 0; kt < g.kp; kt += 16) {
      const uint4 av = rok ? *(const uint4*)(rrow + kt) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const uint4 bv = cok[ni] ? *(const uint4*)(wrw[ni] + kt) : make_uint4(0, 0, 0, 0);
        if constexpr (MX)
          acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, av),
                                                           __builtin_bit_cast(bf16x8v, bv),
                                                           acc[ni], 0, 0, 0);
        else
          acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8v, av),
                                                          __builtin_bit_cast(half8v, bv), acc[ni],
                                                          0, 0, 0);
      }
    }
  }
  if (units) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[ni][q] = apply_scale(os, acc[ni][q]);
  }
}

template <bool MX, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t N = g.N;
  const int K = g.K;
  const int nbn = (int)((N + SN - 1) / SN);
  const int mt = blockIdx.x / nbn, nt = blockIdx.x % nbn;
  if (mt >= g.ntiles_dev[0]) return;
  const int4 t = ((const int4*)g.tiles)[mt];
  const int e = t.x;
  const int64_t m0 = t.y, m_end = t.z;
  const int64_t c0 = (int64_t)nt * SN + wave * 64;   // first output column of this wave
  if (c0 >= N) return;                                // no barriers below: waves are independent

  const int64_t cstride = K / 2, sstride = MX ? K / 32 : K / 16;
  const int64_t r = m0 + l32;
  const bool rok = r < m_end;
  const int64_t arow = rok ? (g.a_rows ? (int64_t)g.a_rows[r] : r) : 0;
  const uint8_t* const ac = g.a_codes + arow * cstride;
  const uint8_t* const as = g.a_scales + arow * sstride;
  const uint8_t* bc[2];
  const uint8_t* bs[2];
  bool cok[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int64_t col = c0 + ni * 32 + l32;
    cok[ni] = col < N;
    bc[ni] = g.w_codes + ((int64_t)e * N + (cok[ni] ? col : 0)) * cstride;
    bs[ni] = g.w_scales + ((int64_t)e * N + (cok[ni] ? col : 0)) * sstride;
  }

  // NVFP4 scale bytes 4h .. 4h + 3 of a chunk as two 16-bit loads (rows are
  // only 2-byte aligned when K % 64 != 0); blocks past K read as zero
  auto scales4 = [&](const uint8_t* sp, int k0) -> uint32_t {
    const int left = K - (k0 + 64 * h);   // channels of this lane's half still inside K
    const uint32_t lo = left >= 32 ? *(const uint16_t*)(sp + k0 / 16 + 4 * h) : 0u;
    const uint32_t hi = left >= 64 ? *(const uint16_t*)(sp + k0 / 16 + 4 * h + 2) : 0u;
    return lo | (hi << 16);
  };
  auto load = [&](SkinnyChunk& c, int k0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // NVFP4: piece 2h + s (channels k0 + 32 (2h + s) ..).  MXFP4: step s,
      // block h (channels k0 + 64 s + 32 h ..): piece 2s + h
      const int piece = MX ? 2 * s + h : 2 * h + s;
      const bool kin = k0 + 32 * piece < K;
      c.a[s] = (rok && kin) ? *(const uint4*)(ac + k0 / 2 + 16 * piece) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        c.b[ni][s] = (cok[ni] && kin) ? *(const uint4*)(bc[ni] + k0 / 2 + 16 * piece)
                                      : make_uint4(0, 0, 0, 0);
    }
    if constexpr (MX) {
      // E8M0 bytes of blocks (k0 / 32) + h and + 2 + h, byte s of the word
      uint32_t sa = 0, sb0 = 0, sb1 = 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int blk = k0 / 32 + 2 * s + h;
        if (blk * 32 < K) {
          if (rok) sa |= (uint32_t)as[blk] << (8 * s);
          if (cok[0]) sb0 |= (uint32_t)bs[0][blk] << (8 * s);
          if (cok[1]) sb1 |= (uint32_t)bs[1][blk] << (8 * s);
        }
      }
      c.sa = sa;
      c.sb[0] = sb0;
      c.sb[1] = sb1;
    } else {
      c.sa = rok ? scales4(as, k0) : 0u;
      c.sb[0] = cok[0] ? scales4(bs[0], k0) : 0u;
      c.sb[1] = cok[1] ? scales4(bs[1], k0) : 0u;
    }
  };

  f32x16v acc[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[ni][q] = 0.0f;

  auto compute = [&](const SkinnyChunk& c) {
    if constexpr (MX) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const i32x8v af = {(int)c.a[s].x, (int)c.a[s].y, (int)c.a[s].z, (int)c.a[s].w, 0, 0, 0, 0};
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const i32x8v bf = {(int)c.b[ni][s].x, (int)c.b[ni][s].y, (int)c.b[ni][s].z,
                             (int)c.b[ni][s].w, 0, 0, 0, 0};
          acc[ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af, bf, acc[ni], 4, 4, 0, (int)((c.sa >> (8 * s)) & 255u), 0,
              (int)((c.sb[ni] >> (8 * s)) & 255u));
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // piece 2h + s holds blocks 4h + 2s and 4h + 2s + 1: bytes 2s, 2s + 1
        const uint32_t pa = c.sa >> (16 * s), pb0 = c.sb[0] >> (16 * s), pb1 = c.sb[1] >> (16 * s);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const half8v af = decode8_s(word_s(c.a[s], j), e4m3_dup_f16_s(pa, j >= 2));
          const half8v b0 = decode8_s(word_s(c.b[0][s], j), e4m3_dup_f16_s(pb0, j >= 2));
          const half8v b1 = decode8_s(word_s(c.b[1][s], j), e4m3_dup_f16_s(pb1, j >= 2));
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b0, acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b1, acc[1], 0, 0, 0);
        }
      }
    }
  };

  // the next chunk loads while the current one is computed (two register
  // sets); occupancy hides the rest of the memory latency
  SkinnyChunk cA, cB;
  load(cA, 0);
  for (int k0 = 0;;) {
    if (k0 + CK < K) load(cB, k0 + CK);
    compute(cA);
    k0 += CK;
    if (k0 >= K) break;
    if (k0 + CK < K) load(cA, k0 + CK);
    compute(cB);
    k0 += CK;
    if (k0 >= K) break;
  }

  skinny_tail<MX>(g, acc, e, arow, rok, cok, c0, l32, h);

  // accumulator element q of lane l: row 8 (q / 4) + 4 (l / 32) + q % 4, column l % 32
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int64_t row = m0 + 8 * (q >> 2) + 4 * h + (q & 3);
    if (row >= m_end) continue;
    if constexpr (EPI == kEpiSwiGLU) {
      // packed W13: columns c0 .. c0 + 31 gate, c0 + 32 .. c0 + 63 up
      const float gv = acc[0][q], uv = acc[1][q];
      const float hv = gv / (1.0f + __expf(-gv)) * uv;
      ((uint16_t*)g.Y)[row * g.ldy + c0 / 2 + l32] = (uint16_t)f32_to_bf16_rne(hv);
    } else {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t col = c0 + ni * 32 + l32;
        if (col >= N) continue;
        if (g.y_bf16)
          ((uint16_t*)g.Y)[row * g.ldy + col] = (uint16_t)f32_to_bf16_rne(acc[ni][q]);
        else
          ((float*)g.Y)[row * g.ldy + col] = acc[ni][q];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same tiles with the operands staged through LDS, three stages filled
// straight from global memory (global_load_lds, four lanes per 64-byte row
// chunk, so every load is fully coalesced) two chunks ahead.  Each wave fills
// its own weight region of a stage (its 64 W rows); the tile's activation
// rows are shared: waves 0 and 1 load the 32 code rows, waves 2 and 3 the
// scales, and one barrier per chunk makes them visible to every wave.  A
// stage is 20.3 KB, so two workgroups fit in a CU's LDS and two waves share
// each SIMD, hiding each other's memory waits.  Needs K % 64 == 0 (NVFP4) or
// K % 128 == 0 (MXFP4: 4-byte scale rows per chunk).
typedef const void __attribute__((address_space(1)))* sk_gptr_t;
typedef void __attribute__((address_space(3)))* sk_lptr_t;

// Stage layout: per wave, 64 W rows x 64 B of codes, then their scales: raw
// (64 x 8 B E4M3, or 64 x 4 B E8M0) or, with WREC, the weights' tiled fp16
// scale records (64 x 16 B); then the shared activation rows (32 x 64 B) and
// their raw scales (32 x 8 B, or 32 x 4 B and copies).
constexpr int SW_CODE = 0;
constexpr int SW_SC = 4096;
template <bool WREC> constexpr int SWREGION = WREC ? 5120 : 4608;   // bytes per wave per stage
template <bool WREC> constexpr int SA_CODE = 4 * SWREGION<WREC>;
template <bool WREC> constexpr int SA_SC = SA_CODE<WREC> + 2048;
template <bool WREC> constexpr int SSTAGE = SA_SC<WREC> + 256;      // 20736 or 22784 bytes

__device__ __forceinline__ int sk_swz(int row, int piece) {
  return row * 64 + ((piece ^ ((row >> 1) ^ (row >> 2)) & 3) << 4);
}

constexpr int sk_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Direct compensation (g.w_hi_t): Y = s_A s_W sum + R W_S^T with the plain
// bf16 residual R and the selected weight columns read here from W_hi^T
// ([K][batch][N] bf16, channel-major interleaved: the 64 columns a wave
// owns are 128 contiguous bytes of each selected channel's row), so no
// gathered W_S is written and read back.  64 channels a pass: each wave
// brings its rows into its own LDS region (`region`, 8 blocks of 8 rows x
// 128 B, block pitch 1088 B so that the two lane halves, which read blocks
// i and i + 1, hit disjoint banks) with eight global -> LDS loads, then reads
// each lane's eight consecutive channels of one column (the bf16 MFMA's B
// operand) out of it.  Padding channels (t >= sel_k) load a valid row; R is
// zero there.  Needs N % 8 == 0.
constexpr int SKD_BLOCK = 1088;
template <bool MX>
__device__ __forceinline__ void skinny_tail_direct(const GemmArgs& g, f32x16v (&acc)[2], int e,
                                                   int64_t ar, bool rok, int64_t c0, int lane,
                                                   uint8_t* region) {
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t N = g.N;
  if constexpr (!MX) {
    const OutScale os = g.a_ts ? out_scale(g.a_ts[0], g.w_ts[e]) : OutScale{1.0f, 0, false};
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[ni][q] = apply_scale(os, acc[ni][q]);
  }
  const uint16_t* rrow = g.r_res + ar * g.ld_r + 8 * h;
  // this lane's 16-byte piece of each row: columns c0 + 8 p .. + 7, p = lane % 8
  // (pieces past N read the last piece of the row again; never stored)
  const int64_t col = min(c0 + 8 * (lane & 7), N - 8);
  const int64_t rstride = g.w_hi_batch * N;
  const uint16_t* const wbase = g.w_hi_t + (int64_t)e * N + col;
  const int Kc = g.K;
  for (int t0 = 0; t0 < g.kp; t0 += 64) {
    const int nb = min(8, (g.kp - t0) >> 3);   // blocks of 8 channels this pass (4 or 8)
    // the previous pass's LDS reads are complete before its rows are replaced
    // (s_waitcnt lgkmcnt(0), the other counters left alone)
    if (t0 > 0) __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nb) {
        const int t = t0 + 8 * i + (lane >> 3);
        int c = g.sel[min(t, g.sel_k - 1)];
        c = c < 0 ? 0 : (c >= Kc ? Kc - 1 : c);
        __builtin_amdgcn_global_load_lds((sk_gptr_t)(wbase + (int64_t)c * rstride),
                                         (sk_lptr_t)(region + i * SKD_BLOCK), 16, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(sk_vmcnt(0));
    for (int kt = 0; kt < nb * 8; kt += 16) {
      const uint4 av = rok ? *(const uint4*)(rrow + t0 + kt) : make_uint4(0, 0, 0, 0);
      // lane half h takes channels kt + 8 h .. + 7: block kt / 8 + h, rows 0..7
      const uint8_t* const blk = region + (kt / 8 + h) * SKD_BLOCK;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const uint16_t* const p = (const uint16_t*)(blk + (ni * 32 + l32) * 2);
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)p[(2 * q) * 64] | ((uint32_t)p[(2 * q + 1) * 64] << 16);
        const uint4 bv = make_uint4(w[0], w[1], w[2], w[3]);
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, av),
                                                         __builtin_bit_cast(bf16x8v, bv), acc[ni],
                                                         0, 0, 0);
      }
    }
  }
}

// (the LDS kernels keep each weight row's offset from the expert's first row
// in 32 bits)
bool skinny_lds_path(const GemmArgs& g) {
  return (g.mx ? g.K % 128 == 0 : g.K % 64 == 0) && g.N * (int64_t)(g.K / 2) <= 0xffffffffLL;
}
static_assert(2 * 8 * SKD_BLOCK <= 20736, "direct compensation regions exceed a stage");

// WREC (K % 128 == 0): the weight scales come from records, [E][K / 128]
// [w_rows_pad][record], so that a wave's 64 rows of one chunk are one
// contiguous, coalesced piece.  WREC 1 (g.w_scales_t): NVFP4 the tiled fp16
// records (16 B, swizzled by row, already widened to fp16), MXFP4 the four
// E8M0 bytes of the chunk (4 B).  WREC 2 (g.w_rec8, NVFP4): the raw E4M3
// bytes of the chunk (8 B; half the bytes of the fp16 records, widened in
// the decode like raw scales).
template <bool MX, int EPI, int WREC = 0>
__global__ __launch_bounds__(256, 2) void gemm_skinny_lds_kernel(GemmArgs g) {
  static_assert(WREC != 2 || !MX, "E4M3 records are NVFP4");
  constexpr int DMA = MX ? 6 : (WREC == 1 ? 6 : 7);   // global -> LDS loads per wave per chunk
  constexpr bool FP16REC = WREC == 1 && !MX;           // fp16 records in a 1 KB region
  constexpr int SWR = SWREGION<FP16REC>, SAC = SA_CODE<FP16REC>, SAS = SA_SC<FP16REC>;
  constexpr int REC_SHIFT = MX ? 2 : (WREC == 2 ? 3 : 4);   // log2 of the record size
  __shared__ __attribute__((aligned(16))) uint8_t st0[SSTAGE<FP16REC>];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SSTAGE<FP16REC>];
  __shared__ __attribute__((aligned(16))) uint8_t st2[SSTAGE<FP16REC>];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t N = g.N;
  const int K = g.K;
  const int nk = (K + CK - 1) / CK;
  const int nbn = (int)((N + SN - 1) / SN);
  const int mt = blockIdx.x / nbn, nt = blockIdx.x % nbn;
  if (mt >= g.ntiles_dev[0]) return;        // uniform over the workgroup
  const int4 t = ((const int4*)g.tiles)[mt];
  const int e = t.x;
  const int64_t m0 = t.y, m_end = t.z;
  // (a wave whose columns are all past N still runs: it loads its share of
  // the activations and takes part in the barriers, and stores nothing)
  const int64_t c0 = (int64_t)nt * SN + wave * 64;
  const int reg = wave * SWR;

  const int64_t cstride = K / 2, sstride = MX ? K / 32 : K / 16;
  const uint8_t* const wcb = g.w_codes + (int64_t)e * N * cstride;
  const uint8_t* const wsb = g.w_scales + (int64_t)e * N * sstride;
  // rows past the tile (or past N) read a valid row again (their results are
  // never stored)
  auto wrow = [&](int r) -> int64_t { return min(c0 + r, N - 1); };
  auto arow_of = [&](int r) -> int64_t {
    const int64_t rr = min(m0 + r, m_end - 1);
    return g.a_rows ? (int64_t)g.a_rows[rr] : rr;
  };
  // per-lane global offsets of this wave's weight loads (row and swizzled piece)
  uint32_t wco[4];
  int wpiece[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 16 * it + (lane >> 2);
    wpiece[it] = (lane & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
    wco[it] = (uint32_t)(wrow(row) * cstride);
  }
  const uint8_t* wsrc[2];
  // WREC: this wave's 64 records of chunk 0 (rows c0 .. c0 + 63 exist in the
  // padded record block even past N)
  const uint8_t* wrec = nullptr;
  if constexpr (WREC == 1)
    wrec = g.w_scales_t + (((int64_t)e * nk * g.w_rows_pad + c0 + lane) << REC_SHIFT);
  else if constexpr (WREC == 2)   // lane l loads dword l % 2 of row c0 + l / 2 (rows 0..31)
    wrec = g.w_rec8 + (((int64_t)e * nk * g.w_rows_pad + c0) << REC_SHIFT) + 4 * lane;
  if constexpr (MX) {
    wsrc[0] = wsb + wrow(lane) * sstride;
    wsrc[1] = wsrc[0];
  } else {
#pragma unroll
    for (int it = 0; it < 2; ++it) wsrc[it] = wsb + wrow(32 * it + (lane >> 1)) * sstride + 4 * (lane & 1);
  }
  // this wave's share of the activation loads: waves 0 and 1 the code rows
  // 16 w .. 16 w + 15, waves 2 and 3 the scale records (the same bytes)
  const int arow = 16 * (wave & 1) + (lane >> 2);
  const int apiece = (lane & 3) ^ (((arow >> 1) ^ (arow >> 2)) & 3);
  const uint8_t* const acsrc = g.a_codes + arow_of(arow) * cstride;
  const uint8_t* asrc;
  if constexpr (MX) asrc = g.a_scales + arow_of(lane & 31) * sstride;
  else asrc = g.a_scales + arow_of(lane >> 1) * sstride + 4 * (lane & 1);

  // chunk c (clamped: past the end, the last chunk again into a stage nobody reads)
  auto issue = [&](int c, uint8_t* const sb) {
    const int cc = min(c, nk - 1);
    const int k0 = cc * CK;
    uint8_t* const base = sb + reg;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      // pieces past K (K % 128 == 64) read the chunk's first half again
      const int pc = (k0 + 32 * wpiece[it] < K) ? wpiece[it] : (wpiece[it] & 1);
      __builtin_amdgcn_global_load_lds((sk_gptr_t)(wcb + wco[it] + k0 / 2 + 16 * pc),
                                       (sk_lptr_t)(base + SW_CODE + it * 1024), 16, 0, 0);
    }
    if constexpr (WREC == 1 && MX) {
      __builtin_amdgcn_global_load_lds(
          (sk_gptr_t)(wrec + ((int64_t)cc * g.w_rows_pad << REC_SHIFT)), (sk_lptr_t)(base + SW_SC),
          4, 0, 0);
    } else if constexpr (WREC == 2) {
      // rows 0..31, then rows 32..63: 256 contiguous bytes each, the raw
      // scales' LDS layout (8 bytes per row)
#pragma unroll
      for (int it = 0; it < 2; ++it)
        __builtin_amdgcn_global_load_lds(
            (sk_gptr_t)(wrec + ((int64_t)cc * g.w_rows_pad << REC_SHIFT) + 256 * it),
            (sk_lptr_t)(base + SW_SC + it * 256), 4, 0, 0);
    } else if constexpr (WREC) {
      __builtin_amdgcn_global_load_lds(
          (sk_gptr_t)(wrec + ((int64_t)cc * g.w_rows_pad << REC_SHIFT)), (sk_lptr_t)(base + SW_SC),
          16, 0, 0);
    } else if constexpr (MX) {
      __builtin_amdgcn_global_load_lds((sk_gptr_t)(wsrc[0] + k0 / 32),
                                       (sk_lptr_t)(base + SW_SC), 4, 0, 0);
    } else {
      // second dword (blocks 4..7) past K reads the first again
      const int dw = (k0 + 64 < K) ? 1 : 0;
#pragma unroll
      for (int it = 0; it < 2; ++it)
        __builtin_amdgcn_global_load_lds(
            (sk_gptr_t)(wsrc[it] + k0 / 16 - 4 * (lane & 1) + 4 * ((lane & 1) & dw)),
            (sk_lptr_t)(base + SW_SC + it * 256), 4, 0, 0);
    }
    if (wave < 2) {
      const int pc = (k0 + 32 * apiece < K) ? apiece : (apiece & 1);
      __builtin_amdgcn_global_load_lds((sk_gptr_t)(acsrc + k0 / 2 + 16 * pc),
                                       (sk_lptr_t)(sb + SAC + (wave & 1) * 1024), 16, 0, 0);
    } else if constexpr (MX) {
      __builtin_amdgcn_global_load_lds((sk_gptr_t)(asrc + k0 / 32), (sk_lptr_t)(sb + SAS), 4, 0,
                                       0);
    } else {
      const int dw = (k0 + 64 < K) ? 1 : 0;
      __builtin_amdgcn_global_load_lds(
          (sk_gptr_t)(asrc + k0 / 16 - 4 * (lane & 1) + 4 * ((lane & 1) & dw)),
          (sk_lptr_t)(sb + SAS), 4, 0, 0);
    }
  };

  f32x16v acc[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[ni][q] = 0.0f;

  // (WREC: wb[ni][s] = the fp16 scale pair of blocks 4h + 2s, 4h + 2s + 1 of
  // W row ni)
  uint32_t wb[2][2] = {{0u, 0u}, {0u, 0u}};
  auto compute = [&](const SkinnyChunk& c) {
    if constexpr (MX) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const i32x8v af = {(int)c.a[s].x, (int)c.a[s].y, (int)c.a[s].z, (int)c.a[s].w, 0, 0, 0, 0};
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const i32x8v bf = {(int)c.b[ni][s].x, (int)c.b[ni][s].y, (int)c.b[ni][s].z,
                             (int)c.b[ni][s].w, 0, 0, 0, 0};
          acc[ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af, bf, acc[ni], 4, 4, 0, (int)((c.sa >> (8 * s)) & 255u), 0,
              (int)((c.sb[ni] >> (8 * s)) & 255u));
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // piece 2h + s holds blocks 4h + 2s and 4h + 2s + 1: bytes 2s, 2s + 1
        const uint32_t pa = c.sa >> (16 * s), pb0 = c.sb[0] >> (16 * s), pb1 = c.sb[1] >> (16 * s);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const half8v af = decode8_s(word_s(c.a[s], j), e4m3_dup_f16_s(pa, j >= 2));
          uint32_t d0, d1;
          if constexpr (FP16REC) {   // fp16 pair: the block's half in both halves
            d0 = __builtin_amdgcn_perm(wb[0][s], wb[0][s], j >= 2 ? 0x03020302u : 0x01000100u);
            d1 = __builtin_amdgcn_perm(wb[1][s], wb[1][s], j >= 2 ? 0x03020302u : 0x01000100u);
          } else {
            d0 = e4m3_dup_f16_s(pb0, j >= 2);
            d1 = e4m3_dup_f16_s(pb1, j >= 2);
          }
          const half8v b0 = decode8_s(word_s(c.b[0][s], j), d0);
          const half8v b1 = decode8_s(word_s(c.b[1][s], j), d1);
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b0, acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b1, acc[1], 0, 0, 0);
        }
      }
    }
  };

  // one chunk from stage sb: its loads (every wave's) have landed after the
  // wait and the barrier; fragments, then the loads of chunk c + 2 into stage
  // nx (last read in the previous chunk, which every wave has finished: it
  // passed the barrier), then the MFMAs
  auto step = [&](int c, const uint8_t* const sb, uint8_t* const nx) {
    __builtin_amdgcn_s_waitcnt(sk_vmcnt(DMA));
    __builtin_amdgcn_s_barrier();
    const uint8_t* const base = sb + reg;
    const int k0 = c * CK;
    SkinnyChunk f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int piece = MX ? 2 * s + h : 2 * h + s;
      const uint4 a = *(const uint4*)(sb + SAC + sk_swz(l32, piece));
      const uint4 b0 = *(const uint4*)(base + SW_CODE + sk_swz(l32, piece));
      const uint4 b1 = *(const uint4*)(base + SW_CODE + sk_swz(32 + l32, piece));
      if constexpr (WREC) {   // K % 128 == 0: every piece is inside K
        f.a[s] = a;
        f.b[0][s] = b0;
        f.b[1][s] = b1;
      } else {
        const bool kin = k0 + 32 * piece < K;
        const uint4 z = make_uint4(0, 0, 0, 0);
        f.a[s] = kin ? a : z;
        f.b[0][s] = kin ? b0 : z;
        f.b[1][s] = kin ? b1 : z;
      }
    }
    if constexpr (MX) {
      // E8M0 of blocks 2s + h: bytes of the row's 4-byte record; 127 (= 1.0)
      // where the block is past K
      const uint32_t ra = *(const uint32_t*)(sb + SAS + l32 * 4);
      const uint32_t rb0 = *(const uint32_t*)(base + SW_SC + l32 * 4);
      const uint32_t rb1 = *(const uint32_t*)(base + SW_SC + (32 + l32) * 4);
      uint32_t sa = 0, sb0 = 0, sb1 = 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int bi = 2 * s + h;
        const bool kin = k0 + 32 * bi < K;
        sa |= (kin ? (ra >> (8 * bi)) & 255u : 127u) << (8 * s);
        sb0 |= (kin ? (rb0 >> (8 * bi)) & 255u : 127u) << (8 * s);
        sb1 |= (kin ? (rb1 >> (8 * bi)) & 255u : 127u) << (8 * s);
      }
      f.sa = sa;
      f.sb[0] = sb0;
      f.sb[1] = sb1;
    } else if constexpr (FP16REC) {
      f.sa = *(const uint32_t*)(sb + SAS + l32 * 8 + 4 * h);
      // record dword d (blocks 2d, 2d + 1) of row r sits at d ^ ((r / 8) % 4);
      // rows l and 32 + l share that swizzle
      const int q = (l32 >> 3) & 3;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int slot = (2 * h + s) ^ q;
        wb[0][s] = *(const uint32_t*)(base + SW_SC + l32 * 16 + slot * 4);
        wb[1][s] = *(const uint32_t*)(base + SW_SC + (32 + l32) * 16 + slot * 4);
      }
    } else {
      f.sa = *(const uint32_t*)(sb + SAS + l32 * 8 + 4 * h);
      f.sb[0] = *(const uint32_t*)(base + SW_SC + l32 * 8 + 4 * h);
      f.sb[1] = *(const uint32_t*)(base + SW_SC + (32 + l32) * 8 + 4 * h);
    }
    issue(c + 2, nx);
    compute(f);
  };
  issue(0, st0);
  issue(1, st1);
  int kc = 0;
  for (; kc < nk; kc += 3) {
    step(kc, st0, st2);
    if (kc + 1 >= nk) break;
    step(kc + 1, st1, st0);
    if (kc + 2 >= nk) break;
    step(kc + 2, st2, st1);
  }
  __builtin_amdgcn_s_waitcnt(sk_vmcnt(0));

  const int64_t r = m0 + l32;
  const bool rok = r < m_end;
  const int64_t ar = rok ? (g.a_rows ? (int64_t)g.a_rows[r] : r) : 0;
  bool cok[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) cok[ni] = c0 + ni * 32 + l32 < N;

  if (g.w_hi_t && g.kp > 0 && g.r_res) {
    // the stages are free once every wave's loads into them (the clamped
    // ones of the last two steps included) have landed: waves 0 and 1 take
    // stage 0 for their compensation rows, waves 2 and 3 stage 1
    __syncthreads();
    uint8_t* const region = (wave < 2 ? st0 : st1) + (wave & 1) * (8 * SKD_BLOCK);
    skinny_tail_direct<MX>(g, acc, e, ar, rok, c0, lane, region);
  } else {
    skinny_tail<MX>(g, acc, e, ar, rok, cok, c0, l32, h);
  }

  // accumulator element q of lane l: row 8 (q / 4) + 4 (l / 32) + q % 4, column l % 32
  if (c0 >= N) return;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int64_t row = m0 + 8 * (q >> 2) + 4 * h + (q & 3);
    if (row >= m_end) continue;
    if constexpr (EPI == kEpiSwiGLU) {
      // packed W13: columns c0 .. c0 + 31 gate, c0 + 32 .. c0 + 63 up
      const float gv = acc[0][q], uv = acc[1][q];
      const float hv = gv / (1.0f + __expf(-gv)) * uv;
      ((uint16_t*)g.Y)[row * g.ldy + c0 / 2 + l32] = (uint16_t)f32_to_bf16_rne(hv);
    } else {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t col = c0 + ni * 32 + l32;
        if (col >= N) continue;
        if (g.y_bf16)
          ((uint16_t*)g.Y)[row * g.ldy + col] = (uint16_t)f32_to_bf16_rne(acc[ni][q]);
        else
          ((float*)g.Y)[row * g.ldy + col] = acc[ni][q];
      }
    }
  }
}

// raw E4M3 scale records: out[b][c][r] = the 8 scale bytes of row r's
// blocks 8 c .. 8 c + 7 (zero past `rows`); one 8-byte record per thread
__global__ __launch_bounds__(256) void e4m3_scale_records_kernel(const uint8_t* __restrict__ sc,
                                                                 int64_t batch, int64_t rows,
                                                                 int32_t K, int64_t rows_pad,
                                                                 uint2* __restrict__ out) {
  const int64_t nk = K / 128, per = nk * rows_pad;
  const int64_t total = batch * per;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / per, rem = i - b * per;
    const int64_t c = rem / rows_pad, r = rem - c * rows_pad;
    out[i] = r < rows ? *(const uint2*)(sc + (b * rows + r) * (K / 16) + 8 * c) : make_uint2(0, 0);
  }
}

}  // namespace

hipError_t launch_e4m3_scale_records(const uint8_t* scales, int64_t batch, int64_t rows, int32_t K,
                                     int64_t rows_pad, uint8_t* out, hipStream_t stream) {
  const int64_t total = batch * (K / 128) * rows_pad;
  if (total == 0) return hipSuccess;
  const int64_t nb = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(e4m3_scale_records_kernel, dim3((unsigned)nb), dim3(256), 0, stream, scales,
                     batch, rows, K, rows_pad, (uint2*)out);
  return hipGetLastError();
}

bool skinny_direct_ok(bool mx, int64_t K, int64_t N) {
  return (mx ? K % 128 == 0 : K % 64 == 0) && N * (K / 2) <= 0xffffffffLL && N % 8 == 0;
}

hipError_t launch_skinny_gemm(const GemmArgs& g, int64_t max_tiles, hipStream_t stream) {
  // direct compensation only on the LDS kernels (checked by the caller with
  // skinny_direct_ok; refused here rather than read out of bounds)
  if (g.w_hi_t && g.kp > 0 && !skinny_direct_ok(g.mx, g.K, g.N)) return hipErrorInvalidValue;
  const int64_t nbn = (g.N + SN - 1) / SN;
  const int64_t nb = max_tiles * nbn;
  if (nb == 0) return hipSuccess;
  const dim3 grid((unsigned)nb), block(256);
  if (!g.mx && g.w_rec8 && g.K % 128 == 0 && skinny_lds_path(g)) {
    if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((gemm_skinny_lds_kernel<false, kEpiSwiGLU, 2>), grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_skinny_lds_kernel<false, kEpiStore, 2>), grid, block, 0, stream, g);
    return hipGetLastError();
  }
  if (g.w_scales_t && g.K % 128 == 0 && skinny_lds_path(g)) {
    if (g.mx) {
      if (g.epilogue == kEpiSwiGLU)
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<true, kEpiSwiGLU, 1>), grid, block, 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<true, kEpiStore, 1>), grid, block, 0, stream, g);
    } else {
      if (g.epilogue == kEpiSwiGLU)
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<false, kEpiSwiGLU, 1>), grid, block, 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<false, kEpiStore, 1>), grid, block, 0, stream, g);
    }
    return hipGetLastError();
  }
  if (skinny_lds_path(g)) {
    if (g.mx) {
      if (g.epilogue == kEpiSwiGLU)
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<true, kEpiSwiGLU>), grid, block, 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<true, kEpiStore>), grid, block, 0, stream, g);
    } else {
      if (g.epilogue == kEpiSwiGLU)
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<false, kEpiSwiGLU>), grid, block, 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_skinny_lds_kernel<false, kEpiStore>), grid, block, 0, stream, g);
    }
    return hipGetLastError();
  }
  if (g.mx) {
    if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, kEpiSwiGLU>), grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<true, kEpiStore>), grid, block, 0, stream, g);
  } else {
    if (g.epilogue == kEpiSwiGLU)
      hipLaunchKernelGGL((gemm_skinny_kernel<false, kEpiSwiGLU>), grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, kEpiStore>), grid, block, 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace q4
