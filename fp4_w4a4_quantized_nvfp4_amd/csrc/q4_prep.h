// Operand preparation for the W4A4 + RAC GEMM (gfx950): the residual gather
// R, the selected weight columns W_S and the tiled fp16 scale records, as
// device bodies that take their block index, so that the stand-alone kernels
// and the one-launch preparation of a dense GEMM share them.
//
// QUADS (arXiv 2607.15810) section 3.3: Eq. 21 (residual of the selected
// channels, multiplied by the matching high-precision weight columns),
// Eq. 24 (the selected channel set S).
#pragma once

#include "q4_device.h"

namespace q4 {

// the four dwords of a 16-byte scale record in swizzled order for row `row`:
// dword d sits at d ^ ((row / 8) % 4), so that 32 consecutive rows reading the
// same dword hit distinct LDS banks
__device__ __forceinline__ uint4 swz_sc_rec(uint4 v, int row) {
  const int q = (row >> 3) & 3;
  uint4 r;
  r.x = q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
  r.y = q == 0 ? v.y : (q == 1 ? v.x : (q == 2 ? v.w : v.z));
  r.z = q == 0 ? v.z : (q == 1 ? v.w : (q == 2 ? v.x : v.y));
  r.w = q == 0 ? v.w : (q == 1 ? v.z : (q == 2 ? v.y : v.x));
  return r;
}

// Whether the channel set holds k ascending, unique channels in [0, cols).
// Every thread of the workgroup must call it (it ends in a workgroup-wide
// reduction).  A kernel that finds the set invalid gathers nothing (k taken as
// 0, so the compensation adds zero) and reports Q4_EINVAL in its status word.
__device__ __forceinline__ bool chan_set_ok(const int32_t* __restrict__ idx, int32_t k,
                                            int64_t cols) {
  int bad = 0;
  for (int t = threadIdx.x; t < k; t += blockDim.x) {
    const int32_t c = idx[t];
    bad |= (c < 0) | ((int64_t)c >= cols) | (t > 0 && idx[t - 1] >= c);
  }
  return __syncthreads_or(bad) == 0;
}

// R[i][t] = bf16(RN32(x[i][S_t] - dequant)) for t < k, 0 for k <= t < ld_r.
// UNITS (NVFP4 GEMM operand): the same bf16 value times 2^-e, s_t = f 2^e
// (f in [0.5, 1)), as fp16 bits -- exact (an 8-bit mantissa fits fp16's 11)
// unless the scaled value is an fp16 subnormal; the compensation is then in
// the units of the W4A4 sum once the weight side carries 1 / (f s_W).
// One thread per (4 consecutive rows, t), t fastest across lanes: S is
// ascending and its channels cluster in a few blocks (the outlier blocks), so
// one load instruction of a wave touches few cache lines, and each row's
// stores are contiguous.  The twelve loads of a thread are issued before any
// is used.  Items: residual_gather_items(rows, ld_r); block `blk` of `nblk`
// (grid-stride).
__host__ __device__ inline int64_t residual_gather_items(int64_t rows, int64_t ld_r) {
  return (rows + 3) / 4 * ld_r;
}

template <bool MX, bool UNITS = false>
__device__ __forceinline__ void residual_gather_part(
    const uint16_t* __restrict__ x, int64_t rows, int32_t cols, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ ts,
    const int32_t* __restrict__ idx, int32_t k, uint16_t* __restrict__ R, int64_t ld_r,
    int64_t blk, int64_t nblk) {
  const int64_t total = residual_gather_items(rows, ld_r);
  const float st = MX ? 1.0f : ts[0];
  int est = 0;
  if (UNITS && !MX) (void)frexpf(st, &est);
  const int64_t cst = cols / 2, sst = MX ? cols / 32 : cols / 16;
  for (int64_t g = blk * 256 + threadIdx.x; g < total; g += nblk * 256) {
    const int64_t i0 = g / ld_r * 4;
    const int t = (int)(g - g / ld_r * ld_r);
    int c = t < k ? idx[t] : 0;
    c = c < 0 ? 0 : (c >= cols ? cols - 1 : c);
    uint16_t xv[4];
    uint8_t cb[4], sb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + q < rows ? i0 + q : rows - 1;
      xv[q] = x[i * cols + c];
      cb[q] = codes[i * cst + (c >> 1)];
      sb[q] = scales[i * sst + (c >> (MX ? 5 : 4))];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q >= rows) break;
      uint32_t out = 0;
      if (t < k) {
        const uint32_t nib = (cb[q] >> ((c & 1) * 4)) & 15u;
        float s;
        if constexpr (MX) {
          const int e = (int)sb[q] - 127;
          s = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : 0x1p-127f;
        } else {
          s = e4m3_to_f32(sb[q]);
        }
        out = f32_to_bf16_rne(fmaf(-(e2m1_value(nib) * s), st, bf16_to_f32(xv[q])));
        if (UNITS && !MX)
          out = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(__uint_as_float(out << 16), -est));
      }
      R[(i0 + q) * ld_r + t] = (uint16_t)out;
    }
  }
}

// 1 / (s_W f_A) for s_A = f_A 2^e_A, f_A in [0.5, 1): the factor that takes a
// selected weight column to the units of the W4A4 sum
__device__ __forceinline__ float wsel_scale_inv(float w_ts, float a_ts) {
  int ea;
  return 1.0f / (w_ts * frexpf(a_ts, &ea));
}

// W_S[b][j][t] = W_hi^T of matrix b at (S_t, j) for t < k, 0 for k <= t < kp:
// a transposing gather through a 64 x 64 LDS tile (the selected rows are
// contiguous in j).  W_hi^T of `batch` matrices is laid out channel-major,
// [K][batch][N] (one matrix: [K][N]): the batch's rows of one selected
// channel are contiguous, so a gather reads 64 contiguous runs rather than
// 64 rows scattered over every matrix.
// With `w_ts` (NVFP4 GEMM operand, the weights' tensor scales, one per matrix
// b) and `a_ts` (the activation's tensor scale, s_A = f 2^e): the value
// w / (s_W[b] f), formed as w times the fp32 reciprocal of s_W[b] f (within
// 2^-23 of the quotient) and rounded to fp16 (relative 2^-11), so that the
// compensation R W_S^T comes in the units of the W4A4 sum.  (wsel_scale_inv
// gives that reciprocal; every reader of W_S forms it the same way.)
// Tile (bx, by) of matrix b covers j in [64 bx, 64 bx + 64), t in [64 by, 64 by + 64).
__device__ __forceinline__ void wsel_gather_part(const uint16_t* __restrict__ w_hi_t, int64_t K,
                                                 int64_t N, int64_t batch,
                                                 const int32_t* __restrict__ idx,
                                                 int32_t k, int32_t kp, uint16_t* __restrict__ ws,
                                                 int64_t b, int64_t bx, int by,
                                                 uint16_t (*tile)[66],
                                                 const float* __restrict__ w_ts = nullptr,
                                                 const float* __restrict__ a_ts = nullptr) {
  const int64_t j0 = bx * 64;
  const int t0 = by * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t* src = w_hi_t + b * N;
  int64_t rowoff[16];
  bool ok[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int t = t0 + ty + 4 * q;
    int c = t < k ? idx[t] : 0;
    c = c < 0 ? 0 : (c >= K ? (int)K - 1 : c);
    rowoff[q] = (int64_t)c * batch * N;
    ok[q] = t < k && j0 + tx < N;
  }
  uint16_t v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = ok[q] ? src[rowoff[q] + j0 + tx] : (uint16_t)0;
  if (w_ts) {
    const float rinv = wsel_scale_inv(w_ts[b], a_ts[0]);
#pragma unroll
    for (int q = 0; q < 16; ++q)
      v[q] = __builtin_bit_cast(uint16_t, (_Float16)(bf16_to_f32(v[q]) * rinv));
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) tile[ty + 4 * q][tx] = v[q];
  __syncthreads();
  uint16_t* dst = ws + b * N * kp;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int64_t j = j0 + ty + 4 * q;
    const int t = t0 + tx;
    if (j < N && t < kp) dst[j * kp + t] = tile[tx][ty + 4 * q];
  }
}

// Tiled fp16 scale records of an NVFP4 operand: record (c, r) holds the eight
// E4M3 block scales of row r over K columns [128 c, 128 c + 128) as fp16
// (exact, subnormal scales included), in swz_sc_rec order for r % 256;
// layout [K / 128][rows_pad][16 B], rows past `rows` zero.  Block `blk` of
// `nblk` (grid-stride).
__device__ __forceinline__ void scale_tile_part(const uint8_t* __restrict__ sc, int64_t rows,
                                                int32_t K, int64_t rows_pad,
                                                uint4* __restrict__ out, int64_t blk,
                                                int64_t nblk) {
  const int64_t total = (int64_t)(K / 128) * rows_pad;
  for (int64_t i = blk * 256 + threadIdx.x; i < total; i += nblk * 256) {
    const int64_t c = i / rows_pad, r = i - c * rows_pad;
    uint2 raw = make_uint2(0, 0);
    if (r < rows) raw = *(const uint2*)(sc + r * (K / 16) + 8 * c);
    const half2v k256 = {(_Float16)256.0f, (_Float16)256.0f};
    // the E4M3 byte shifted left by 7 is an fp16 of value 2^-8 times the
    // scale; the multiply by 256 is exact
    const uint32_t d0 = __builtin_amdgcn_perm(0u, raw.x, 0x0c010c00u) << 7;
    const uint32_t d1 = __builtin_amdgcn_perm(0u, raw.x, 0x0c030c02u) << 7;
    const uint32_t d2 = __builtin_amdgcn_perm(0u, raw.y, 0x0c010c00u) << 7;
    const uint32_t d3 = __builtin_amdgcn_perm(0u, raw.y, 0x0c030c02u) << 7;
    const uint4 rec = make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d0) * k256),
                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d1) * k256),
                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d2) * k256),
                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d3) * k256));
    out[i] = swz_sc_rec(rec, (int)(r & 255));
  }
}

}  // namespace q4
