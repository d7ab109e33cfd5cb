// One-launch operand preparation for a dense W4A4 + RAC GEMM (gfx950).
//
// QUADS (arXiv 2607.15810) section 3.3, Eq. 21: before the product, the
// residual of the selected channels (R) and the matching weight columns (W_S)
// are gathered -- for NVFP4 as fp16 operands in the units of the W4A4 sum
// (R = bf16(r) 2^-e_A exactly, W_S = w / (s_W f_A) rounded to fp16, with
// s_A = f_A 2^e_A), so the GEMM adds them to its unscaled sum and applies
// s_A s_W once; MXFP4 keeps bf16 (no tensor scale) -- and the dense 256 x 256
// kernel also reads the NVFP4
// block scales of both operands as tiled fp16 records.  The four jobs are
// small and independent, so one grid runs them side by side: its workgroups
// are split into consecutive ranges, one per job, instead of four launches
// that each drain before the next starts.
#include "q4_internal.h"
#include "q4_prep.h"
#include "../../include/q4rac.h"

namespace q4 {
namespace {

struct PrepArgs {
  // residual gather
  const uint16_t* x;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_ts;
  uint16_t* R;
  // weight-column gather
  const uint16_t* w_hi_t;
  uint16_t* W_S;
  const int32_t* idx;
  // scale records
  const uint8_t* w_scales;
  const float* w_ts;   // NVFP4: R and W_S as fp16 operands in the W4A4 sum's units
  uint4* a_tiles;
  uint4* w_tiles;
  int64_t M, N, a_pad, w_pad;
  int32_t K, k, kp;
  // workgroup ranges, in launch order: W_S tiles, R, A records, W records
  int64_t n_ws, n_r, n_ta, n_tw;
  int64_t ws_gx;  // W_S tiles along N
  int32_t* status;  // optional: Q4_OK, or Q4_EINVAL for an invalid channel set
};

template <bool MX>
__global__ __launch_bounds__(256) void rac_prep_kernel(PrepArgs p) {
  __shared__ uint16_t tile[64][66];
  int64_t b = blockIdx.x;
  // every gathering workgroup checks the whole channel set (at most 1024
  // entries, L2-resident); an invalid set gathers zeros, so the GEMM adds no
  // compensation, and workgroup 0 reports it
  const bool gathers = b < p.n_ws + p.n_r;
  const bool ok = gathers ? chan_set_ok(p.idx, p.k, p.K) : true;
  if (b == 0 && threadIdx.x == 0 && p.status) p.status[0] = ok ? 0 : 1;
  const int32_t k = ok ? p.k : 0;
  if (b < p.n_ws) {
    const int64_t by = b / p.ws_gx;
    wsel_gather_part(p.w_hi_t, p.K, p.N, 1, p.idx, k, p.kp, p.W_S, 0, b - by * p.ws_gx, (int)by,
                     tile, MX ? nullptr : p.w_ts, p.a_ts);
    return;
  }
  b -= p.n_ws;
  if (b < p.n_r) {
    residual_gather_part<MX, true>(p.x, p.M, p.K, p.a_codes, p.a_scales, p.a_ts, p.idx, k, p.R,
                                   p.kp, b, p.n_r);
    return;
  }
  if (b - p.n_r >= p.n_ta + p.n_tw) return;  // the status-only workgroup
  b -= p.n_r;
  if (b < p.n_ta) {
    scale_tile_part(p.a_scales, p.M, p.K, p.a_pad, p.a_tiles, b, p.n_ta);
    return;
  }
  b -= p.n_ta;
  scale_tile_part(p.w_scales, p.N, p.K, p.w_pad, p.w_tiles, b, p.n_tw);
}

int64_t grid_stride_blocks(int64_t items) {
  const int64_t g = (items + 255) / 256;
  return g > 8192 ? 8192 : g;
}

}  // namespace

hipError_t launch_rac_prep(bool mx, const uint16_t* x, int64_t M, int64_t N, int32_t K,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                           const uint8_t* w_scales, const float* w_ts, const uint16_t* w_hi_t,
                           const int32_t* idx,
                           int32_t k, int32_t kp, uint16_t* R, uint16_t* W_S, uint8_t* a_tiles,
                           uint8_t* w_tiles, int64_t a_pad, int64_t w_pad, hipStream_t stream,
                           int32_t* status) {
  PrepArgs p{};
  p.status = status;
  p.x = x;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_ts = a_ts;
  p.R = R;
  p.w_hi_t = w_hi_t;
  p.W_S = W_S;
  p.idx = idx;
  p.w_scales = w_scales;
  p.w_ts = w_ts;
  p.a_tiles = (uint4*)a_tiles;
  p.w_tiles = (uint4*)w_tiles;
  p.M = M;
  p.N = N;
  p.a_pad = a_pad;
  p.w_pad = w_pad;
  p.K = K;
  p.k = k;
  p.kp = kp;
  const bool rac = k > 0 && kp > 0 && R && W_S;
  const bool tiles = !mx && a_tiles && w_tiles;
  p.ws_gx = (N + 63) / 64;
  p.n_ws = rac ? p.ws_gx * ((kp + 63) / 64) : 0;
  p.n_r = rac ? grid_stride_blocks(residual_gather_items(M, kp)) : 0;
  p.n_ta = tiles ? grid_stride_blocks((int64_t)(K / 128) * a_pad) : 0;
  p.n_tw = tiles ? grid_stride_blocks((int64_t)(K / 128) * w_pad) : 0;
  int64_t grid = p.n_ws + p.n_r + p.n_ta + p.n_tw;
  if (grid == 0 && status) grid = 1;   // one workgroup writes the status word
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (mx)
    hipLaunchKernelGGL(rac_prep_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rac_prep_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Page-literal compensation (QUADS section 3.3, Eq. 20-21): the quantization
// error dX = dequant(x) - x is itself an activation for the NVFP4 quantizer
// Q_A -- carried as bf16 like any activation, with its own FP32 tensor scale
// s_R = RN32(amax|dX| / 2688) (1 for an all-zero tensor) and its own E4M3
// scale per sixteen channels -- and is masked to the selected channels after
// quantization.  The corrected activation Q_A(x) - M_S * dequant(Q_A(dX))
// multiplies the NVFP4 weight, so
//   Y = s_A s_W sum_K d_A d_W - s_R s_W sum_{t<k} R'[i][t] W'[j][t],
//   R'[i][t] = c' sb' of Q_A(dX)[i][S_t],  W'[j][t] = c_W sb_W of W[j][S_t],
// both exact in fp16 (a code times an E4M3 value has at most 6 significant
// bits, and within fp16's normal range), so the fp16 MFMA tail of the GEMM
// forms the second sum exactly up to fp32 accumulation, and the GEMM applies
// -s_R s_W.

namespace {

// The residuals r = RN32(x - c s s_A) of the sixteen elements of one block
// (dX = bf16(-r)).  xa, xb: the block's sixteen bf16; cw: its eight code
// bytes; s: its block scale; sa: the tensor scale.  The E2M1 values come from
// the FP4 conversion instruction at unit scale (exact), c s is exact in fp32
// and the fma rounds once.
__device__ __forceinline__ void block_resid(const uint4 xa, const uint4 xb, const uint2 cw,
                                            float s, float sa, float (&r)[16]) {
  const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
  const uint32_t cws[2] = {cw.x, cw.y};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    f32x2v c2[4];
    c2[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 0);
    c2[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 1);
    c2[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 2);
    c2[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 3);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = 8 * q + 2 * b;
      r[e] = fmaf(-(c2[b].x * s), sa, bf16_lo(xw[e >> 1]));
      r[e + 1] = fmaf(-(c2[b].y * s), sa, bf16_hi(xw[e >> 1]));
    }
  }
}

// bf16 of a non-negative or negative fp32 value, as an fp32 value
__device__ __forceinline__ float bf16_round(float v) {
  return __uint_as_float(f32_to_bf16_rne(v) << 16);
}

struct Eq21AmaxArgs {
  const uint4* x;          // bf16 [rows][cols], 16 elements = two uint4
  const uint2* codes;      // [rows][cols/2], 8 bytes per block
  const uint8_t* scales;   // [rows][cols/16]
  const float* a_ts;
  int64_t nblocks;         // rows * cols / 16
  uint32_t* slots;         // [gridDim.x] fp32 bits of each workgroup's max |dX|
};

__global__ __launch_bounds__(256) void eq21_amax_kernel(Eq21AmaxArgs p) {
  __shared__ uint32_t wmax[4];
  const float sa = p.a_ts[0];
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  // four blocks per thread and round, all loads issued before any is used
  // (blocks past the end load block 0 and are not counted)
  for (int64_t b0 = (int64_t)blockIdx.x * 256 + threadIdx.x; b0 < p.nblocks; b0 += 4 * stride) {
    uint4 xa[4], xb[4];
    uint2 cw[4];
    uint32_t sb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = b0 + u * stride < p.nblocks ? b0 + u * stride : 0;
      xa[u] = p.x[2 * b];
      xb[u] = p.x[2 * b + 1];
      cw[u] = p.codes[b];
      sb[u] = p.scales[b];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float r[16];
      block_resid(xa[u], xb[u], cw[u], e4m3_to_f32(sb[u]), sa, r);
      float mu = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) mu = fmaxf(mu, fabsf(r[e]));
      m = b0 + u * stride < p.nblocks ? fmaxf(m, mu) : m;
    }
  }
  // max |dX| = bf16(max |r|): rounding to bf16 is monotone
  m = bf16_round(m);
  // |dX| >= 0: fp32 bit patterns order like the values
  uint32_t mb = __float_as_uint(m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mb;
  __syncthreads();
  if (threadIdx.x == 0)
    p.slots[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

struct Eq21PrepArgs {
  // residual codes of the selected channels
  const uint16_t* x;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_ts;
  const uint32_t* slots;
  int32_t nslots;
  float* r_ts;             // s_R (workspace), written by workgroup 0 of that job
  float* r_ts_out;         // optional copy for the caller
  uint16_t* R;             // fp16 [M][kp]
  // weight columns
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  uint16_t* W_S;           // fp16 [N][kp]
  const int32_t* idx;
  // scale records
  uint4* a_tiles;
  uint4* w_tiles;
  int64_t M, N, a_pad, w_pad;
  int32_t K, k, kp;
  // workgroup ranges, in launch order: W', R', A records, W records
  int64_t n_w, n_r, n_ta, n_tw;
  int32_t* status;  // optional: Q4_OK, or Q4_EINVAL for an invalid channel set
};

__device__ __forceinline__ int clamp_chan(const int32_t* idx, int t, int k, int K) {
  const int c = t < k ? idx[t] : 0;
  return c < 0 ? 0 : (c >= K ? K - 1 : c);
}

__global__ __launch_bounds__(256) void eq21_prep_kernel(Eq21PrepArgs p) {
  __shared__ uint32_t red[256];
  __shared__ int32_t sidx[Q4_MAX_TOPK];
  int64_t b = blockIdx.x;
  // an invalid channel set (not ascending, unique and in [0, K)) gathers
  // zeros, so the GEMM adds no compensation; workgroup 0 reports it
  const bool gathers = b < p.n_w + p.n_r;
  const bool ok = gathers ? chan_set_ok(p.idx, p.k, p.K) : true;
  if (b == 0 && threadIdx.x == 0 && p.status) p.status[0] = ok ? 0 : 1;
  const int32_t kk = ok ? p.k : 0;
  if (gathers) {
    // the channel set, clamped into [0, K), staged once per workgroup
    for (int t = threadIdx.x; t < p.kp; t += 256) sidx[t] = clamp_chan(p.idx, t, kk, p.K);
    __syncthreads();
  }
  if (b < p.n_w) {
    // W'[j][t] = c_W sb_W of W[j][S_t]; one thread per (8 consecutive rows j,
    // t), t across lanes: S is ascending and clusters in a few blocks, so a
    // wave's load touches few lines, and each row's stores are contiguous
    const int64_t total = (p.N + 7) / 8 * p.kp;
    for (int64_t g = b * 256 + threadIdx.x; g < total; g += p.n_w * 256) {
      const int64_t j0 = g / p.kp * 8;
      const int t = (int)(g - g / p.kp * p.kp);
      const int c = sidx[t];
      uint32_t cb[8], sb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t j = j0 + q < p.N ? j0 + q : p.N - 1;
        cb[q] = p.w_codes[j * (p.K / 2) + (c >> 1)];
        sb[q] = p.w_scales[j * (p.K / 16) + (c >> 4)];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (j0 + q >= p.N) break;
        const float val = e2m1_value((cb[q] >> ((c & 1) * 4)) & 15u) * e4m3_to_f32(sb[q]);
        p.W_S[(j0 + q) * p.kp + t] =
            t < kk ? __builtin_bit_cast(uint16_t, (_Float16)val) : (uint16_t)0;
      }
    }
    return;
  }
  b -= p.n_w;
  if (b < p.n_r) {
    // s_R from the per-workgroup maxima of |dX| (every workgroup of this job
    // reduces them; the slots are a few KB in L2)
    uint32_t m = 0;
    for (int i = threadIdx.x; i < p.nslots; i += 256) m = max(m, p.slots[i]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (threadIdx.x < o) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + o]);
      __syncthreads();
    }
    const float amax = __uint_as_float(red[0]);
    // RN32(amax / 2688): the fp64 quotient rounded to fp32 (53 >= 2 * 24 + 2,
    // so the double rounding equals one rounding of the exact quotient)
    const float sr = amax == 0.0f ? 1.0f : (float)((double)amax / 2688.0);
    if (b == 0 && threadIdx.x == 0) {
      p.r_ts[0] = sr;
      if (p.r_ts_out) p.r_ts_out[0] = sr;
    }
    const float inv6 = 1.0f / (6.0f * sr);
    const double st6 = 6.0 * (double)sr;
    const float sa = p.a_ts[0];
    // R'[i][t]: one thread per (4 consecutive rows i, t), t across lanes (as
    // W' above; lanes of one block load the same 32 bytes); the four blocks'
    // x, codes and scale are loaded before any is used
    const int64_t total = (p.M + 3) / 4 * p.kp;
    for (int64_t g = b * 256 + threadIdx.x; g < total; g += p.n_r * 256) {
      const int64_t i0 = g / p.kp * 4;
      const int t = (int)(g - g / p.kp * p.kp);
      const int c = sidx[t];
      uint4 xa[4], xb[4];
      uint2 cw[4];
      uint32_t sb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = i0 + q < p.M ? i0 + q : p.M - 1;
        const int64_t blk = i * (p.K / 16) + (c >> 4);
        const uint4* xp = (const uint4*)(p.x + blk * 16);
        xa[q] = xp[0];
        xb[q] = xp[1];
        cw[q] = *(const uint2*)(p.a_codes + blk * 8);
        sb[q] = p.a_scales[blk];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (i0 + q >= p.M) break;
        float r[16];
        block_resid(xa[q], xb[q], cw[q], e4m3_to_f32(sb[q]), sa, r);
        float ab = 0.0f, rc = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          ab = fmaxf(ab, fabsf(r[e]));
          rc = e == (c & 15) ? r[e] : rc;
        }
        // the block amax of dX = bf16(-r) is bf16(max |r|) (monotone rounding)
        ab = bf16_round(ab);
        const float dc = bf16_round(-rc);
        const uint32_t sc = ab == 0.0f ? 0u : e4m3_scale_code(ab, inv6, st6);
        const float sbv = e4m3_to_f32(sc);
        const uint32_t nib = e2m1_nibble_exact(dc, sbv, sr);
        p.R[(i0 + q) * p.kp + t] =
            t < kk ? __builtin_bit_cast(uint16_t, (_Float16)(e2m1_value(nib) * sbv)) : (uint16_t)0;
      }
    }
    return;
  }
  b -= p.n_r;
  if (b < p.n_ta) {
    scale_tile_part(p.a_scales, p.M, p.K, p.a_pad, p.a_tiles, b, p.n_ta);
    return;
  }
  b -= p.n_ta;
  scale_tile_part(p.w_scales, p.N, p.K, p.w_pad, p.w_tiles, b, p.n_tw);
}

}  // namespace

hipError_t launch_eq21_prep(const uint16_t* x, int64_t M, int64_t N, int32_t K,
                            const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                            const uint8_t* w_codes, const uint8_t* w_scales, const int32_t* idx,
                            int32_t k, int32_t kp, uint16_t* R, uint16_t* W_S, uint32_t* slots,
                            int32_t nslots, float* r_ts, float* r_ts_out, uint8_t* a_tiles,
                            uint8_t* w_tiles, int64_t a_pad, int64_t w_pad, hipStream_t stream,
                            int32_t* status) {
  Eq21AmaxArgs a{};
  a.x = (const uint4*)x;
  a.codes = (const uint2*)a_codes;
  a.scales = a_scales;
  a.a_ts = a_ts;
  a.nblocks = M * (K / 16);
  a.slots = slots;
  hipLaunchKernelGGL(eq21_amax_kernel, dim3((unsigned)nslots), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Eq21PrepArgs p{};
  p.x = x;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_ts = a_ts;
  p.slots = slots;
  p.nslots = nslots;
  p.r_ts = r_ts;
  p.r_ts_out = r_ts_out;
  p.R = R;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.W_S = W_S;
  p.idx = idx;
  p.a_tiles = (uint4*)a_tiles;
  p.w_tiles = (uint4*)w_tiles;
  p.M = M;
  p.N = N;
  p.a_pad = a_pad;
  p.w_pad = w_pad;
  p.K = K;
  p.k = k;
  p.kp = kp;
  p.status = status;
  const bool tiles = a_tiles && w_tiles;
  p.n_w = grid_stride_blocks((N + 7) / 8 * kp);
  p.n_r = grid_stride_blocks((M + 3) / 4 * kp);
  p.n_ta = tiles ? grid_stride_blocks((int64_t)(K / 128) * a_pad) : 0;
  p.n_tw = tiles ? grid_stride_blocks((int64_t)(K / 128) * w_pad) : 0;
  const int64_t grid = p.n_w + p.n_r + p.n_ta + p.n_tw;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(eq21_prep_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace q4
