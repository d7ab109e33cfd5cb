// Online NVFP4 / MXFP4 activation quantization with per-channel residual
// statistics, channel selection and residual gathers (gfx950).
//
// QUADS (arXiv 2607.15810): section 2.2 "FP4" (format), section 3.3 Eq. 20
// (quantization error), Eq. 23 (per-channel residual norm over the token
// batch), Eq. 24 (top-k channel selection), Eq. 21 (residual on the selected
// channels).  The page fuses quantization and residual extraction in one
// kernel; here one pass over x emits codes, block scales and fp64 per-channel
// partial sums of squared residuals.
#include "q4_internal.h"

namespace q4 {

// ====================================================================== amax
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t w) {
  uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  return lo > hi ? lo : hi;
}

// max |x| as a bf16 bit pattern (non-negative bf16 order is integer order);
// order-independent, so the atomic combine is deterministic.
__global__ __launch_bounds__(256) void amax_kernel(const uint4* __restrict__ x, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v0 = x[i], v1 = x[i + stride], v2 = x[i + 2 * stride], v3 = x[i + 3 * stride];
    uint32_t a = max(max(absmax_bf16x2(v0.x), absmax_bf16x2(v0.y)), max(absmax_bf16x2(v0.z), absmax_bf16x2(v0.w)));
    uint32_t b = max(max(absmax_bf16x2(v1.x), absmax_bf16x2(v1.y)), max(absmax_bf16x2(v1.z), absmax_bf16x2(v1.w)));
    uint32_t c = max(max(absmax_bf16x2(v2.x), absmax_bf16x2(v2.y)), max(absmax_bf16x2(v2.z), absmax_bf16x2(v2.w)));
    uint32_t d = max(max(absmax_bf16x2(v3.x), absmax_bf16x2(v3.y)), max(absmax_bf16x2(v3.z), absmax_bf16x2(v3.w)));
    m = max(m, max(max(a, b), max(c, d)));
  }
  for (; i < n16; i += stride) {
    uint4 v = x[i];
    m = max(m, max(max(absmax_bf16x2(v.x), absmax_bf16x2(v.y)), max(absmax_bf16x2(v.z), absmax_bf16x2(v.w))));
  }
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m) atomicMax(out, m);
  }
}

// ====================================================================== quantize
struct QuantKArgs {
  const uint16_t* x;
  int64_t rows;
  int32_t cols;
  int32_t nstrips;      // ceil(cols / 512)
  int64_t ntiles;       // ceil(rows / 64)
  const float* ts_in;   // NVFP4 supplied tensor scale or null
  const uint32_t* amax; // NVFP4 amax (bf16 bits) when ts_in is null
  uint8_t* codes;
  uint8_t* scales;
  float* ts_out;
  double* partial;      // [ntiles][cols]
  int32_t reverse;      // process tiles last-to-first (reuse of the last-level cache)
};

__device__ __forceinline__ float nvfp4_tensor_scale_dev(const QuantKArgs& a) {
  if (a.ts_in) return a.ts_in[0];
  float am = __uint_as_float(a.amax[0] << 16);
  // RN32(amax / 2688): the fp64 quotient is never an fp32 midpoint
  // (2688 = 21 * 2^7, amax has 8 significant bits), so one more rounding to
  // fp32 gives the correctly rounded quotient.
  return am == 0.0f ? 1.0f : (float)((double)am / 2688.0);
}

// One wave per (64-row tile, 512-channel strip); lane l owns channels
// strip*512 + 8l .. +7 and walks the tile's rows in order, so its fp64 sums of
// squared residuals follow the fixed row order of the definition.
template <bool MX>
__global__ __launch_bounds__(256) void quantize_kernel(QuantKArgs a) {
  const int lane = threadIdx.x & 63;
  int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nunits = a.ntiles * a.nstrips;
  if (unit >= nunits) return;
  if (a.reverse) unit = nunits - 1 - unit;
  const int64_t tile = unit / a.nstrips;
  const int strip = (int)(unit % a.nstrips);
  const int cols = a.cols;
  const int col0 = strip * 512 + lane * 8;
  const bool active = col0 < cols;

  float st = 1.0f;
  if constexpr (!MX) {
    st = nvfp4_tensor_scale_dev(a);
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.ts_out) a.ts_out[0] = st;
  }
  const float inv6st = 1.0f / (6.0f * st);
  const double st6 = 6.0 * (double)st;

  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;

  const int64_t r0 = tile * kScoreTileRows;
  const int nr = (int)min((int64_t)kScoreTileRows, a.rows - r0);
  const uint16_t* xp = a.x + r0 * cols + (active ? col0 : 0);
  const int64_t cstride = cols / 2, sstride = MX ? cols / 32 : cols / 16;
  constexpr int U = 8;

  for (int rr = 0; rr < nr; rr += U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (active && rr + u < nr)
        v[u] = *(const uint4*)(xp + (int64_t)(rr + u) * cols);
      else
        v[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (rr + u >= nr) break;
      const int64_t row = r0 + rr + u;
      float xf[8];
      xf[0] = bf16_lo(v[u].x); xf[1] = bf16_hi(v[u].x);
      xf[2] = bf16_lo(v[u].y); xf[3] = bf16_hi(v[u].y);
      xf[4] = bf16_lo(v[u].z); xf[5] = bf16_hi(v[u].z);
      xf[6] = bf16_lo(v[u].w); xf[7] = bf16_hi(v[u].w);
      float m = fmaxf(fmaxf(fmaxf(fabsf(xf[0]), fabsf(xf[1])), fmaxf(fabsf(xf[2]), fabsf(xf[3]))),
                      fmaxf(fmaxf(fabsf(xf[4]), fabsf(xf[5])), fmaxf(fabsf(xf[6]), fabsf(xf[7]))));
      m = wave_xor_max(m, 1);                  // 16-element block = lane pair
      uint32_t sc;
      float s;
      if constexpr (MX) {
        m = wave_xor_max(m, 2);                // 32-element block = lane quad
        // floor(log2 m) - 2 clamped to [-127, 127]: exponent field - 129
        int ef = (int)((__float_as_uint(m) >> 23) & 255u);
        int e = max(ef - 129, -127);
        sc = (uint32_t)(e + 127);
        s = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : 0x1p-127f;
      } else {
        sc = e4m3_scale_code(m, inv6st, st6);
        s = e4m3_to_f32(sc);
      }
      const float S = s * st;
      const bool fast = S >= 0x1p-100f;
      const float rinv = fast ? __builtin_amdgcn_rcpf(S) : 0.0f;
      const float rlo = rinv * (1.0f - 0x1p-20f), rhi = rinv * (1.0f + 0x1p-20f);
      uint32_t lo = 0, hi = 0;
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xf[0] * rlo, xf[1] * rlo, 1.0f, 0);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xf[2] * rlo, xf[3] * rlo, 1.0f, 1);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xf[4] * rlo, xf[5] * rlo, 1.0f, 2);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xf[6] * rlo, xf[7] * rlo, 1.0f, 3);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xf[0] * rhi, xf[1] * rhi, 1.0f, 0);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xf[2] * rhi, xf[3] * rhi, 1.0f, 1);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xf[4] * rhi, xf[5] * rhi, 1.0f, 2);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xf[6] * rhi, xf[7] * rhi, 1.0f, 3);
      uint32_t code = lo;
      if (!fast || lo != hi) {
        // a value within 2^-20 of a rounding boundary (or an extreme scale):
        // decide every element exactly
        code = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) code |= e2m1_nibble_exact(xf[i], s, st) << (4 * i);
      }
      // residual r = RN32(x - c s st): c*s is exact, one fused rounding
      float cv[8];
      {
        f32x2v c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
        f32x2v c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 1);
        f32x2v c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 2);
        f32x2v c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 3);
        cv[0] = c0.x; cv[1] = c0.y; cv[2] = c1.x; cv[3] = c1.y;
        cv[4] = c2.x; cv[5] = c2.y; cv[6] = c3.x; cv[7] = c3.y;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float r = fmaf(-(cv[i] * s), st, xf[i]);
        double rd = (double)r;
        acc[i] = fma(rd, rd, acc[i]);
      }
      if (active) {
        *(uint32_t*)(a.codes + row * cstride + (col0 >> 1)) = code;
        if constexpr (MX) {
          if ((lane & 3) == 0) a.scales[row * sstride + (col0 >> 5)] = (uint8_t)sc;
        } else {
          if ((lane & 1) == 0) a.scales[row * sstride + (col0 >> 4)] = (uint8_t)sc;
        }
      }
    }
  }
  if (active) {
    double* pp = a.partial + tile * cols + col0;
#pragma unroll
    for (int i = 0; i < 8; ++i) pp[i] = acc[i];
  }
}

// ====================================================================== scores
// score_j = sum over tiles ascending of the tile partial sums (fp64)
__global__ __launch_bounds__(256) void score_reduce_kernel(const double* __restrict__ partial,
                                                           int64_t ntiles, int32_t cols,
                                                           double* __restrict__ scores) {
  int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= cols) return;
  double s = 0.0;
  int64_t t = 0;
  for (; t + 8 <= ntiles; t += 8) {
    double p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = partial[(t + u) * cols + j];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += p[u];
  }
  for (; t < ntiles; ++t) s += partial[t * cols + j];
  scores[j] = s;
}

// ====================================================================== top-k
// One workgroup.  Radix select (8 bits per pass, most significant first) finds
// the k-th largest key (non-negative fp64 bit patterns order as integers),
// then an ordered scan emits every key above it and the first equal keys by
// channel index, in ascending channel order.
__device__ __forceinline__ int block_excl_scan_bits(bool flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint64_t b = __ballot(flag);
  int in_wave = __popcll(b & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wsum[w] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    int v = wsum[i];
    before += (i < w) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

__global__ __launch_bounds__(1024) void topk_kernel(const double* __restrict__ scores, int32_t cols,
                                                    int32_t k, int32_t* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_kleft;
  __shared__ int wsum[16];
  const uint64_t* keys = (const uint64_t*)scores;
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  int kleft = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < cols; j += 1024) {
      uint64_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0;
      for (int d = 255; d >= 0; --d) {
        int h = (int)hist[d];
        if (cum + h >= kleft) {
          prefix |= (uint64_t)d << shift;
          kleft -= cum;
          break;
        }
        cum += h;
      }
      s_prefix = prefix;
      s_kleft = kleft;
    }
    __syncthreads();
    prefix = s_prefix;
    kleft = s_kleft;
    mask |= 0xffull << shift;
  }
  const uint64_t T = prefix;   // the k-th largest key; kleft of its copies are taken
  int base_eq = 0, base_sel = 0;
  for (int c0 = 0; c0 < cols; c0 += 1024) {
    const int j = c0 + tid;
    const uint64_t key = j < cols ? keys[j] : 0ull;
    const bool eq = j < cols && key == T;
    const bool gt = j < cols && key > T;
    int tot_eq, tot_sel;
    const int eq_rank = base_eq + block_excl_scan_bits(eq, wsum, &tot_eq);
    const bool sel = gt || (eq && eq_rank < kleft);
    const int pos = base_sel + block_excl_scan_bits(sel, wsum, &tot_sel);
    if (sel) out[pos] = j;
    base_eq += tot_eq;
    base_sel += tot_sel;
  }
}

// ====================================================================== gathers
// R[i][t] = bf16(RN32(x[i][S_t] - dequant)) for t < k, 0 for k <= t < ld_r
template <bool MX>
__global__ __launch_bounds__(256) void residual_gather_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int32_t cols, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ ts,
    const int32_t* __restrict__ idx, int32_t k, uint16_t* __restrict__ R, int64_t ld_r) {
  const int64_t total = rows * ld_r;
  const float st = MX ? 1.0f : ts[0];
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * 256) {
    const int64_t i = g / ld_r;
    const int t = (int)(g - i * ld_r);
    uint32_t out = 0;
    if (t < k) {
      int j = idx[t];
      j = j < 0 ? 0 : (j >= cols ? cols - 1 : j);
      const float xv = bf16_to_f32(x[i * cols + j]);
      const uint32_t nib = (codes[i * (cols / 2) + (j >> 1)] >> ((j & 1) * 4)) & 15u;
      float s;
      if constexpr (MX) {
        const int e = (int)scales[i * (cols / 32) + (j >> 5)] - 127;
        s = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : 0x1p-127f;
      } else {
        s = e4m3_to_f32(scales[i * (cols / 16) + (j >> 4)]);
      }
      const float r = fmaf(-(e2m1_value(nib) * s), st, xv);
      out = f32_to_bf16_rne(r);
    }
    R[g] = (uint16_t)out;
  }
}

// W_S[b][j][t] = w_hi_t[b][S_t][j] for t < k, 0 for k <= t < kp (a transposing
// gather through a 64 x 64 LDS tile; the selected rows are contiguous in j).
__global__ __launch_bounds__(256) void wsel_gather_kernel(const uint16_t* __restrict__ w_hi_t,
                                                          int64_t K, int64_t N,
                                                          const int32_t* __restrict__ idx,
                                                          int32_t k, int32_t kp,
                                                          uint16_t* __restrict__ ws) {
  __shared__ uint16_t tile[64][66];
  const int64_t b = blockIdx.z;
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int t0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t* src = w_hi_t + b * K * N;
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r;
    const int64_t j = j0 + tx;
    uint16_t v = 0;
    if (t < k && j < N) {
      int c = idx[t];
      c = c < 0 ? 0 : (c >= K ? (int)K - 1 : c);
      v = src[(int64_t)c * N + j];
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  uint16_t* dst = ws + b * N * kp;
  for (int r = ty; r < 64; r += 4) {
    const int64_t j = j0 + r;
    const int t = t0 + tx;
    if (j < N && t < kp) dst[j * kp + t] = tile[tx][r];
  }
}

// out[b][c][r] = in[b][r][c]
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int64_t rows, int64_t cols,
                                                             uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[64][66];
  const int64_t b = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t* src = in + b * rows * cols;
  uint16_t* dst = out + b * rows * cols;
  for (int r = ty; r < 64; r += 4) {
    const int64_t rr = r0 + r, cc = c0 + tx;
    tile[r][tx] = (rr < rows && cc < cols) ? src[rr * cols + cc] : (uint16_t)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t cc = c0 + r, rr = r0 + tx;
    if (cc < cols && rr < rows) dst[cc * rows + rr] = tile[tx][r];
  }
}

// packed row p of expert e <- logical row: group g = p / 64, q = p % 64;
// q < 32 -> gate row 32g + q, else up row F + 32g + (q - 32)
__global__ __launch_bounds__(256) void moe_pack_w13_kernel(const uint16_t* __restrict__ w13,
                                                           int32_t F, int32_t H,
                                                           uint16_t* __restrict__ out) {
  const int64_t e = blockIdx.z;
  const int p = blockIdx.y;
  const int g = p >> 6, q = p & 63;
  const int src_row = q < 32 ? 32 * g + q : F + 32 * g + (q - 32);
  const uint16_t* s = w13 + (e * 2 * F + src_row) * (int64_t)H;
  uint16_t* d = out + (e * 2 * F + p) * (int64_t)H;
  for (int h = blockIdx.x * 256 + threadIdx.x; h < H; h += gridDim.x * 256) d[h] = s[h];
}

// ====================================================================== launchers
size_t quantize_workspace_bytes(int64_t rows, int64_t cols) {
  const int64_t ntiles = (rows + kScoreTileRows - 1) / kScoreTileRows;
  return 256 + align256((size_t)ntiles * (size_t)cols * 8) + align256((size_t)cols * 8);
}

hipError_t launch_quantize(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                           const float* ts_in, uint8_t* codes, uint8_t* scales, float* ts_out,
                           double* chan_score, int32_t topk, int32_t* chan_idx, void* ws,
                           hipStream_t stream) {
  uint8_t* base = (uint8_t*)ws;
  uint32_t* amax = (uint32_t*)base;
  const int64_t ntiles = (rows + kScoreTileRows - 1) / kScoreTileRows;
  double* partial = (double*)(base + 256);
  double* scores = chan_score ? chan_score
                              : (double*)(base + 256 + align256((size_t)ntiles * cols * 8));
  const bool need_amax = !mx && ts_in == nullptr;
  if (need_amax) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(256), 0, stream, amax, (int64_t)1, 0u);
    const int64_t n16 = rows * cols / 8;
    if (n16 > 0) {
      int64_t grid = (n16 + 256 * 8 - 1) / (256 * 8);
      grid = grid < 1 ? 1 : (grid > 4096 ? 4096 : grid);
      hipLaunchKernelGGL(amax_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                         (const uint4*)x, n16, amax);
    }
  }
  QuantKArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.nstrips = (int32_t)((cols + 511) / 512);
  a.ntiles = ntiles;
  a.ts_in = ts_in;
  a.amax = amax;
  a.codes = codes;
  a.scales = scales;
  a.ts_out = ts_out;
  a.partial = partial;
  a.reverse = need_amax ? 1 : 0;
  const int64_t units = ntiles * a.nstrips;
  if (units > 0) {
    const unsigned grid = (unsigned)((units + 3) / 4);
    if (mx)
      hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
  } else if (!mx && ts_out) {
    // no rows: still report s_t (1, or the supplied value)
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(64), 0, stream, ts_in, ts_out);
  }
  hipLaunchKernelGGL(score_reduce_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0,
                     stream, (const double*)partial, ntiles, (int32_t)cols, scores);
  if (topk > 0)
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(1024), 0, stream, (const double*)scores,
                       (int32_t)cols, topk, chan_idx);
  return hipGetLastError();
}

__global__ void tensor_scale_kernel(const float* ts_in, float* ts_out) {
  if (threadIdx.x == 0) ts_out[0] = ts_in ? ts_in[0] : 1.0f;
}

hipError_t launch_select(const double* scores, int64_t cols, int32_t topk, int32_t* idx,
                         hipStream_t stream) {
  if (topk > 0)
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(1024), 0, stream, scores, (int32_t)cols, topk,
                       idx);
  return hipGetLastError();
}

hipError_t launch_residual_gather(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                                  const uint8_t* codes, const uint8_t* scales, const float* ts,
                                  const int32_t* idx, int32_t k, uint16_t* R, int64_t ld_r,
                                  hipStream_t stream) {
  const int64_t total = rows * ld_r;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  grid = grid > 65536 ? 65536 : grid;
  if (mx)
    hipLaunchKernelGGL(residual_gather_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       rows, (int32_t)cols, codes, scales, ts, idx, k, R, ld_r);
  else
    hipLaunchKernelGGL(residual_gather_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                       x, rows, (int32_t)cols, codes, scales, ts, idx, k, R, ld_r);
  return hipGetLastError();
}

hipError_t launch_wsel_gather(const uint16_t* w_hi_t, int64_t batch, int64_t K, int64_t N,
                              const int32_t* idx, int32_t k, int32_t kp, uint16_t* ws,
                              hipStream_t stream) {
  if (batch == 0 || N == 0 || kp == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((kp + 63) / 64), (unsigned)batch);
  hipLaunchKernelGGL(wsel_gather_kernel, grid, dim3(256), 0, stream, w_hi_t, K, N, idx, k, kp, ws);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t batch, int64_t rows, int64_t cols,
                                 uint16_t* out, hipStream_t stream) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)batch);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_moe_pack_w13(const uint16_t* w13, int32_t E, int32_t F, int32_t H,
                               uint16_t* out, hipStream_t stream) {
  if (E == 0) return hipSuccess;
  unsigned gx = (unsigned)((H + 255) / 256);
  gx = gx > 16 ? 16 : gx;
  hipLaunchKernelGGL(moe_pack_w13_kernel, dim3(gx, (unsigned)(2 * F), (unsigned)E), dim3(256), 0,
                     stream, w13, F, H, out);
  return hipGetLastError();
}

}  // namespace q4
