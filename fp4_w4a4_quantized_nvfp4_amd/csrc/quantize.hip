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
#include "q4_nvfp4_enc.h"
#include "q4_prep.h"

namespace q4 {

// ====================================================================== amax
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p,
                     n, v);
  return hipGetLastError();
}

__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t w) {
  uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  return lo > hi ? lo : hi;
}

// Per-workgroup max |x| as a bf16 bit pattern (non-negative bf16 order is
// integer order).  Each workgroup writes its own slot; the quantize kernel
// reduces the slots, so no atomics are involved and the result is exact.
// The tensor is walked front to back in segments of 32 KB (eight 16-byte
// loads per thread in flight), workgroup b taking segments b, b + grid, ...:
// each workgroup reads contiguous memory, and the data read last (the end of
// the tensor) is what the quantize pass, walking groups in reverse, reads
// first while it is still in the last-level cache.
constexpr int kAmaxBlocks = 1024;
constexpr int kAmaxUnroll = 8;
constexpr int64_t kAmaxSeg = 256 * kAmaxUnroll;   // uint4 per segment

__global__ __launch_bounds__(256) void amax_kernel(const uint4* __restrict__ x, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  uint32_t m = 0;
  const int64_t nseg = (n16 + kAmaxSeg - 1) / kAmaxSeg;
  for (int64_t sg = blockIdx.x; sg < nseg; sg += gridDim.x) {
    const int64_t base = sg * kAmaxSeg + threadIdx.x;
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      v[u] = base + u * 256 < n16 ? x[base + u * 256] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      m = max(m, max(max(absmax_bf16x2(v[u].x), absmax_bf16x2(v[u].y)),
                     max(absmax_bf16x2(v[u].z), absmax_bf16x2(v[u].w))));
  }
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// ====================================================================== quantize
struct QuantKArgs {
  const uint16_t* x;
  int64_t rows;
  int32_t cols;
  int32_t nstrips;      // ceil(cols / 512)
  int64_t ngroups;      // ceil(rows / 256)
  const float* ts_in;   // NVFP4 supplied tensor scale or null
  const uint32_t* amax; // NVFP4 per-workgroup amax slots (bf16 bits) when ts_in is null
  int32_t namax;        // number of slots
  uint8_t* codes;
  uint8_t* scales;
  float* ts_out;
  double* partial;      // [ngroups][cols]
  int32_t reverse;      // process groups last-to-first (reuse of the last-level cache)
};

// tensor scale of the launch and its tie mode; every thread of the
// workgroup must call it
__device__ float nvfp4_tensor_scale_dev(const QuantKArgs& a, uint32_t* red, int* tie_mode) {
  if (a.ts_in) {
    const float st = a.ts_in[0];
    *tie_mode = supplied_tie_mode(st);
    return st;
  }
  uint32_t m = 0;
  for (int i = threadIdx.x; i < a.namax; i += blockDim.x) m = max(m, a.amax[i]);
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = max(m, red[w]);
  float am = __uint_as_float(m << 16);
  // RN32(amax / 2688): the fp64 quotient is never an fp32 midpoint
  // (2688 = 21 * 2^7, amax has 8 significant bits), so one more rounding to
  // fp32 gives the correctly rounded quotient.
  const float st = am == 0.0f ? 1.0f : (float)((double)am / 2688.0);
  *tie_mode = am == 0.0f ? kTieEven : tie_mode_of(st, am);
  return st;
}

// One workgroup = 8 waves = one group of 8 TR rows of one strip of 64 * CPL
// channels; wave w owns the TR-row tile w of the group, lane l owns channels
// strip * 64 * CPL + CPL * l .. + CPL - 1 (CPL = 8 or 16 channels per lane;
// TR = 32, or 8 for small tensors, so that they still spread over the CUs).
// Every lane sums its squared residuals over its tile's rows in order; the
// eight tile sums are then added in tile order through LDS, giving one fp64
// partial per (group, channel).  Codes and scales: nvfp4_lane_encode (near
// ties are frequent: s_t is a rounded simple rational, so many x / (s s_t)
// fall within 2^-24 of a midpoint).
template <bool MX, int CPL, int TR = kScoreTileRows>
__global__ __launch_bounds__(512, 4) void quantize_kernel(QuantKArgs a) {
  constexpr int NW = CPL / 8;              // code words (8 nibbles) per lane per row
  constexpr int U = 64 / CPL;              // rows in flight per lane
  constexpr int STRIP = 64 * CPL;
  __shared__ uint8_t tab[128];
  __shared__ uint32_t red[16];
  __shared__ double part[kScoreGroupTiles][64][CPL + 1];
  // the wave index is uniform per wave: keep it (and the row range derived from
  // it) in scalar registers, so the row loop is a scalar loop
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t wg = blockIdx.x;
  const int64_t nwg = a.ngroups * a.nstrips;
  if (a.reverse) wg = nwg - 1 - wg;
  const int64_t group = wg / a.nstrips;
  const int strip = (int)(wg % a.nstrips);
  const int cols = a.cols;
  const int col0 = strip * STRIP + lane * CPL;
  const bool active = col0 < cols;

  float st = 1.0f;
  int eDp = 0;
  int tie_mode = kTieEven;
  if constexpr (!MX) {
    st = nvfp4_tensor_scale_dev(a, red, &tie_mode);
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.ts_out) a.ts_out[0] = st;
    int eD;
    const double Dm = frexp(6.0 * (double)st, &eD);   // 6 s_t = Dm 2^eD, Dm in [0.5, 1)
    eDp = eD - 1;
    if (threadIdx.x < 128) tab[threadIdx.x] = (uint8_t)e4m3_mantissa_entry(threadIdx.x, 2.0 * Dm);
  }
  __syncthreads();
  const float inv6st = 1.0f / (6.0f * st);
  const double st6 = 6.0 * (double)st;

  double acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.0;

  const int64_t r0 = group * (TR * kScoreGroupTiles) + wave * TR;
  const int nr = (int)max((int64_t)0, min((int64_t)TR, a.rows - r0));
  const int64_t cstride = cols / 2, sstride = MX ? cols / 32 : cols / 16;

  // x, codes and scales of this wave's tile through buffer resources based at
  // the tile's first row, sized to its nr rows: the row goes into the scalar
  // offset, the lane's channels into one per-lane offset.  Anything outside
  // the range (rows past the tile, lanes past the last channel) loads zeros
  // and stores nothing, so no access needs a branch.
  auto rsrc = [](const void* base, int64_t bytes) __attribute__((always_inline)) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const uint32_t n = bytes <= 0 ? 0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)n), 0x00020000);
  };
  const int64_t rb = nr > 0 ? r0 : 0;
  const __amdgpu_buffer_rsrc_t x_rs = rsrc(a.x + rb * cols, (int64_t)nr * cols * 2);
  const __amdgpu_buffer_rsrc_t c_rs = rsrc(a.codes + rb * cstride, (int64_t)nr * cstride);
  const __amdgpu_buffer_rsrc_t s_rs = rsrc(a.scales + rb * sstride, (int64_t)nr * sstride);
  constexpr uint32_t kOut = 0x80000000u;   // a per-lane offset past every range
  const uint32_t x_voff = active ? (uint32_t)col0 * 2u : kOut;
  const uint32_t c_voff = active ? (uint32_t)(col0 >> 1) : kOut;
  bool writes_scale;
  if constexpr (MX) writes_scale = (lane & (32 / CPL - 1)) == 0;
  else writes_scale = CPL == 16 || (lane & 1) == 0;
  const uint32_t s_voff = (active && writes_scale) ? (uint32_t)(col0 >> (MX ? 5 : 4)) : kOut;
  const int x_rowb = cols * 2;

  // ring of U rows in flight per lane: slot u holds row rr + u and is
  // refilled with row rr + u + U once that row is done, so the loop carries no
  // register copies
  uint4 buf[U][NW];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int soff = u * x_rowb;
#pragma unroll
    for (int q = 0; q < NW; ++q)
      buf[u][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, x_voff + 16 * q, soff, 0));
    // keep the slots' issue order (slot 0 oldest), the order the loop refills
    // them in, so the wait before each row covers that row's loads only
    __builtin_amdgcn_sched_barrier(0);
  }

  // one row: codes, block scale, residual statistics (w: the row's raw words)
  auto do_row = [&](const uint4* w, int64_t row) __attribute__((always_inline)) {
    float xf[CPL];
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      xf[8 * q + 0] = bf16_lo(w[q].x); xf[8 * q + 1] = bf16_hi(w[q].x);
      xf[8 * q + 2] = bf16_lo(w[q].y); xf[8 * q + 3] = bf16_hi(w[q].y);
      xf[8 * q + 4] = bf16_lo(w[q].z); xf[8 * q + 5] = bf16_hi(w[q].z);
      xf[8 * q + 6] = bf16_lo(w[q].w); xf[8 * q + 7] = bf16_hi(w[q].w);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) m = fmaxf(m, fabsf(xf[i]));
    if constexpr (!MX && CPL == 8) m = fmaxf(m, dpp_quad_xor1(m));   // 16-block = lane pair
    if constexpr (MX) {
      m = fmaxf(m, dpp_quad_xor1(m));                                // 32-block
      if constexpr (CPL == 8) m = fmaxf(m, dpp_quad_xor2(m));
    }
    uint32_t code[NW], sc;
    float s;
    nvfp4_lane_encode<MX, CPL>(w, xf, m, st, eDp, tab, inv6st, st6, tie_mode, code, &sc, &s);
    // residual r = RN32(x - c s st): c*s is exact, one fused rounding
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      f32x2v c2[4];
      c2[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[q], 1.0f, 0);
      c2[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[q], 1.0f, 1);
      c2[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[q], 1.0f, 2);
      c2[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[q], 1.0f, 3);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i0 = 8 * q + 2 * b;
        const float r0v = fmaf(-(c2[b].x * s), st, xf[i0]);
        const float r1v = fmaf(-(c2[b].y * s), st, xf[i0 + 1]);
        const double d0 = (double)r0v, d1 = (double)r1v;
        acc[i0] = fma(d0, d0, acc[i0]);
        acc[i0 + 1] = fma(d1, d1, acc[i0 + 1]);
      }
    }
    // add this row into the sums here: left to itself the compiler sinks
    // every row's accumulation to the end of the unrolled rows, keeping all
    // their residuals live at once
#pragma unroll
    for (int i = 0; i < CPL; ++i) asm volatile("" : "+v"(acc[i]));
    {
      const int rl = (int)(row - rb);
      if constexpr (NW == 2) {
        const u32x2v cw = {code[0], code[1]};
        __builtin_amdgcn_raw_buffer_store_b64(cw, c_rs, c_voff, rl * (int)cstride, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(code[0], c_rs, c_voff, rl * (int)cstride, 0);
      }
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, s_rs, s_voff, rl * (int)sstride, 0);
    }
  };

  // full groups of U rows through the ring; the (rare) ragged rows of a
  // tile's end one at a time
  const int nfull = nr & ~(U - 1);
  for (int rr = 0; rr < nfull; rr += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      do_row(buf[u], r0 + rr + u);
      const int soff = (rr + u + U) * x_rowb;
#pragma unroll
      for (int q = 0; q < NW; ++q)
        buf[u][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, x_voff + 16 * q, soff, 0));
      // rows one after another: interleaving them only raises register use
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int r = nfull; r < nr; ++r) {
    uint4 w[NW];
#pragma unroll
    for (int q = 0; q < NW; ++q)
      w[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, x_voff + 16 * q, r * x_rowb, 0));
    do_row(w, r0 + r);
  }
  // tile sums -> group sum, tiles in order
#pragma unroll
  for (int i = 0; i < CPL; ++i) part[wave][lane][i] = acc[i];
  __syncthreads();
#pragma unroll
  for (int h = 0; h < NW; ++h) {
    const int c = threadIdx.x + 512 * h;   // channel strip * STRIP + c
    double gsum = 0.0;
#pragma unroll
    for (int w = 0; w < kScoreGroupTiles; ++w) gsum += part[w][c / CPL][c % CPL];
    const int col = strip * STRIP + c;
    if (col < cols) a.partial[group * cols + col] = gsum;
  }
}

// ====================================================================== scores
// score_j = sum of the group partial sums (fp64), in a fixed order: W waves
// per 64 channels, wave w summing groups [w G / W, (w + 1) G / W) in
// ascending order, then the W sums added in wave order.  Many groups (a
// tensor of many rows) spread over W waves; few keep W = 1, which spreads
// the loads over as many CUs as possible.  (ngroups_dev: the group count is
// mult * ngroups_dev[0], read on the device.)
template <int W>
__global__ __launch_bounds__(64 * W) void score_reduce_kernel(const double* __restrict__ partial,
                                                              int64_t ngroups, int32_t cols,
                                                              double* __restrict__ scores,
                                                              const int32_t* __restrict__ ngroups_dev,
                                                              int32_t mult) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const bool live = j < cols;
  if (ngroups_dev) ngroups = (int64_t)ngroups_dev[0] * mult;
  const int64_t g0 = ngroups * w / W, g1 = ngroups * (w + 1) / W;
  double s = 0.0;
  // up to B loads in flight (8 or 16 waves per workgroup, two or four per
  // SIMD: a smaller batch); slots past the range read as +0.0, which leaves
  // the (non-negative) running sum unchanged
  constexpr int B = W >= 8 ? 16 : 64;
  for (int64_t t = g0; t < g1; t += B) {
    double p[B];
#pragma unroll
    for (int u = 0; u < B; ++u) p[u] = (live && t + u < g1) ? partial[(t + u) * cols + j] : 0.0;
#pragma unroll
    for (int u = 0; u < B; ++u) s += p[u];
  }
  if constexpr (W == 1) {
    if (live) scores[j] = s;
  } else {
    __shared__ double red[W][64];
    red[w][lane] = s;
    __syncthreads();
    if (w == 0 && live) {
      double tot = 0.0;
#pragma unroll
      for (int i = 0; i < W; ++i) tot += red[i][lane];
      scores[j] = tot;
    }
  }
}

// waves per 64 channels for a reduction over ngroups groups: 8 or 16 from
// 128 groups on (16-32 groups per wave), else one wave, which spreads fewer
// groups over more CUs (measured faster for 32 and 64 groups)
static int score_waves(int64_t ngroups) { return ngroups >= 256 ? 16 : (ngroups >= 128 ? 8 : 1); }

static void launch_score_reduce_host(const double* partial, int64_t ngroups, int64_t cols,
                                     double* scores, hipStream_t stream) {
  const dim3 grid((unsigned)((cols + 63) / 64));
  switch (score_waves(ngroups)) {
    case 16:
      hipLaunchKernelGGL(score_reduce_kernel<16>, grid, dim3(1024), 0, stream, partial, ngroups,
                         (int32_t)cols, scores, nullptr, 0);
      break;
    case 8:
      hipLaunchKernelGGL(score_reduce_kernel<8>, grid, dim3(512), 0, stream, partial, ngroups,
                         (int32_t)cols, scores, nullptr, 0);
      break;
    default:
      hipLaunchKernelGGL(score_reduce_kernel<1>, grid, dim3(64), 0, stream, partial, ngroups,
                         (int32_t)cols, scores, nullptr, 0);
  }
}

// ====================================================================== top-k
// One workgroup of 1024 threads.  Radix select over the fp64 bit patterns
// (non-negative doubles order as unsigned integers), eight 8-bit digits from
// the top: a wave-aggregated histogram, then one wave finds the digit that
// holds the k-th largest key.  The emit pass takes every key above it and the
// lowest-index copies of it, in ascending channel order.
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0, mask = 0;
  int kleft = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < cols; j0 += 1024) {
      const int j = j0 + tid;
      const uint64_t key = j < cols ? keys[j] : 0ull;
      const bool valid = j < cols && (key & mask) == prefix;
      const uint32_t digit = (uint32_t)(key >> shift) & 255u;
      uint64_t pending = __ballot(valid);
      while (pending) {
        const int leader = __ffsll((unsigned long long)pending) - 1;
        const uint32_t d0 = (uint32_t)__shfl((int)digit, leader, 64);
        const uint64_t same = __ballot(valid && digit == d0) & pending;
        if (lane == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
        pending &= ~same;
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t c[4];
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        sum += c[q];
      }
      uint32_t incl = sum;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += v;
      }
      uint32_t cum = incl - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (cum < (uint32_t)kleft && cum + c[q] >= (uint32_t)kleft) {
          s_prefix = prefix | ((uint64_t)(255 - 4 * lane - q) << shift);
          s_kleft = kleft - (int)cum;
        }
        cum += c[q];
      }
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

// Register-resident variant for cols <= 1024 * KPT: thread t holds the keys
// of channels t*KPT .. t*KPT + KPT - 1 (loaded once), the radix passes stop as
// soon as the bin that holds the k-th largest key is taken whole, and the
// emit pass needs two block scans (ties by channel index, then positions).
__device__ __forceinline__ int block_excl_scan_int(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int s = wsum[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// Register-resident top-k (cols <= 1024 * KPT), one workgroup of 1024
// threads holding KPT keys each (fp64 bit patterns: non-negative doubles
// order as unsigned integers).  Radix select with 11-bit digits from the
// first bit where two keys differ (two histogram buffers, so one pass costs
// two barriers).  Once the bin holding the k-th key has at most 64 keys and
// is not taken whole, those are ranked directly (key descending, channel
// ascending).  The emit pass takes every key above the boundary and the
// chosen keys on it, in ascending channel order.
template <int KPT>
__global__ __launch_bounds__(1024) void topk_reg_kernel(const double* __restrict__ scores,
                                                        int32_t cols, int32_t k,
                                                        int32_t* __restrict__ out) {
  constexpr int DB = 11, NB = 1 << DB;   // digit bits, bins
  constexpr int BPL = NB / 64;           // bins per lane in the boundary search
  constexpr int kCand = 64;
  __shared__ uint32_t hist[2][NB];
  __shared__ uint64_t s_prefix;
  __shared__ uint64_t s_or[16];
  __shared__ int s_kleft, s_done, s_cnt, s_nc;
  __shared__ int wsum[16];
  __shared__ uint64_t c_key[kCand];
  __shared__ int c_idx[kCand];
  __shared__ int c_rank[kCand];
  const uint64_t* keys = (const uint64_t*)scores;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = tid * KPT;
  uint64_t kv[KPT];
#pragma unroll
  for (int q = 0; q < KPT; ++q) kv[q] = j0 + q < cols ? keys[j0 + q] : 0ull;
  const uint64_t ref = keys[0];
  for (int i = tid; i < NB; i += 1024) hist[0][i] = 0;
  if (tid == 0) s_nc = 0;
  if (tid < kCand) c_rank[tid] = 0;
  // Bits that every key shares need no pass: the radix passes start at the
  // highest bit where two keys differ (OR of key ^ key 0 over all keys).
  uint64_t dx = 0;
#pragma unroll
  for (int q = 0; q < KPT; ++q)
    if (j0 + q < cols) dx |= kv[q] ^ ref;
  for (int o = 32; o >= 1; o >>= 1) dx |= (uint64_t)__shfl_xor((long long)dx, o, 64);
  if (lane == 0) s_or[wave] = dx;
  __syncthreads();
  uint64_t dall = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) dall |= s_or[w];
  const int lead = dall ? __clzll((long long)dall) : 64;   // bits all keys share
  uint64_t mask = lead == 0 ? 0ull : (lead == 64 ? ~0ull : ~0ull << (64 - lead));
  uint64_t prefix = ref & mask;
  int kleft = k;
  bool done = false;
  int cnt = 0x7fffffff;
  // DB-bit digits from the first differing bit down; the last pass may
  // overlap bits already fixed by the prefix (equal on every key it counts)
  int pb = 0;
  for (int shift = 64 - lead - DB; lead < 64; shift -= DB, pb ^= 1) {
    const int sh = shift < 0 ? 0 : shift;
    uint32_t* h = hist[pb];
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const bool valid = j0 + q < cols && (kv[q] & mask) == prefix;
      if (valid) atomicAdd(&h[(uint32_t)(kv[q] >> sh) & (NB - 1)], 1u);
    }
    for (int i = tid; i < NB; i += 1024) hist[pb ^ 1][i] = 0;   // for the next pass
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits NB-1-BPL*l .. NB-BPL-BPL*l (descending); its sum is
      // read in a lane-rotated order (bank-conflict free), then the one lane
      // range holding the k-th key is scanned bin by bin across the wave
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < BPL; ++q) sum += h[NB - 1 - BPL * lane - ((q + lane) & (BPL - 1))];
      uint32_t incl = sum;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += v;
      }
      const uint32_t before = incl - sum;
      const uint64_t hit = __ballot(before < (uint32_t)kleft && incl >= (uint32_t)kleft);
      const int L = hit ? (int)__builtin_ctzll(hit) : 63;   // exactly one lane holds it
      const uint32_t base = (uint32_t)__shfl((int)before, L, 64);
      const int dig = NB - 1 - BPL * L - lane;                  // lanes < BPL: descending digits
      const uint32_t cb = lane < BPL ? h[dig] : 0u;
      uint32_t inc2 = cb;
      for (int o = 1; o < BPL; o <<= 1) {
        const uint32_t v = (uint32_t)__shfl_up((int)inc2, o, 64);
        if (lane >= o) inc2 += v;
      }
      const uint32_t cum = base + inc2 - cb;
      if (lane < BPL && cum < (uint32_t)kleft && cum + cb >= (uint32_t)kleft) {
        s_prefix = prefix | ((uint64_t)dig << sh);
        s_kleft = kleft - (int)cum;
        s_done = (cum + cb == (uint32_t)kleft) ? 1 : 0;   // the whole bin is taken
        s_cnt = (int)cb;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    kleft = s_kleft;
    mask |= (uint64_t)(NB - 1) << sh;
    done = s_done != 0;
    cnt = s_cnt;
    if (done || sh == 0 || cnt <= kCand) break;
  }
  // the boundary bin: taken whole (done), ranked (at most kCand keys), or
  // keys all equal (every bit decided), taken by channel order
  const bool ranked = !done && cnt <= kCand && lead < 64;
  int slot[KPT];
  int eq_rank = 0;
  if (ranked) {
    // candidate slots: a ballot per key position, one atomic per wave
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const bool c = j0 + q < cols && (kv[q] & mask) == prefix;
      const uint64_t b = __ballot(c);
      int base = 0;
      if (b != 0ull) {
        if (lane == 0) base = atomicAdd(&s_nc, (int)__popcll(b));
        base = __shfl(base, 0, 64);
      }
      slot[q] = -1;
      if (c) {
        const int sl = base + (int)__popcll(b & ((1ull << lane) - 1ull));
        c_key[sl] = kv[q];
        c_idx[sl] = j0 + q;
        slot[q] = sl;
      }
    }
    __syncthreads();
    // rank of candidate l = number of candidates before it (key descending,
    // channel ascending); the sixteen waves each compare against every
    // sixteenth candidate and add their counts
    if (lane < cnt) {
      const uint64_t key = c_key[lane];
      const int id = c_idx[lane];
      int r = 0;
      for (int i = wave; i < cnt; i += 16) {
        const uint64_t k2 = c_key[i];
        r += (k2 > key || (k2 == key && c_idx[i] < id)) ? 1 : 0;
      }
      if (r) atomicAdd(&c_rank[lane], r);
    }
    __syncthreads();
  } else if (!done) {
    int neq = 0;
#pragma unroll
    for (int q = 0; q < KPT; ++q) neq += (j0 + q < cols && (kv[q] & mask) == prefix) ? 1 : 0;
    int etot;
    eq_rank = block_excl_scan_int(neq, wsum, &etot);
  }
  bool sel[KPT];
  int nsel = 0;
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const bool valid = j0 + q < cols;
    const uint64_t mk = kv[q] & mask;
    const bool eq = valid && mk == prefix;
    bool take_eq = done;
    if (ranked) take_eq = eq && c_rank[slot[q]] < kleft;
    else if (!done) take_eq = eq_rank < kleft;
    sel[q] = valid && (mk > prefix || (eq && take_eq));
    eq_rank += eq ? 1 : 0;
    nsel += sel[q] ? 1 : 0;
  }
  int tot;
  int pos = block_excl_scan_int(nsel, wsum, &tot);
#pragma unroll
  for (int q = 0; q < KPT; ++q)
    if (sel[q]) out[pos++] = j0 + q;
}

// ====================================================================== gathers
// residual gather (body in q4_prep.h)
template <bool MX, bool UNITS>
__global__ __launch_bounds__(256) void residual_gather_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int32_t cols, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ ts,
    const int32_t* __restrict__ idx, int32_t k, uint16_t* __restrict__ R, int64_t ld_r,
    int32_t* __restrict__ status) {
  const bool ok = chan_set_ok(idx, k, cols);
  if (status && blockIdx.x == 0 && threadIdx.x == 0) status[0] = ok ? 0 : 1;
  residual_gather_part<MX, UNITS>(x, rows, cols, codes, scales, ts, idx, ok ? k : 0, R, ld_r,
                                  blockIdx.x, gridDim.x);
}

// selected weight columns, one 64 x 64 tile per workgroup (body in q4_prep.h)
__global__ __launch_bounds__(256) void wsel_gather_kernel(const uint16_t* __restrict__ w_hi_t,
                                                          int64_t K, int64_t N,
                                                          const int32_t* __restrict__ idx,
                                                          int32_t k, int32_t kp,
                                                          uint16_t* __restrict__ ws,
                                                          const float* __restrict__ w_ts,
                                                          const float* __restrict__ a_ts) {
  __shared__ uint16_t tile[64][66];
  const bool ok = chan_set_ok(idx, k, K);
  wsel_gather_part(w_hi_t, K, N, gridDim.z, idx, ok ? k : 0, kp, ws, blockIdx.z, blockIdx.x, blockIdx.y,
                   tile, w_ts, a_ts);
}

// The same gather in CH x 256 tiles with 8-byte accesses (N % 4 == 0): each
// wave reads one selected row's 256 columns per load (lane l: columns
// 4 l .. 4 l + 3), the tile is transposed through LDS, and each lane writes
// four consecutive channels of one output row.  Tile (bx, by) of matrix b:
// j in [256 bx, 256 bx + 256), t in [CH by, CH by + CH).  The loads go out
// before the channel-set check (every channel is clamped into [0, K)); an
// invalid set then zeroes what they read.
template <int CH>
__global__ __launch_bounds__(256) void wsel_gather_wide_kernel(const uint16_t* __restrict__ w_hi_t,
                                                               int64_t K, int64_t N,
                                                               const int32_t* __restrict__ idx,
                                                               int32_t k, int32_t kp,
                                                               uint16_t* __restrict__ ws,
                                                               const float* __restrict__ w_ts,
                                                               const float* __restrict__ a_ts) {
  constexpr int TP = 264;           // LDS row pitch (u16): 256 columns + 8 of pad
  constexpr int LPR = CH / 4;       // lanes per output row (four channels each)
  constexpr int RPI = 64 / LPR;     // output rows per wave and store
  __shared__ __attribute__((aligned(16))) uint16_t tile[CH][TP];
  const int64_t b = blockIdx.z;
  const int64_t j0 = (int64_t)blockIdx.x * 256;
  const int t0 = blockIdx.y * CH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* src = w_hi_t + b * N;   // channel-major [K][batch][N]
  const int64_t cstride = (int64_t)gridDim.z * N;
  const int64_t jl = j0 + 4 * lane;
  const bool jok = jl < N;   // N % 4 == 0: the lane's four columns are all in or all out
  uint2 v[CH / 4];
#pragma unroll
  for (int q = 0; q < CH / 4; ++q) {
    const int t = t0 + 4 * q + wave;
    int c = t < k ? idx[t] : 0;
    c = c < 0 ? 0 : (c >= K ? (int)K - 1 : c);
    v[q] = (t < k && jok) ? *(const uint2*)(src + (int64_t)c * cstride + jl) : make_uint2(0, 0);
  }
  const bool ok = chan_set_ok(idx, k, K);
  const float rinv = w_ts ? wsel_scale_inv(w_ts[b], a_ts[0]) : 1.0f;
#pragma unroll
  for (int q = 0; q < CH / 4; ++q) {
    uint2 w = ok ? v[q] : make_uint2(0, 0);
    if (w_ts) {
      auto cv = [&](uint32_t x) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(bf16_lo(x) * rinv));
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(bf16_hi(x) * rinv));
        return lo | (hi << 16);
      };
      w = make_uint2(cv(w.x), cv(w.y));
    }
    *(uint2*)&tile[4 * q + wave][4 * lane] = w;
  }
  __syncthreads();
  uint16_t* dst = ws + b * N * kp;
  const int tt = 4 * (lane % LPR);
#pragma unroll
  for (int q = 0; q < 256 / (4 * RPI); ++q) {
    const int jj = 4 * RPI * q + RPI * wave + lane / LPR;
    const int64_t j = j0 + jj;
    const uint32_t a0 = tile[tt][jj], a1 = tile[tt + 1][jj], a2 = tile[tt + 2][jj], a3 = tile[tt + 3][jj];
    if (j < N && t0 + tt < kp) *(uint2*)(dst + j * kp + t0 + tt) = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
  }
}

// out[b][c][r] = in[b][r][c], or (interleave) out[c][b][r] = in[b][r][c]
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int64_t rows, int64_t cols,
                                                             uint16_t* __restrict__ out,
                                                             int32_t interleave) {
  __shared__ uint16_t tile[64][66];
  const int64_t b = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t* src = in + b * rows * cols;
  // output row c of matrix b: interleaved rows c * batch + b
  uint16_t* dst = interleave ? out + b * rows : out + b * rows * cols;
  const int64_t orow = interleave ? (int64_t)gridDim.z * rows : rows;
  for (int r = ty; r < 64; r += 4) {
    const int64_t rr = r0 + r, cc = c0 + tx;
    tile[r][tx] = (rr < rows && cc < cols) ? src[rr * cols + cc] : (uint16_t)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t cc = c0 + r, rr = r0 + tx;
    if (cc < cols && rr < rows) dst[cc * orow + rr] = tile[tx][r];
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
__global__ void tensor_scale_kernel(const float* ts_in, float* ts_out) {
  if (threadIdx.x == 0) ts_out[0] = ts_in ? ts_in[0] : 1.0f;
}

// rows per score tile: 32 (256-row groups), or 8 for a tensor whose 256-row
// groups would make fewer than 128 workgroups, each walking its rows one
// after another (decode-sized activations: 256 x 4096 would be 8 workgroups)
// 8-row score tiles (four times the workgroups) while the 32-row tiles would
// give fewer workgroups than the chip has compute units
static int quant_tile_rows(int64_t rows, int64_t cols) {
  const int64_t units = (rows + 255) / 256 * ((cols + 511) / 512);
  return units < 256 ? 8 : kScoreTileRows;
}

static int64_t score_groups(int64_t rows, int64_t cols) {
  const int64_t g = (int64_t)quant_tile_rows(rows, cols) * kScoreGroupTiles;
  return (rows + g - 1) / g;
}

size_t quantize_workspace_bytes(int64_t rows, int64_t cols) {
  return align256(kAmaxBlocks * 4) +
         align256((size_t)score_groups(rows, cols) * (size_t)cols * 8) + align256((size_t)cols * 8);
}

hipError_t launch_quantize(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                           const float* ts_in, uint8_t* codes, uint8_t* scales, float* ts_out,
                           double* chan_score, int32_t topk, int32_t* chan_idx, void* ws,
                           hipStream_t stream) {
  uint8_t* base = (uint8_t*)ws;
  uint32_t* amax = (uint32_t*)base;
  const int64_t ngroups = score_groups(rows, cols);
  const bool small = quant_tile_rows(rows, cols) != kScoreTileRows;
  const size_t amax_bytes = align256(kAmaxBlocks * 4);
  double* partial = (double*)(base + amax_bytes);
  double* scores = chan_score ? chan_score
                              : (double*)(base + amax_bytes + align256((size_t)ngroups * cols * 8));
  const bool need_amax = !mx && ts_in == nullptr;
  int32_t namax = 0;
  if (need_amax) {
    const int64_t n16 = rows * cols / 8;
    if (n16 > 0) {
      // two workgroups per CU (on 16384 x 7168 bf16 read cold from HBM: 1.8 us
      // faster than one per CU, no gain from twice the loads in flight)
      int64_t grid = (n16 + kAmaxSeg - 1) / kAmaxSeg;
      grid = grid < 1 ? 1 : (grid > 512 ? 512 : grid);
      namax = (int32_t)grid;
      hipLaunchKernelGGL(amax_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                         (const uint4*)x, n16, amax);
    }
  }
  QuantKArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = (int32_t)cols;
  // 16 channels per lane halves the per-block work; 8 per lane when that
  // would leave fewer than 256 workgroups (one per CU)
  const bool wide = !small && ngroups * ((cols + 1023) / 1024) >= 256;
  a.nstrips = (int32_t)(wide ? (cols + 1023) / 1024 : (cols + 511) / 512);
  a.ngroups = ngroups;
  a.ts_in = ts_in;
  a.amax = amax;
  a.namax = namax;
  a.codes = codes;
  a.scales = scales;
  a.ts_out = ts_out;
  a.partial = partial;
  a.reverse = need_amax ? 1 : 0;
  const int64_t units = ngroups * a.nstrips;
  if (units > 0) {
    const unsigned grid = (unsigned)units;
    if (small && mx)
      hipLaunchKernelGGL((quantize_kernel<true, 8, 8>), dim3(grid), dim3(512), 0, stream, a);
    else if (small)
      hipLaunchKernelGGL((quantize_kernel<false, 8, 8>), dim3(grid), dim3(512), 0, stream, a);
    else if (mx && wide)
      hipLaunchKernelGGL((quantize_kernel<true, 16>), dim3(grid), dim3(512), 0, stream, a);
    else if (mx)
      hipLaunchKernelGGL((quantize_kernel<true, 8>), dim3(grid), dim3(512), 0, stream, a);
    else if (wide)
      hipLaunchKernelGGL((quantize_kernel<false, 16>), dim3(grid), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((quantize_kernel<false, 8>), dim3(grid), dim3(512), 0, stream, a);
  } else if (!mx && ts_out) {
    // no rows: still report s_t (1, or the supplied value)
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(64), 0, stream, ts_in, ts_out);
  }
  launch_score_reduce_host((const double*)partial, ngroups, cols, scores, stream);
  if (topk > 0) return launch_select(scores, cols, topk, chan_idx, stream);
  return hipGetLastError();
}

hipError_t launch_score_reduce_dev(const double* partial, const int32_t* ngroups_dev, int32_t mult,
                                   int64_t cols, double* scores, hipStream_t stream) {
  if (cols <= 0) return hipSuccess;
  // (the half-tile sums of a prefill-shaped layer: hundreds of rows)
  hipLaunchKernelGGL(score_reduce_kernel<16>, dim3((unsigned)((cols + 63) / 64)), dim3(1024), 0,
                     stream, partial, (int64_t)0, (int32_t)cols, scores, ngroups_dev, mult);
  return hipGetLastError();
}

hipError_t launch_copy_scale(const float* ts_in, float* ts_out, hipStream_t stream) {
  hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(64), 0, stream, ts_in, ts_out);
  return hipGetLastError();
}

hipError_t launch_select(const double* scores, int64_t cols, int32_t topk, int32_t* idx,
                         hipStream_t stream) {
  if (topk <= 0) return hipSuccess;
  const int c = (int)cols;
  if (cols <= 1024)
    hipLaunchKernelGGL(topk_reg_kernel<1>, dim3(1), dim3(1024), 0, stream, scores, c, topk, idx);
  else if (cols <= 2048)
    hipLaunchKernelGGL(topk_reg_kernel<2>, dim3(1), dim3(1024), 0, stream, scores, c, topk, idx);
  else if (cols <= 4096)
    hipLaunchKernelGGL(topk_reg_kernel<4>, dim3(1), dim3(1024), 0, stream, scores, c, topk, idx);
  else if (cols <= 8192)
    hipLaunchKernelGGL(topk_reg_kernel<8>, dim3(1), dim3(1024), 0, stream, scores, c, topk, idx);
  else if (cols <= 16384)
    hipLaunchKernelGGL(topk_reg_kernel<16>, dim3(1), dim3(1024), 0, stream, scores, c, topk, idx);
  else
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(1024), 0, stream, scores, c, topk, idx);
  return hipGetLastError();
}

// ====================================================================== QDQ
// Trainer-side weight fake quantization (QUADS section 3.2, Eq. 12): the value
// each code stands for, c sb s_t, from codes, E4M3 scales and the tensor
// scale.  One thread per 16-element block.  fp32 output: (c sb) s_t with one
// rounding (c sb is exact in fp32).  bf16 output: the exact value (c sb has at
// most 6 significant bits, s_t 24: exact in fp64) rounded once to bf16, by
// round-to-odd to fp32 (24 >= 8 + 2 bits, so the second rounding is exact)
// and then to nearest even.
__global__ __launch_bounds__(256) void dequant_nvfp4_kernel(const uint2* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ ts,
                                                            int64_t nblocks, int32_t y_bf16,
                                                            void* __restrict__ y) {
  const float st = ts[0];
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * 256) {
    const uint2 cw = codes[b];
    const float s = e4m3_to_f32(scales[b]);
    float v[16];
    const uint32_t cws[2] = {cw.x, cw.y};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f32x2v c2[4];
      c2[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 0);
      c2[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 1);
      c2[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 2);
      c2[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cws[q], 1.0f, 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = c2[j].x * s;
        v[8 * q + 2 * j + 1] = c2[j].y * s;
      }
    }
    if (y_bf16) {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t h[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const double ex = (double)v[2 * i + u] * (double)st;
          float f = __double2float_rz(ex);
          if ((double)f != ex) f = __uint_as_float(__float_as_uint(f) | 1u);
          h[u] = f32_to_bf16_rne(f);
        }
        o[i] = h[0] | (h[1] << 16);
      }
      uint4* dst = (uint4*)((uint16_t*)y + b * 16);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
      float4* dst = (float4*)((float*)y + b * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_float4(v[4 * i] * st, v[4 * i + 1] * st, v[4 * i + 2] * st, v[4 * i + 3] * st);
    }
  }
}

hipError_t launch_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* ts,
                                int64_t rows, int64_t cols, int32_t y_bf16, void* y,
                                hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 16);
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  grid = grid > 8192 ? 8192 : grid;
  hipLaunchKernelGGL(dequant_nvfp4_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint2*)codes, scales, ts, nblocks, y_bf16, y);
  return hipGetLastError();
}

hipError_t launch_residual_gather(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                                  const uint8_t* codes, const uint8_t* scales, const float* ts,
                                  const int32_t* idx, int32_t k, uint16_t* R, int64_t ld_r,
                                  hipStream_t stream, int32_t* status, bool units) {
  const int64_t total = residual_gather_items(rows, ld_r);
  if (total == 0 && !status) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  grid = grid > 65536 ? 65536 : (grid < 1 ? 1 : grid);
  if (mx)
    hipLaunchKernelGGL((residual_gather_kernel<true, false>), dim3((unsigned)grid), dim3(256), 0,
                       stream, x, rows, (int32_t)cols, codes, scales, ts, idx, k, R, ld_r, status);
  else if (units)
    hipLaunchKernelGGL((residual_gather_kernel<false, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, x, rows, (int32_t)cols, codes, scales, ts, idx, k, R, ld_r, status);
  else
    hipLaunchKernelGGL((residual_gather_kernel<false, false>), dim3((unsigned)grid), dim3(256), 0,
                       stream, x, rows, (int32_t)cols, codes, scales, ts, idx, k, R, ld_r, status);
  return hipGetLastError();
}

hipError_t launch_wsel_gather(const uint16_t* w_hi_t, int64_t batch, int64_t K, int64_t N,
                              const int32_t* idx, int32_t k, int32_t kp, uint16_t* ws,
                              hipStream_t stream, const float* w_ts, const float* a_ts) {
  if (batch == 0 || N == 0 || kp == 0) return hipSuccess;
  if (N % 4 == 0) {
    constexpr int CH = 32;   // channels per workgroup
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)((kp + CH - 1) / CH), (unsigned)batch);
    hipLaunchKernelGGL(wsel_gather_wide_kernel<CH>, grid, dim3(256), 0, stream, w_hi_t, K, N, idx,
                       k, kp, ws, w_ts, a_ts);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((kp + 63) / 64), (unsigned)batch);
  hipLaunchKernelGGL(wsel_gather_kernel, grid, dim3(256), 0, stream, w_hi_t, K, N, idx, k, kp, ws,
                     w_ts, a_ts);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t batch, int64_t rows, int64_t cols,
                                 uint16_t* out, hipStream_t stream, bool interleave) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)batch);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, in, rows, cols, out,
                     interleave ? 1 : 0);
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
