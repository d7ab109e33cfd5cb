// Top-k MoE routing, token sort and combine for the grouped expert layer
// (gfx950).  The QUADS page (arXiv 2607.15810, section 3.3) compensates MoE
// projections -- the W13 activation site -- without spelling out the MoE block;
// these kernels implement the standard top-k softmax router and a
// deterministic token-sorted layout for a grouped GEMM.
#include "q4_internal.h"

namespace q4 {

// ====================================================================== route
// one wave per token: repeated arg-max over the logits (ties -> smaller
// expert), then softmax over the selected logits
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int64_t T,
                                                        int32_t E, int32_t topk,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lg = logits + t * E;
  constexpr int MAXPER = 16;   // E <= 1024
  float v[MAXPER];
  const int per = (E + 63) / 64;
#pragma unroll
  for (int q = 0; q < MAXPER; ++q) {
    const int ex = q * 64 + lane;
    v[q] = (q < per && ex < E) ? lg[ex] : -INFINITY;
  }
  bool taken[MAXPER];
#pragma unroll
  for (int q = 0; q < MAXPER; ++q) taken[q] = !(q < per && q * 64 + lane < E);
  float sel[16];
  int sel_e[16];
  for (int s = 0; s < topk; ++s) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) {
      const int ex = q * 64 + lane;
      if (!taken[q] && (v[q] > bv || (v[q] == bv && ex < be))) {
        bv = v[q];
        be = ex;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
#pragma unroll
    for (int q = 0; q < MAXPER; ++q)
      if (q * 64 + lane == be) taken[q] = true;
    sel[s] = bv;
    sel_e[s] = be;
  }
  if (lane == 0) {
    const float mx = sel[0];
    float sum = 0.0f;
    float ex[16];
    for (int s = 0; s < topk; ++s) {
      ex[s] = __expf(sel[s] - mx);
      sum += ex[s];
    }
    for (int s = 0; s < topk; ++s) {
      idx[t * topk + s] = sel_e[s];
      w[t * topk + s] = ex[s] / sum;
    }
  }
}

// ====================================================================== sort
// block-wide exclusive scan of 0/1 flags (ballot + per-wave counts)
__device__ __forceinline__ int block_scan_flag(bool flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint64_t b = __ballot(flag);
  const int in_wave = __popcll(b & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wsum[wv] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int c = wsum[i];
    before += (i < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

// counts[e] = number of routed rows (t, s) with idx == e
__global__ __launch_bounds__(1024) void moe_count_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                         int32_t* __restrict__ counts) {
  __shared__ int wsum[16];
  const int e = blockIdx.x;
  int c = 0;
  for (int64_t b0 = 0; b0 < n; b0 += 1024) {
    const int64_t i = b0 + threadIdx.x;
    int tot;
    block_scan_flag(i < n && idx[i] == e, wsum, &tot);
    c += tot;
  }
  if (threadIdx.x == 0) counts[e] = c;
}

// offsets = exclusive scan of counts; one M tile entry {e, begin, end, 0} per
// kGemmBM rows of each expert
__global__ __launch_bounds__(1024) void moe_offsets_kernel(const int32_t* __restrict__ counts,
                                                           int32_t E, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles) {
  __shared__ int s_off[1025];
  __shared__ int s_tile[1025];
  if (threadIdx.x == 0) {
    int o = 0, tcount = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = o;
      s_tile[e] = tcount;
      o += counts[e];
      tcount += (counts[e] + kGemmBM - 1) / kGemmBM;
    }
    s_off[E] = o;
    s_tile[E] = tcount;
    ntiles[0] = tcount;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int nt = s_tile[e + 1] - s_tile[e];
    for (int q = 0; q < nt; ++q) {
      int4 v;
      v.x = e;
      v.y = s_off[e] + q * kGemmBM;
      v.z = min(s_off[e] + (q + 1) * kGemmBM, s_off[e + 1]);
      v.w = 0;
      ((int4*)tiles)[s_tile[e] + q] = v;
    }
  }
}

// stable scatter: rows of expert e in flat (t, s) order
__global__ __launch_bounds__(1024) void moe_scatter_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv_perm) {
  __shared__ int wsum[16];
  const int e = blockIdx.x;
  int base = offsets[e];
  for (int64_t b0 = 0; b0 < n; b0 += 1024) {
    const int64_t i = b0 + threadIdx.x;
    const bool f = i < n && idx[i] == e;
    int tot;
    const int r = block_scan_flag(f, wsum, &tot);
    if (f) {
      perm[base + r] = (int32_t)i;
      inv_perm[i] = base + r;
    }
    base += tot;
  }
}

__global__ __launch_bounds__(256) void moe_arows_kernel(const int32_t* __restrict__ perm, int64_t n,
                                                        int32_t topk, int32_t* __restrict__ a_rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < n) a_rows[r] = perm[r] / topk;
}

// y[t][h] = sum over slots s = 0..topk-1 of w[t][s] * out[inv_perm[t*topk+s]][h]
// (fp32, slot order fixed).  One workgroup per (token, 1024 columns).
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ out,
                                                          const int32_t* __restrict__ inv_perm,
                                                          const float* __restrict__ w, int64_t T,
                                                          int32_t topk, int32_t H, void* Y,
                                                          int32_t y_bf16) {
  const int nch = (H + 1023) / 1024;
  const int64_t t = blockIdx.x / nch;
  const int h0 = (int)(blockIdx.x % nch) * 1024 + threadIdx.x * 4;
  if (t >= T || h0 >= H) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int s = 0; s < topk; ++s) {
    const float p = w[t * topk + s];
    const int64_t r = inv_perm[t * topk + s];
    const float4 v = *(const float4*)(out + r * H + h0);
    a0 = fmaf(p, v.x, a0);
    a1 = fmaf(p, v.y, a1);
    a2 = fmaf(p, v.z, a2);
    a3 = fmaf(p, v.w, a3);
  }
  if (y_bf16) {
    uint2 o;
    o.x = f32_to_bf16_rne(a0) | (f32_to_bf16_rne(a1) << 16);
    o.y = f32_to_bf16_rne(a2) | (f32_to_bf16_rne(a3) << 16);
    *(uint2*)((uint16_t*)Y + t * H + h0) = o;
  } else {
    *(float4*)((float*)Y + t * H + h0) = make_float4(a0, a1, a2, a3);
  }
}

// ====================================================================== launchers
hipError_t launch_moe_route(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* idx,
                            float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream,
                     logits, T, E, topk, idx, w);
  return hipGetLastError();
}

size_t moe_sort_workspace_bytes(int64_t T, int32_t E, int32_t topk) {
  (void)T;
  (void)topk;
  return align256((size_t)E * 4);
}

hipError_t launch_moe_sort(const int32_t* idx, int64_t T, int32_t E, int32_t topk, int32_t* perm,
                           int32_t* offsets, int32_t* inv_perm, int32_t* tiles, int32_t* ntiles,
                           int32_t* counts, hipStream_t stream) {
  const int64_t n = T * topk;
  hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)E), dim3(1024), 0, stream, idx, n, counts);
  hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(1024), 0, stream, (const int32_t*)counts,
                     E, offsets, tiles, ntiles);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3((unsigned)E), dim3(1024), 0, stream, idx, n,
                     (const int32_t*)offsets, perm, inv_perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows_index(const int32_t* perm, int64_t n, int32_t topk, int32_t* a_rows,
                                   hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_arows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     perm, n, topk, a_rows);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* out, const int32_t* inv_perm, const float* topk_w,
                              int64_t T, int32_t topk, int32_t H, void* Y, int32_t y_bf16,
                              hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t nch = (H + 1023) / 1024;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)(T * nch)), dim3(256), 0, stream, out,
                     inv_perm, topk_w, T, topk, H, Y, y_bf16);
  return hipGetLastError();
}

}  // namespace q4
