// Top-k MoE routing, token sort and combine for the grouped expert layer
// (gfx950).  The QUADS page (arXiv 2607.15810, section 3.3) compensates MoE
// projections -- the W13 activation site -- without spelling out the MoE block;
// these kernels implement the standard top-k softmax router and a
// deterministic token-sorted layout for a grouped GEMM.
#include "q4_internal.h"

namespace q4 {

// ====================================================================== route
// 64-bit value of lane (lane's DPP source under CTRL), every lane active
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t k) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xf,
                                                            0xf, false);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xf, 0xf,
                                                            false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t k, int l) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, l);
  return ((uint64_t)hi << 32) | lo;
}

// one wave per token: repeated arg-max over the logits (ties -> smaller
// expert), then softmax over the selected logits.  MAXPER logits per lane
// (E <= 64 MAXPER).
template <int MAXPER>
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int64_t T,
                                                        int32_t E, int32_t topk,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lg = logits + t * E;
  float v[MAXPER];
  const int per = (E + 63) / 64;
#pragma unroll
  for (int q = 0; q < MAXPER; ++q) {
    const int ex = q * 64 + lane;
    // a NaN logit ranks below every number (as -inf; ties to the smaller
    // expert), so every token gets topk distinct experts in [0, E)
    const float l = (q < per && ex < E) ? lg[ex] : -INFINITY;
    v[q] = l == l ? l : -INFINITY;
  }
  bool taken[MAXPER];
#pragma unroll
  for (int q = 0; q < MAXPER; ++q) taken[q] = !(q < per && q * 64 + lane < E);
  // Each candidate is one 64-bit key: the logit's bits in an order-keeping
  // form above the complement of the expert index, so the largest key is the
  // largest logit and, among equal logits, the smaller expert (-0 counts as
  // +0, as the float comparison has it).  A taken (or absent) candidate is
  // key 0, below every logit, -inf included.
  auto key_of = [](float x, int ex) {
    const uint32_t u = __float_as_uint(x + 0.0f);   // -0 -> +0: equal logits, equal keys
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)~ex;
  };
  float sel[16];
  int sel_e[16];
  for (int s = 0; s < topk; ++s) {
    uint64_t kb = 0;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q)
      if (!taken[q]) kb = max(kb, key_of(v[q], q * 64 + lane));
    // wave maximum: within rows of 16 lanes by DPP (lane pairs, quads,
    // half rows, rows), then over the four rows' lanes 0, 16, 32, 48
    kb = max(kb, dpp_u64<0xB1>(kb));    // quad_perm [1, 0, 3, 2]
    kb = max(kb, dpp_u64<0x4E>(kb));    // quad_perm [2, 3, 0, 1]
    kb = max(kb, dpp_u64<0x141>(kb));   // row_half_mirror
    kb = max(kb, dpp_u64<0x140>(kb));   // row_mirror
    kb = max(max(readlane_u64(kb, 0), readlane_u64(kb, 16)),
             max(readlane_u64(kb, 32), readlane_u64(kb, 48)));
    const int be = (int)~(uint32_t)kb;
    const uint32_t o = (uint32_t)(kb >> 32);
#pragma unroll
    for (int q = 0; q < MAXPER; ++q)
      if (q * 64 + lane == be) taken[q] = true;
    sel[s] = __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
    sel_e[s] = be;
  }
  if (lane == 0) {
    const float mx = sel[0];
    float sum = 0.0f;
    float ex[16];
    for (int s = 0; s < topk; ++s) {
      // equal to the largest: weight 1 before normalisation (also when every
      // selected logit is -inf, which then gives uniform weights)
      ex[s] = sel[s] == mx ? 1.0f : __expf(sel[s] - mx);
      sum += ex[s];
    }
    for (int s = 0; s < topk; ++s) {
      idx[t * topk + s] = sel_e[s];
      w[t * topk + s] = ex[s] / sum;
    }
  }
}

// ====================================================================== sort
// The token sort is a stable counting sort over blocks of 1024 routed rows:
// per-block expert histograms, per-expert bases (one thread per expert walks
// the blocks in order), then a scatter in which each row's rank inside its
// block comes from its rank inside its wave (wave_rank) and per-wave counts.

// An expert index outside [0, E) is invalid: it is counted as expert 0 (so
// every index the sort writes stays in bounds), its slot gets weight 0 in the
// combine, and the call's status word reports Q4_EINVAL.
__device__ __forceinline__ int routed_expert(const int32_t* __restrict__ idx, int64_t i, bool valid,
                                             int32_t E, bool& bad) {
  const int e = valid ? idx[i] : -1;
  bad = valid && (e < 0 || e >= E);
  return bad ? 0 : e;
}

// Rank of this lane's expert among the wave's lanes below it with the same
// expert, and (last) whether no lane above it has that expert: the wave's 64
// experts go to its LDS row `ids` and every lane compares against all of them
// (sixteen 16-byte broadcast reads), so the cost does not grow with the number
// of distinct experts in the wave.  Invalid lanes take part with key -1, which
// no expert equals, and get last = false.
__device__ __forceinline__ int wave_rank(int e, bool valid, int* ids, bool& last) {
  const int lane = threadIdx.x & 63;
  const int key = valid ? e : -1;
  ids[lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int below = 0, above = 0;
#pragma unroll
  for (int j4 = 0; j4 < 16; ++j4) {
    const int4 v = ((const int4*)ids)[j4];
    const int k[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 4 * j4 + c;
      const int eq = k[c] == key ? 1 : 0;
      below += j < lane ? eq : 0;
      above += j > lane ? eq : 0;
    }
  }
  // the row is reused by the next call: every lane has read it first
  __builtin_amdgcn_wave_barrier();
  last = valid && above == 0;
  return below;
}

// bt[b][e] = rows of block b routed to expert e; flags[b] = block b holds an
// invalid expert index
__global__ __launch_bounds__(1024) void moe_block_hist_kernel(const int32_t* __restrict__ idx,
                                                              int64_t n, int32_t E,
                                                              int32_t* __restrict__ bt,
                                                              int32_t* __restrict__ flags) {
  __shared__ int hist[1024];
  __shared__ int ids[16][64];
  const int wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 1024) hist[e] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  const bool valid = i < n;
  bool bad;
  const int e = routed_expert(idx, i, valid, E, bad);
  const int any_bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) flags[blockIdx.x] = any_bad;
  bool last;
  const int rank = wave_rank(e, valid, ids[wv], last);
  if (last) atomicAdd(&hist[e], rank + 1);
  __syncthreads();
  for (int q = threadIdx.x; q < E; q += 1024) bt[(int64_t)blockIdx.x * E + q] = hist[q];
}

// Per-expert offsets and tile starts as exclusive prefix sums over e < E of
// the counts s_cnt[e], ceil(s_cnt[e] / kGemmBM) and (bm2 > 0) ceil(s_cnt[e] /
// bm2), totals at index E; also writes ntiles[0] and ntiles2[0].  Needs a
// 1024-thread workgroup and E <= 1024; wave shuffles, then the waves' totals
// through LDS (no serial walk over the experts).
__device__ __forceinline__ void expert_scan(const int* s_cnt, int32_t E, int bm2, int* s_off,
                                            int* s_tile, int* s_tile2, int (*wsum)[3],
                                            int32_t* __restrict__ ntiles,
                                            int32_t* __restrict__ ntiles2) {
  const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
  const int c = e < E ? s_cnt[e] : 0;
  const int v[3] = {c, (c + kGemmBM - 1) / kGemmBM, bm2 > 0 ? (c + bm2 - 1) / bm2 : 0};
  int inc[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int u = __shfl_up(inc[q], o, 64);
      if (lane >= o) inc[q] += u;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 3; ++q) wsum[wv][q] = inc[q];
  }
  __syncthreads();
  int base[3] = {0, 0, 0};
  for (int w = 0; w < wv; ++w) {
#pragma unroll
    for (int q = 0; q < 3; ++q) base[q] += wsum[w][q];
  }
  int* const out[3] = {s_off, s_tile, s_tile2};
  if (e < E) {
#pragma unroll
    for (int q = 0; q < 3; ++q) out[q][e] = base[q] + inc[q] - v[q];
  }
  if (e == E - 1) {
#pragma unroll
    for (int q = 0; q < 3; ++q) out[q][E] = base[q] + inc[q];
    ntiles[0] = base[1] + inc[1];
    if (ntiles2) ntiles2[0] = base[2] + inc[2];
  }
  __syncthreads();
}

// tile entries {e, begin, end, 0}, at most bm rows each, for every expert
__device__ __forceinline__ void write_tiles(const int* s_off, const int* s_tile, int32_t E, int bm,
                                            int32_t* __restrict__ tiles) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int nt = s_tile[e + 1] - s_tile[e];
    for (int q = 0; q < nt; ++q) {
      int4 v;
      v.x = e;
      v.y = s_off[e] + q * bm;
      v.z = min(s_off[e] + (q + 1) * bm, s_off[e + 1]);
      v.w = 0;
      ((int4*)tiles)[s_tile[e] + q] = v;
    }
  }
}

// counts and offsets per expert, bt[b][e] -> rows of expert e in blocks
// before b, one M tile entry {e, begin, end, 0} per kGemmBM rows and, when
// tiles2 is given, a second table with bm2 rows per tile
__global__ __launch_bounds__(1024) void moe_offsets_kernel(int32_t* __restrict__ bt, int64_t nb,
                                                           int32_t E, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles, int32_t bm2,
                                                           int32_t* __restrict__ tiles2,
                                                           int32_t* __restrict__ ntiles2,
                                                           const int32_t* __restrict__ flags,
                                                           int32_t* __restrict__ status) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_tile[1025];
  __shared__ int s_tile2[1025];
  __shared__ int wsum[16][3];
  int bad = 0;
  for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) bad |= flags[b];
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0 && status) status[0] = bad ? 1 : 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // sixteen blocks' counts loaded before any is rewritten, so the walk
    // waits for one load round trip per sixteen blocks
    int c = 0;
    for (int64_t b0 = 0; b0 < nb; b0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = b0 + u < nb ? bt[(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (b0 + u < nb) bt[(b0 + u) * E + e] = c;
        c += v[u];
      }
    }
    s_cnt[e] = c;
  }
  __syncthreads();
  expert_scan(s_cnt, E, tiles2 ? bm2 : 0, s_off, s_tile, s_tile2, wsum, ntiles,
              tiles2 ? ntiles2 : nullptr);
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  write_tiles(s_off, s_tile, E, kGemmBM, tiles);
  if (tiles2) write_tiles(s_off, s_tile2, E, bm2, tiles2);
}

// stable scatter: rows of expert e in flat (t, s) order
__global__ __launch_bounds__(1024) void moe_scatter_kernel(const int32_t* __restrict__ idx,
                                                           int64_t n, int32_t E,
                                                           const int32_t* __restrict__ bt,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv_perm,
                                                           int32_t topk,
                                                           int32_t* __restrict__ a_rows) {
  __shared__ int wcnt[16][1024];
  __shared__ int ids[16][64];
  const int wv = threadIdx.x >> 6;
  for (int q = threadIdx.x; q < 16 * E; q += 1024) wcnt[q / E][q % E] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  const bool valid = i < n;
  bool bad;
  const int e = routed_expert(idx, i, valid, E, bad);
  bool last;
  int rank = wave_rank(e, valid, ids[wv], last);
  if (last) wcnt[wv][e] = rank + 1;
  __syncthreads();
  if (valid) {
    for (int w = 0; w < wv; ++w) rank += wcnt[w][e];
    const int pos = offsets[e] + bt[(int64_t)blockIdx.x * E + e] + rank;
    perm[pos] = (int32_t)i;
    inv_perm[i] = pos;
    if (a_rows) a_rows[pos] = (int32_t)(i / topk);
  }
}

// The whole sort in one workgroup for few routed rows (decode-shaped layers,
// n <= kSortSmallBlocks * 1024): expert counts, offsets and tile tables, then
// the stable scatter block by block in flat order (in-wave ranks and per-wave
// counts, a running base per expert).  Same outputs as the three
// kernels above, one launch instead of three.
constexpr int kSortSmallBlocks = 8;
__global__ __launch_bounds__(1024) void moe_sort_small_kernel(
    const int32_t* __restrict__ idx, int64_t n, int32_t E, int32_t topk,
    int32_t* __restrict__ perm, int32_t* __restrict__ offsets, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles, int32_t* __restrict__ a_rows,
    int32_t bm2, int32_t* __restrict__ tiles2, int32_t* __restrict__ ntiles2,
    int32_t* __restrict__ status) {
  __shared__ int wcnt[16][1024];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_tile[1025];
  __shared__ int s_tile2[1025];
  __shared__ int wsum[16][3];
  __shared__ int ids[16][64];
  const int wv = threadIdx.x >> 6;
  const int nb = (int)((n + 1023) / 1024);
  for (int e = threadIdx.x; e < E; e += 1024) s_cnt[e] = 0;
  for (int q = threadIdx.x; q < 16 * E; q += 1024) wcnt[q / E][q % E] = 0;
  __syncthreads();
  // counts; each thread keeps its rows' experts, in-wave ranks and
  // last-of-expert flags for the scatter
  int ex[kSortSmallBlocks], rk[kSortSmallBlocks];
  bool lst[kSortSmallBlocks];
  int bad_any = 0;
#pragma unroll
  for (int b = 0; b < kSortSmallBlocks; ++b) {
    const int64_t i = (int64_t)b * 1024 + threadIdx.x;
    const bool valid = b < nb && i < n;
    bool bad;
    ex[b] = routed_expert(idx, i, valid, E, bad);
    bad_any |= bad;
    rk[b] = b < nb ? wave_rank(ex[b], valid, ids[wv], lst[b]) : 0;
    if (b >= nb) lst[b] = false;
    if (lst[b]) atomicAdd(&s_cnt[ex[b]], rk[b] + 1);
  }
  bad_any = __syncthreads_or(bad_any);
  if (threadIdx.x == 0 && status) status[0] = bad_any ? 1 : 0;
  expert_scan(s_cnt, E, tiles2 ? bm2 : 0, s_off, s_tile, s_tile2, wsum, ntiles,
              tiles2 ? ntiles2 : nullptr);
  for (int e = threadIdx.x; e <= E; e += 1024) offsets[e] = s_off[e];
  write_tiles(s_off, s_tile, E, kGemmBM, tiles);
  if (tiles2) write_tiles(s_off, s_tile2, E, bm2, tiles2);
  // s_cnt becomes the running base of each expert
  for (int e = threadIdx.x; e < E; e += 1024) s_cnt[e] = s_off[e];
  __syncthreads();
#pragma unroll
  for (int b = 0; b < kSortSmallBlocks; ++b) {
    if (b >= nb) break;                        // uniform
    const int64_t i = (int64_t)b * 1024 + threadIdx.x;
    const bool valid = i < n;
    const int e = ex[b];
    int rank = rk[b];
    if (lst[b]) wcnt[wv][e] = rank + 1;
    __syncthreads();
    if (valid) {
      for (int w = 0; w < wv; ++w) rank += wcnt[w][e];
      const int pos = s_cnt[e] + rank;
      perm[pos] = (int32_t)i;
      inv_perm[i] = pos;
      if (a_rows) a_rows[pos] = (int32_t)(i / topk);
    }
    __syncthreads();
    // advance the bases past this block and clear the wave counts
    for (int e2 = threadIdx.x; e2 < E; e2 += 1024) {
      int add = 0;
      for (int w = 0; w < 16; ++w) {
        add += wcnt[w][e2];
        wcnt[w][e2] = 0;
      }
      s_cnt[e2] += add;
    }
    __syncthreads();
  }
}

// y[t][h] = sum over slots s = 0..topk-1 of w[t][s] * out[inv_perm[t*topk+s]][h]
// (fp32 sums, slot order fixed; a slot with an invalid expert index
// contributes nothing).  The W2 rows `out` are fp32 (IN_BF16 false) or bf16:
// the expert outputs are rounded to the layer's output type before they are
// combined.  A lane takes C columns (one 16-byte load per slot), a workgroup
// 256 C columns of one token.
template <bool IN_BF16>
__global__ __launch_bounds__(256) void moe_combine_kernel(const void* __restrict__ out,
                                                          const int32_t* __restrict__ inv_perm,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ idx,
                                                          int32_t E, int64_t T, int32_t topk,
                                                          int32_t H, void* Y, int32_t y_bf16) {
  constexpr int C = IN_BF16 ? 8 : 4;
  const int nch = (H + 256 * C - 1) / (256 * C);
  const int64_t t = blockIdx.x / nch;
  const int h0 = (int)(blockIdx.x % nch) * (256 * C) + threadIdx.x * C;
  if (t >= T || h0 >= H) return;   // H % C == 0: a lane's columns are all in or all out
  float a[C];
#pragma unroll
  for (int i = 0; i < C; ++i) a[i] = 0.0f;
  for (int s = 0; s < topk; ++s) {
    const int32_t ex = idx[t * topk + s];
    const float p = (ex >= 0 && ex < E) ? w[t * topk + s] : 0.0f;
    const int64_t r = inv_perm[t * topk + s];
    // each W2 row is read once: nontemporal (16 bytes; the elements are
    // taken by name, not by a subscript of the loaded vector)
    if constexpr (IN_BF16) {
      const uint4 v = __builtin_bit_cast(
          uint4, __builtin_nontemporal_load((const u32x4v*)((const uint16_t*)out + r * H + h0)));
      const uint32_t pair[4] = {v.x, v.y, v.z, v.w};   // two bf16 columns each
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[2 * i] = fmaf(p, __builtin_bit_cast(float, pair[i] << 16), a[2 * i]);
        a[2 * i + 1] = fmaf(p, __builtin_bit_cast(float, pair[i] & 0xffff0000u), a[2 * i + 1]);
      }
    } else {
      const f32x4v v = __builtin_nontemporal_load((const f32x4v*)((const float*)out + r * H + h0));
      a[0] = fmaf(p, v.x, a[0]);
      a[1] = fmaf(p, v.y, a[1]);
      a[2] = fmaf(p, v.z, a[2]);
      a[3] = fmaf(p, v.w, a[3]);
    }
  }
  if (y_bf16) {
    uint32_t o[C / 2];
#pragma unroll
    for (int i = 0; i < C / 2; ++i)
      o[i] = f32_to_bf16_rne(a[2 * i]) | (f32_to_bf16_rne(a[2 * i + 1]) << 16);
    if constexpr (C == 8)
      *(uint4*)((uint16_t*)Y + t * H + h0) = make_uint4(o[0], o[1], o[2], o[3]);
    else
      *(uint2*)((uint16_t*)Y + t * H + h0) = make_uint2(o[0], o[1]);
  } else {
#pragma unroll
    for (int i = 0; i < C; i += 4)
      *(float4*)((float*)Y + t * H + h0 + i) = make_float4(a[i], a[i + 1], a[i + 2], a[i + 3]);
  }
}

// ====================================================================== launchers
hipError_t launch_moe_route(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* idx,
                            float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4));
  if (E <= 128)
    hipLaunchKernelGGL(moe_route_kernel<2>, grid, dim3(256), 0, stream, logits, T, E, topk, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(moe_route_kernel<4>, grid, dim3(256), 0, stream, logits, T, E, topk, idx, w);
  else
    hipLaunchKernelGGL(moe_route_kernel<16>, grid, dim3(256), 0, stream, logits, T, E, topk, idx, w);
  return hipGetLastError();
}

// block histograms [nb][E], then one invalid-index flag per block
size_t moe_sort_workspace_bytes(int64_t T, int32_t E, int32_t topk) {
  const int64_t nb = (T * topk + 1023) / 1024;
  const size_t b = (size_t)(nb > 0 ? nb : 1);
  return align256(b * E * 4) + align256(b * 4);
}

hipError_t launch_moe_sort(const int32_t* idx, int64_t T, int32_t E, int32_t topk, int32_t* perm,
                           int32_t* offsets, int32_t* inv_perm, int32_t* tiles, int32_t* ntiles,
                           int32_t* counts, hipStream_t stream, int32_t* a_rows, int32_t bm2,
                           int32_t* tiles2, int32_t* ntiles2, int32_t* status) {
  const int64_t n = T * topk;
  const int64_t nb = (n + 1023) / 1024;
  if (nb <= kSortSmallBlocks && E <= 1024) {
    hipLaunchKernelGGL(moe_sort_small_kernel, dim3(1), dim3(1024), 0, stream, idx, n, E, topk,
                       perm, offsets, inv_perm, tiles, ntiles, a_rows, bm2, tiles2, ntiles2,
                       status);
    return hipGetLastError();
  }
  int32_t* flags = counts + align256((size_t)(nb > 0 ? nb : 1) * E * 4) / 4;
  if (nb > 0)
    hipLaunchKernelGGL(moe_block_hist_kernel, dim3((unsigned)nb), dim3(1024), 0, stream, idx, n,
                       E, counts, flags);
  hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(1024), 0, stream, counts, nb, E, offsets,
                     tiles, ntiles, bm2, tiles2, ntiles2, (const int32_t*)flags, status);
  if (nb > 0)
    hipLaunchKernelGGL(moe_scatter_kernel, dim3((unsigned)nb), dim3(1024), 0, stream, idx, n, E,
                       (const int32_t*)counts, (const int32_t*)offsets, perm, inv_perm, topk,
                       a_rows);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* out, int32_t out_bf16, const int32_t* inv_perm,
                              const float* topk_w, const int32_t* topk_idx, int32_t E, int64_t T,
                              int32_t topk, int32_t H, void* Y, int32_t y_bf16,
                              hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (H % (out_bf16 ? 8 : 4)) return hipErrorInvalidValue;
  const int64_t cols = 256 * (out_bf16 ? 8 : 4), nch = (H + cols - 1) / cols;
  if (out_bf16)
    hipLaunchKernelGGL(moe_combine_kernel<true>, dim3((unsigned)(T * nch)), dim3(256), 0, stream,
                       out, inv_perm, topk_w, topk_idx, E, T, topk, H, Y, y_bf16);
  else
    hipLaunchKernelGGL(moe_combine_kernel<false>, dim3((unsigned)(T * nch)), dim3(256), 0, stream,
                       out, inv_perm, topk_w, topk_idx, E, T, topk, H, Y, y_bf16);
  return hipGetLastError();
}

}  // namespace q4
